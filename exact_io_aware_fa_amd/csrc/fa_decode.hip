// fa_decode.hip -- split-KV decode attention over a packed, variable-length
// KV cache, bf16 in/out, fp32 accumulation, for gfx950.
//
// One new query token per sequence attends to every row of that sequence's
// cache; only the real cache length is read (ai6s.net page, section "what
// ops-transformer adds", third item).  Work is split along the cache: each
// wave reduces pieces of (sequence, kv head) key ranges with the online
// softmax (ai6s.net page, section "FlashAttention changes the dataflow, not
// the algorithm") and writes, per piece, a partial output normalised by its
// own row sum plus the piece's logsumexp.  A second kernel merges the pieces
// of a sequence with weights exp(LSE_s - LSE), LSE = log sum_s exp(LSE_s),
// which is the same rescaling the online softmax applies tile by tile.
//
// gfx950 mapping (split kernel).  The kernel streams the cache once and does
// 8 flops per byte, so it is bound by HBM bandwidth.
//  * Work is split evenly ("stream-K"): the units are the (sequence, key)
//    pairs in that order, K = total keys of them, and key range r of R takes
//    units [floor(r K / R), floor((r+1) K / R)).  Every range holds the same
//    number of cache rows whatever the mix of lengths, so the waves of a
//    launch finish together; R spans a few rounds of resident waves.
//  * workgroup = one key range and HW kv heads (HW = the largest divisor of
//    Hkv up to 8), one wave per kv head; no barriers.  The waves of a
//    workgroup stream the same rows, so together they read whole cache rows
//    (HW heads x d x 2 bytes) rather than each a slice strided by the row;
//    this layout reads measurably faster that way.  Adjacent workgroups hold
//    the other head groups of the range.  A wave writes one partial result
//    per sequence piece of its range.  All G = Hq/Hkv <= 16 query heads of a
//    kv head share every K/V byte, so the cache is read from HBM once.
//  * A piece is streamed in 32-key tiles with two register sets: the loads of
//    tile t+1 are issued before tile t is computed.  The buffer view ends at
//    the piece's last row, so the ragged last tile (and the tile past the end
//    that the pipeline loads) read 0 without touching memory.
//  * K and V rows are loaded whole (4 rows of 256 bytes per instruction at
//    d=128; loads that cover only part of a 128-byte line per row measurably
//    lower the bandwidth of this strided layout) and stored row-major in
//    per-wave LDS tiles, with 16-byte chunks XOR-swizzled by the row.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K slices are read back with
//    ds_read_b128 as the A operand; Q^T (G heads padded to 16 columns) is the
//    B operand.  Lane (head j, group c) then holds keys 4c..4c+3 and
//    16+4c..16+4c+3 of the tile, which are exactly its slice of the B operand
//    P^T of the following O^T += V^T P^T.
//  * V^T, the A operand of that product, is read transposed from the V tile
//    with ds_read_b64_tr_b16.
//
// Paged cache (PAGED): rows live in blocks of a power-of-two size >= 32 that a
// block table maps per sequence; the new token's K/V row may be appended
// first.  A prep kernel writes the appended rows into their blocks and the
// prefix sums of each sequence's 32-key tiles; the split then takes whole
// tiles as its units, so that every tile lies inside one block and its rows
// are found with one table lookup (a scalar load) per tile.  The combine is
// the same, over tile units.
#include <mutex>

#include "fa.h"
#include "fa_common.h"
#include "fa_kernels.h"

// Partial results of fa_decode_noalloc: a static array on every device the
// library runs on, for callers that cannot allocate.  In host code the name
// stands for a host-side shadow, not a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_SCRATCH_BYTES];

namespace fa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];   // per device, set on its first lookup
}  // namespace

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *ptr = scratch_addr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

namespace {

// Cache rows are read once per call and the cache is far larger than the
// caches, so they are loaded non-temporal (policy bit NT): streamed rather
// than allocated.  Measured after a prefill launch, this took the decode
// workload from 0.360 to 0.321 ms: the streamed rows no longer push the
// prefill's freshly written output out of the cache (as write-backs to HBM)
// while the decode runs.
__device__ __forceinline__ u32x4 load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
constexpr int kTile = kDecodeTile;  // keys per tile
constexpr int kGMax = 16;           // query heads per kv head (one MFMA column block)
constexpr float kRescaleSlack = 8.0f;

// Chunk swizzles (XOR on the 16-byte chunk index of a row of CPR chunks):
//  K: the 16 rows of one A-operand read (same logical chunk) hit different banks;
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
//  V: rows 4c..4c+3 of one transposed read land in different banks.
template <int CPR>
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << (CPR >= 16 ? 2 : 1); }

template <int D>
struct KvTile {
  u32x4 k[kTile * D * 2 / 1024];       // K rows, 1 KB per wave load
  u32x4 v[kTile * D * 2 / 1024];       // V rows, 1 KB per wave load
  int nv;                              // rows of the tile that are keys of the piece (may be <= 0)
};

// ---- the even split.  bound(r) = floor(r K / R) is the first unit of range r.
__device__ __forceinline__ int64_t part_bound(int64_t r, int64_t K, int R) { return r * K / R; }

// The range whose units include u (0 <= u < K): the largest r with
// bound(r) <= u, i.e. floor(((u+1) R - 1) / K); it is never an empty range.
__device__ __forceinline__ int range_of(int64_t u, int64_t K, int R) {
  return (int)(((u + 1) * R - 1) / K);
}

// Partial-result slot of a sequence piece: a piece that starts at its
// sequence's first key uses slot R + b; a piece that continues one from the
// previous range (it starts at its range's first unit) uses slot r.  Slot s
// holds rows (s * Hkv + g) * G + j, one per query head.
__device__ __forceinline__ int64_t piece_slot(bool first_key, int r, int R, int b) {
  return first_key ? (int64_t)R + b : (int64_t)r;
}

// The sequence holding unit u: the largest b < B with cu[b] <= u (cu is
// non-decreasing and cu[0] = 0), found 64 entries at a time.
__device__ __forceinline__ int sequence_of(const int32_t* __restrict__ cu, int B, int64_t u) {
  const int lane = threadIdx.x & 63;
  for (int c0 = 0;; c0 += 64) {
    const int i = c0 + lane;
    const bool le = i < B && (int64_t)cu[i] <= u;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    if (cnt < 64 || c0 + 64 >= B) return c0 + cnt - 1;
  }
}

constexpr int kMaxHW = 8;           // kv heads (waves) per split workgroup

// Units: (sequence, key) pairs with cu the packed cache's offsets, or
// (PAGED) (sequence, 32-key tile) pairs with cu the tile prefix sums.
template <int D, bool PAGED>
__global__ __launch_bounds__(64 * kMaxHW, 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cu, float* __restrict__ part_o, float* __restrict__ part_lse, int B, int Hq,
    int Hkv, int R, float c, const int32_t* __restrict__ table, const int32_t* __restrict__ seqlens,
    int max_blocks, int bs_log2, int num_blocks, int append) {
  constexpr int DT = D / 32;                  // MFMA k-steps of S^T (32 head-dim values each)
  constexpr int DB = D / 16;                  // 16-wide head-dim blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;               // rows per wave load
  constexpr int VL = kTile / RPL;             // loads per tile and tensor
  constexpr int kWaveLds = 2 * kTile * D * 2;  // a wave's K and V tiles
  extern __shared__ __attribute__((aligned(1024))) char dyn_lds[];

  const int HW = blockDim.x >> 6;                      // waves = kv heads per workgroup
  const int HG = Hkv / HW;                             // workgroups per key range
  const int r = blockIdx.x / HG;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = (blockIdx.x % HG) * HW + wave;         // this wave's kv head
  const int64_t K = (int64_t)cu[B];
  int64_t u = part_bound(r, K, R);
  const int64_t u_end = part_bound(r + 1, K, R);
  if (u >= u_end) return;                              // no units for this range
  const int G = Hq / Hkv;

  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int grp = lane >> 4;                           // 0..3
  const uint32_t rstride = (uint32_t)Hkv * D * 2;     // bytes between cache rows
  // lane l of load u takes row u*RPL + l/CPR, logical chunk l%CPR
  const int row_l = lane / CPR;
  const uint32_t ld_lane = (uint32_t)row_l * rstride + (lane % CPR) * 16;

  // ---- lane-constant LDS byte offsets
  // tile stores: row u*RPL + row_l, physical chunk (lane%CPR) ^ swz
  // K read (A operand of S^T): row 16kb + l16, logical chunk 4s + grp (the
  // swizzle depends on the row's low 4 bits only, so kb adds 16 rows)
  int k_rd[DT];
#pragma unroll
  for (int st = 0; st < DT; ++st) k_rd[st] = l16 * (2 * D) + (((4 * st + grp) ^ swz_k<CPR>(l16)) * 16);
  // V^T read (ds_read_b64_tr_b16): lane r of group grp points at key row
  // 4grp + r/4 (+16 for the second read) and head-dim 16db + 4(r%4).
  const int trow = 4 * grp + (l16 >> 2);
  int v_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk16 = 2 * db + ((l16 & 3) >> 1);
    v_rd[db] = trow * (2 * D) + ((chunk16 ^ swz_v<CPR>(trow)) * 16) + (l16 & 1) * 8;
  }
  char* const sKb = dyn_lds + wave * kWaveLds;
  char* const sVb = sKb + kWaveLds / 2;

  int b = sequence_of(cu, B, u);
  while (u < u_end) {
    const int start = cu[b];
    const int L = cu[b + 1] - start;
    if (u >= (int64_t)start + L) {                     // past sequence b (or it is empty)
      ++b;
      continue;
    }
    // ---- the piece: units [k0, k0 + n) of (sequence b, kv head g), i.e.
    // keys [k0, k0 + n), or (PAGED) the keys of tiles [k0, k0 + n), of which
    // the first nkeys exist
    const int k0 = (int)(u - start);
    const int64_t piece_end = min(u_end, (int64_t)start + L);
    const int n = (int)(piece_end - u);
    const int nkeys = PAGED ? min(max(seqlens[b], 0) + append - k0 * kTile, n * kTile) : n;

    // buffer views over the piece's rows of kv head g; rows >= n read 0
    const int64_t row0 = PAGED ? 0 : ((int64_t)(start + k0) * Hkv + g) * D;
    const uint32_t nbytes = PAGED ? 0u : (uint32_t)((n - 1) * Hkv + 1) * D * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(kc + row0, nbytes);
    const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(vc + row0, nbytes);
    auto load_tile = [&](KvTile<D>& t, const int tile) {
      if constexpr (!PAGED) {
        t.nv = n - tile * kTile;
        const uint32_t base = (uint32_t)tile * kTile * rstride + ld_lane;
#pragma unroll
        for (int i = 0; i < VL; ++i) t.k[i] = load16_stream(k_rsrc, base + i * RPL * rstride);
#pragma unroll
        for (int i = 0; i < VL; ++i) t.v[i] = load16_stream(v_rsrc, base + i * RPL * rstride);
      } else {
        // the tile's rows: one block, found by one (scalar) table lookup; a
        // tile past the piece, past the table's row or with an entry outside
        // [0, num_blocks) is empty (its view has no bytes, so it reads 0)
        const int key0 = (k0 + tile) * kTile;
        const int blk = key0 >> bs_log2;
        int nv = min(nkeys - tile * kTile, kTile);
        const bool in_table = nv > 0 && blk < max_blocks;
        const int pb = table[in_table ? (int64_t)b * max_blocks + blk : 0];
        const bool ok = in_table && pb >= 0 && pb < num_blocks;
        nv = ok ? nv : 0;
        t.nv = nv;
        const int64_t prow = ok ? ((int64_t)pb << bs_log2) + (key0 & ((1 << bs_log2) - 1)) : 0;
        const uint32_t tbytes = nv > 0 ? (uint32_t)((nv - 1) * Hkv + 1) * D * 2 : 0u;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(kc + (prow * Hkv + g) * D, tbytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vc + (prow * Hkv + g) * D, tbytes);
#pragma unroll
        for (int i = 0; i < VL; ++i) t.k[i] = load16_stream(kr, ld_lane + i * RPL * rstride);
#pragma unroll
        for (int i = 0; i < VL; ++i) t.v[i] = load16_stream(vr, ld_lane + i * RPL * rstride);
      }
      // issue these loads before any of the following compute (the scheduler
      // would otherwise hoist the previous tile's first wait above them)
      __builtin_amdgcn_sched_barrier(0);
    };

    // Q^T as B operand: column j = query head g*G + j (zero for j >= G)
    bf16x8 qf[DT];
    {
      const bool valid = l16 < G;
      const uint16_t* src = q + ((int64_t)b * Hq + g * G + (valid ? l16 : 0)) * D + grp * 8;
#pragma unroll
      for (int st = 0; st < DT; ++st) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (valid) x = load16(src + st * 32);
        qf[st] = __builtin_bit_cast(bf16x8, x);
      }
    }

    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;   // reference max of head l16 (base-2 domain), same in its 4 lanes
    float l_part = 0.0f;       // fp32 weights of this lane's keys (for LSE)
    float l_rnd = 0.0f;        // bf16-rounded weights of this lane's keys (for O)

    auto compute_tile = [&](const KvTile<D>& t, const int tile) {
      // K and V rows -> LDS (the previous tile's reads were issued before;
      // LDS accesses of one wave complete in order)
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int row = i * RPL + row_l;
        store16(sKb + row * (2 * D) + (((lane % CPR) ^ swz_k<CPR>(row)) * 16), t.k[i]);
      }
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int row = i * RPL + row_l;
        store16(sVb + row * (2 * D) + (((lane % CPR) ^ swz_v<CPR>(row)) * 16), t.v[i]);
      }
      // S^T: lane (head l16, group grp) item r of block kb = key 16kb + 4grp + r
      f32x4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < DT; ++st) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, load16(sKb + kb * 16 * (2 * D) + k_rd[st]));
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[st], s[kb], 0, 0, 0);
        }
      }
      // mask keys past the piece's end, then the online softmax of head l16
      const int thr = t.nv - 1 - 4 * grp;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][r] = 16 * kb + r <= thr ? s[kb][r] : -INFINITY;
          mx = fmaxf(mx, s[kb][r]);
        }
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      const float mt = mx * c;
      const bool need = mt > m_ref + kRescaleSlack;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
        const float m_new = need ? mt : m_ref;
        const float alpha = need ? fast_exp2(m_ref - m_new) : 1.0f;   // 0 when m_ref was -inf
        m_ref = m_new;
        l_part *= alpha;
        l_rnd *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
      float p[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[4 * kb + r] = fast_exp2(fmaf(s[kb][r], c, -mu));
          l_part += p[4 * kb + r];
        }
      const bf16x8 pf = pack_bf16x8_sum(p, &l_rnd);
      // O^T += V^T P^T: items 0..3 = keys 4grp.., items 4..7 = keys 16+4grp..
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr16(sVb + v_rd[db]);
        const u32x2 hi = lds_read_tr16(sVb + v_rd[db] + 16 * (2 * D));
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, acc[db], 0, 0, 0);
      }
    };

    // two-stage register pipeline over the piece's tiles.  Tiles past the end
    // read 0 (no memory traffic) and are fully masked, so they add nothing;
    // the loads and computes are unconditional so that the only waits are for
    // the tile about to be used (a load issued on one path only would make the
    // compiler wait for every load at the join).
    const int ntiles = PAGED ? n : (n + kTile - 1) / kTile;
    KvTile<D> ta, tb;
    load_tile(ta, 0);
    for (int t = 0; t < ntiles; t += 2) {
      load_tile(tb, t + 1);
      compute_tile(ta, t);
      load_tile(ta, t + 2);
      compute_tile(tb, t + 1);
    }

    // partial result of the piece: O_s = O / l_rnd, LSE_s = (m + log2 l) ln 2
    l_part += __shfl_xor(l_part, 16, 64);
    l_part += __shfl_xor(l_part, 32, 64);
    l_rnd += __shfl_xor(l_rnd, 16, 64);
    l_rnd += __shfl_xor(l_rnd, 32, 64);
    if (l16 < G) {
      const int64_t slot = (piece_slot(k0 == 0, r, R, b) * Hkv + g) * G + l16;
      // (a piece without keys -- possible only in a paged cache whose table
      // points outside it -- writes O = 0 and LSE = -inf, weight 0 in the merge)
      const float inv = l_rnd > 0.0f ? 1.0f / l_rnd : 0.0f;
      float* dst = part_o + slot * D + 4 * grp;
      // lane (head l16, group grp) item r of block db holds head-dim 16db + 4grp + r
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = acc[db] * inv;
      if (grp == 0) part_lse[slot] = (m_ref + fast_log2(l_part)) * kLn2;
    }
    u = piece_end;
  }
}

// One wave per (sequence, query head), kCombineWaves per workgroup: merges the
// pieces of its sequence -- the first piece, in slot R + b, and one
// continuation per non-empty key range that starts inside the sequence, in
// that range's slot -- as LSE = M + ln sum_s exp(LSE_s - M), O = sum_s
// exp(LSE_s - LSE) O_s with M the largest LSE_s.  Lane i takes piece i of
// each 64-piece chunk: it reads the piece's LSE (one round of loads for the
// max, one for the weights), and then every lane folds all pieces of the
// chunk for its D/64 head-dim values, the weight and slot of piece u read
// from lane u.
constexpr int kCombineWaves = 4;
constexpr int kCombineThreads = 64 * kCombineWaves;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, const int32_t* __restrict__ cu,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int R) {
  constexpr int PER = D / 64;                          // head-dim values per lane
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (bh >= (int64_t)B * Hq) return;
  const int b = (int)(bh / Hq), h = (int)(bh % Hq);
  const int G = Hq / Hkv;
  const int g = h / G, j = h % G;
  const int start = cu[b];
  const int L = cu[b + 1] - start;
  if (L == 0 || R == 0) {                              // no keys: O = 0, LSE = -inf
#pragma unroll
    for (int p = 0; p < PER; ++p) o[bh * D + lane + 64 * p] = 0;
    if (lane == 0) lse[bh] = -INFINITY;
    return;
  }
  const int64_t K = (int64_t)cu[B];
  const int lo = range_of(start, K, R), hi = range_of((int64_t)start + L - 1, K, R);
  const int npieces = 1 + (hi - lo);
  // a range has no units only when there are fewer units than ranges
  const bool may_be_empty = K < R;
  auto slot_of = [&](const int i) { return (piece_slot(i == 0, lo + i, R, b) * Hkv + g) * G + j; };
  auto present = [&](const int i) {
    return i == 0 || !may_be_empty || part_bound(lo + i, K, R) < part_bound(lo + i + 1, K, R);
  };
  // the largest piece LSE (lane i holds piece i of each 64-piece chunk)
  float M = -INFINITY;
  for (int c0 = 0; c0 < npieces; c0 += 64) {
    const int i = c0 + lane;
    if (i < npieces && present(i)) M = fmaxf(M, part_lse[slot_of(i)]);
  }
  M = max_xor32(max_xor16(M));
  M = fmaxf(M, __shfl_xor(M, 8, 64));
  M = fmaxf(M, __shfl_xor(M, 4, 64));
  M = fmaxf(M, __shfl_xor(M, 2, 64));
  M = fmaxf(M, __shfl_xor(M, 1, 64));
  // each lane weighs its piece; then every lane folds the chunk's pieces for
  // its head-dim values, reading each piece's weight and slot from its lane
  // An absent piece (a lane past the last piece, or an empty range) takes the
  // slot of piece 0 with weight 0: that slot is always written by this call,
  // so the product with the zero weight reads a finite value (a slot no piece
  // wrote may hold anything, Inf or NaN included, and 0 * Inf is NaN).
  float acc[PER] = {}, wlane_sum = 0.0f;
  const int slot0 = (int)slot_of(0);
  for (int c0 = 0; c0 < npieces; c0 += 64) {
    const int i = c0 + lane;
    const bool ok = i < npieces && present(i);
    const int sl = ok ? (int)slot_of(i) : slot0;
    const float ls = ok ? part_lse[sl] : -INFINITY;
    const float w = ls == -INFINITY ? 0.0f : fast_exp2((ls - M) * kLog2e);
    wlane_sum += w;
    const int n = min(64, npieces - c0);
    constexpr int kU = 8;                              // pieces whose loads are in flight together
    for (int u0 = 0; u0 < n; u0 += kU) {
      float wv[kU], ov[kU][PER];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int src = min(u0 + u, n - 1);
        const int su = __builtin_amdgcn_readlane(sl, src);
        wv[u] = u0 + u < n ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), src))
                           : 0.0f;
#pragma unroll
        for (int p = 0; p < PER; ++p) ov[u][p] = part_o[(int64_t)su * D + lane + 64 * p];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] = fmaf(wv[u], ov[u][p], acc[p]);
    }
  }
  float wsum = wlane_sum;
  wsum += __shfl_xor(wsum, 32, 64);
  wsum += __shfl_xor(wsum, 16, 64);
  wsum += __shfl_xor(wsum, 8, 64);
  wsum += __shfl_xor(wsum, 4, 64);
  wsum += __shfl_xor(wsum, 2, 64);
  wsum += __shfl_xor(wsum, 1, 64);
  // (no piece with a key: O = 0, LSE = -inf, as for an empty sequence)
#pragma unroll
  for (int p = 0; p < PER; ++p)
    o[bh * D + lane + 64 * p] = __builtin_bit_cast(uint16_t, (__bf16)(wsum > 0.0f ? acc[p] / wsum : 0.0f));
  if (lane == 0) lse[bh] = wsum > 0.0f ? M + fast_log2(wsum) * kLn2 : -INFINITY;
}

// Paged-cache preparation.  Workgroup 0 writes cu_tiles[b] = the tiles of
// sequences 0..b-1, a sequence of L rows (L + append after the append) having
// ceil(L / 32); workgroup 1 + b appends sequence b's new K and V rows at its
// logical row seqlens[b] (skipped when that row lies past the table's row or
// in a block outside [0, num_blocks)).
constexpr int kPrepThreads = 256;

__device__ __forceinline__ int tiles_of(int32_t L, int append) {
  return (int)(((int64_t)max(L, 0) + append + kTile - 1) / kTile);
}

template <int D>
__global__ __launch_bounds__(kPrepThreads) void paged_prep_kernel(
    const int32_t* __restrict__ seqlens, int32_t* __restrict__ cu_tiles, const int32_t* __restrict__ table,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, int B, int Hkv, int max_blocks, int bs_log2, int num_blocks, int append) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    // thread t sums a contiguous run of sequences; an exclusive scan of the
    // runs' sums (in LDS) gives each run its starting offset
    __shared__ int32_t part[kPrepThreads];
    const int per = (B + kPrepThreads - 1) / kPrepThreads;
    const int lo = min(B, tid * per), hi = min(B, lo + per);
    int32_t sum = 0;
    for (int i = lo; i < hi; ++i) sum += tiles_of(seqlens[i], append);
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kPrepThreads; off <<= 1) {
      const int32_t x = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += x;
      __syncthreads();
    }
    int32_t run = tid > 0 ? part[tid - 1] : 0;
    for (int i = lo; i < hi; ++i) {
      run += tiles_of(seqlens[i], append);
      cu_tiles[i + 1] = run;
    }
    if (tid == 0) cu_tiles[0] = 0;
    return;
  }
  const int b = blockIdx.x - 1;
  const int L = seqlens[b];
  if (L < 0) return;
  const int blk = L >> bs_log2;
  if (blk >= max_blocks) return;
  const int pb = table[(int64_t)b * max_blocks + blk];
  if (pb < 0 || pb >= num_blocks) return;
  const int64_t row = ((int64_t)pb << bs_log2) + (L & ((1 << bs_log2) - 1));
  const int chunks = Hkv * D / 8;                      // 16-byte chunks of one row
  for (int i = tid; i < chunks; i += kPrepThreads) {
    store16(kc + row * Hkv * D + i * 8, load16(k_new + (int64_t)b * Hkv * D + i * 8));
    store16(vc + row * Hkv * D + i * 8, load16(v_new + (int64_t)b * Hkv * D + i * 8));
  }
}

// Waves (kv heads) per split workgroup: the largest divisor of Hkv up to kMaxHW.
int heads_per_group(int Hkv) {
  for (int hw = kMaxHW; hw > 1; --hw)
    if (Hkv % hw == 0) return hw;
  return 1;
}

template <int D, bool PAGED>
hipError_t launch(const DecodeArgs& a) {
  const int32_t* cu = a.cu;
  const int append = a.k_new ? 1 : 0;
  if (PAGED) {
    const int64_t grid = 1 + (append ? (int64_t)a.B : 0);
    hipLaunchKernelGGL((paged_prep_kernel<D>), dim3((unsigned)grid), dim3(kPrepThreads), 0, a.stream, a.seqlens,
                       a.cu_tiles, a.block_table, (const uint16_t*)a.k_new, (const uint16_t*)a.v_new,
                       (uint16_t*)const_cast<void*>(a.k_cache), (uint16_t*)const_cast<void*>(a.v_cache), a.B,
                       a.Hkv, a.max_blocks, a.bs_log2, a.num_blocks, append);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    cu = a.cu_tiles;
  }
  if (a.ranges > 0) {
    const int hw = heads_per_group(a.Hkv);
    const int64_t grid = (int64_t)a.ranges * (a.Hkv / hw);
    const size_t lds = (size_t)hw * 2 * kTile * D * 2;
    hipLaunchKernelGGL((decode_split_kernel<D, PAGED>), dim3((unsigned)grid), dim3(64 * hw), lds, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, cu,
                       a.part_o, a.part_lse, a.B, a.Hq, a.Hkv, a.ranges, a.scale * kLog2e, a.block_table,
                       a.seqlens, a.max_blocks, a.bs_log2, a.num_blocks, append);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t combine_blocks = ((int64_t)a.B * a.Hq + kCombineWaves - 1) / kCombineWaves;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)combine_blocks), dim3(kCombineThreads), 0,
                     a.stream, a.part_o, a.part_lse, cu, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.ranges);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a) {
  return a.d == 64 ? launch<64, false>(a) : launch<128, false>(a);
}

hipError_t launch_decode_paged_bf16(const DecodeArgs& a) {
  return a.d == 64 ? launch<64, true>(a) : launch<128, true>(a);
}

int decode_max_group() { return kGMax; }

}  // namespace fa
