// fa_prefill_bf16.hip -- tiled exact attention forward, bf16 in/out, fp32
// accumulation, for gfx950 (MI355X).
//
// The method (ai6s.net page, section "FlashAttention changes the dataflow, not
// the algorithm"): Q, K and V are cut into tiles along the sequence axis; each
// workgroup keeps its Q tile on chip, streams K/V tiles through LDS, computes
// the tile of scores, folds it into a running row max and row sum (online
// softmax, rescaling the partial output when the max moves) and multiplies by
// the V tile.  Only O (and LSE) are written back; the score matrix never
// reaches HBM.  The causal mask is applied inside the tile and fully masked
// tiles are never loaded (same page, section "what ops-transformer adds",
// second item).
//
// gfx950 mapping
//  * workgroup = 8 waves = 384 query rows of one (batch, query head); wave w
//    owns rows 48w..48w+47 as three 16-row blocks.  A KV tile is 32 keys.
//    Smaller workgroups serve other launches (see the tile choice at the
//    end): 256 rows (32 per wave, two workgroups per CU) for non-causal head
//    dim 64, 128 rows (16 per wave) for causal head dim 64 up to 4096 rows
//    and for head dim 128 launches with fewer 384-row tiles than CUs.
//    Every K and V operand a wave reads from LDS feeds the MFMAs of its three
//    row blocks, and a copied tile serves 384 rows.  On this chip a wave's
//    MFMAs and another wave's softmax (exponentials above all) barely overlap
//    on a SIMD, so the time per tile is close to the MFMA time plus the
//    softmax's vector time: the softmax is kept to as few vector instructions
//    as possible.
//  * Query tiles are aligned to the end of the sequence (a partial tile holds
//    the first rows, which see the fewest keys) and ordered by kv head, so
//    that with 8 kv heads each XCD holds one kv head of every sequence;
//    causal tiles with the most keys are scheduled first.  In the diagonal
//    band, the first half of the tile's rows stops computing after its last
//    key tile (see the ping-pong schedule below).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: K from LDS is the A operand, Q sits in
//    registers as the B operand for the whole kernel.  The K rows of each
//    16-key block are fed permuted so that lane (row j, group c) ends up
//    holding keys 8c..8c+7 of the tile, which is exactly its slice of the B
//    operand P^T of the following O^T += V^T P^T.  V stays row-major in LDS
//    and its A operand (8 consecutive keys of one head-dim column per lane) is
//    read with ds_read_b64_tr_b16.
//  * Ping-pong schedule.  Waves w and w+4 share a SIMD and belong to
//    different groups.  Per tile a wave runs an MFMA block (P.V of the
//    previous tile, then S of this tile) and a VALU block (softmax of this
//    tile).  Group 1 runs half a tile behind group 0, and workgroup barriers
//    separate the phases, so in every phase one wave of each SIMD issues MFMAs
//    while the other runs its softmax.
//  * Only group 0 moves data: K/V tiles reach LDS by buffer_load ... lds (no
//    staging registers; rows past the end of the slice read 0), kPD tiles
//    ahead through rings of kNS = kPD + 1 stages.
//  * LDS rows are XOR-swizzled per 16-byte chunk so that each read pattern is
//    free of bank conflicts.
//  * Softmax in the base-2 domain: p = 2^(s*c - m), c = scale*log2(e).  The
//    reference max m is set by the row's first visible tile and moves only
//    when a tile's max exceeds it by more than kRescaleSlack; any consistent
//    reference gives the same O = sum p v / sum p.  Each lane compares only
//    the max of its own 8 scores with the row's threshold; the row max is
//    reduced across lanes only when the reference moves.  One fp32 row sum
//    normalises O and gives the LSE.  The rare rescale of O is applied just
//    before the next P.V.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kBC = 32;             // keys per KV tile
constexpr int kThreads = kWaves * 64;
// Query rows per wave, RW: 48 (three 16-row blocks, one workgroup per CU),
// 32 (two blocks, head dim 64 only: at most 128 VGPRs, so two workgroups share
// a CU and short sequences run in one round of resident workgroups) or 16 (one
// block: 128-row workgroups for launches with few query tiles; 59 VGPRs at
// head dim 64, 104 at 128).
template <int D, int RW>
constexpr int waves_per_eu() { return RW == 48 ? 2 : 4; }
// Weights may exceed 1 by up to 2^kRescaleSlack before O is rescaled: fp32
// sums and bf16 weights hold that exactly in range, and the rescale (vector
// work on all accumulators) then happens only for an extreme jump of the max.
constexpr float kRescaleSlack = 64.0f;
#ifndef PREFILL_PD
#define PREFILL_PD 3
#endif
constexpr int kPD = PREFILL_PD;     // tiles of copy look-ahead
constexpr int kNS = kPD + 1;        // LDS stages per tensor

// Key of A-operand row i of 16-key block kb: lane (j, c) of the result then
// holds keys 8c + 4kb + r, i.e. keys 8c..8c+7 over the two blocks.
__device__ __forceinline__ int pi16(int kb, int i) { return 8 * (i >> 2) + 4 * kb + (i & 3); }

// Chunk swizzles (XOR on the 16-byte chunk index within a row of CPR chunks):
//  K (ds_read_b128 of rows pi16(kb, 0..15), one chunk): the swizzle maps those
//  16 rows to 16 different chunks;
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  return ((((row >> 3) & 3) << 2) | (row & 3)) & (CPR - 1);
}
//  V (ds_read_b64_tr_b16: 16 lanes read 32 bytes of each of 4 consecutive
//  rows; the two 16-lane groups served together read rows 8 apart): the 8
//  chunks of one group and the 8 of the other fall on different banks.
template <int CPR>
__device__ __forceinline__ int swz_v(int row) {
  return ((row & 3) << (CPR >= 16 ? 2 : 1)) ^ (((row >> 3) & 1) << 1);
}

// VARLEN: q/o are packed [total_q, Hq, d] and k/v [total_k, Hkv, d], sequence
// b owning rows cu_q[b]..cu_q[b+1]-1 and cu_k[b]..cu_k[b+1]-1; LSE is
// [Hq, total_q].  N_arg / Nk_arg are then upper bounds that size the grid.
template <int D, bool CAUSAL, bool VARLEN, int RW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_eu<D, RW>())))
void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int N_arg, int Nk_arg, int Hq, int Hkv, float c,
    int n_qtiles, int n_work, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int total_q) {
  constexpr int kRows = RW;                 // query rows per wave
  constexpr int kRB = kRows / 16;           // 16-row blocks per wave
  constexpr int kBR = kRows * kWaves;       // query rows per workgroup
  constexpr int DT = D / 32;                // MFMA k-steps of S^T = K Q^T (32 head-dim values each)
  constexpr int DB = D / 16;                // 16-wide head-dim blocks of O^T
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPI = 1024 / (2 * D);       // rows per 1 KB wave copy instruction
  constexpr int TILE_ELEMS = kBC * D;
  constexpr int DMA_PER_WAVE = TILE_ELEMS * 2 / 1024 / (kWaves / 2);   // issued by group 0
  static_assert(DMA_PER_WAVE >= 1, "each issuing wave issues at least one copy per tensor");

  // One LDS variable per stage: the compiler keeps apart the accesses it can
  // attribute to different variables, so a copy in flight into one stage does
  // not make it wait before reads of another (the tile loops below are
  // unrolled so that every stage is named statically).
  static_assert(kNS >= 2 && kNS <= 4, "two to four stages per tensor");
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sK2[kNS > 2 ? TILE_ELEMS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sK3[kNS > 3 ? TILE_ELEMS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sV2[kNS > 2 ? TILE_ELEMS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sV3[kNS > 3 ? TILE_ELEMS : 8];
  // stage st of each ring (a constant st names one variable)
  auto kS = [&](const int st) -> char* {
    return reinterpret_cast<char*>(st == 0 ? sK0 : st == 1 ? sK1 : st == 2 ? sK2 : sK3);
  };
  auto vS = [&](const int st) -> char* {
    return reinterpret_cast<char*>(st == 0 ? sV0 : st == 1 ? sV1 : st == 2 ? sV2 : sV3);
  };

  // Work items in the order (kv head, batch, query tile, query head in the
  // group): a contiguous eighth of the items runs on one XCD, so with 8 kv
  // heads each XCD holds one kv head of every sequence (equal work even when
  // the sequences' lengths differ), and the heads of one group, which read
  // the same K/V, run side by side on one L2.
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  const int n_batch = n_work / (Hq * n_qtiles);
  int rest = logical;
  const int hig = rest % G;
  rest /= G;
  const int qrank = rest % n_qtiles;
  rest /= n_qtiles;
  const int b = rest % n_batch;
  const int g = rest / n_batch;
  const int h = g * G + hig;

  // ---- this sequence's extents and first rows
  int N = N_arg, Nk = Nk_arg;
  int64_t q_row0 = (int64_t)b * N_arg, k_row0 = (int64_t)b * Nk_arg;
  int64_t lse_row0 = ((int64_t)b * Hq + h) * N_arg;    // LSE of query row 0 (rows contiguous)
  if (VARLEN) {
    const int qs = cu_q[b], ks = cu_k[b];
    N = cu_q[b + 1] - qs;
    Nk = cu_k[b + 1] - ks;
    q_row0 = qs;
    k_row0 = ks;
    lse_row0 = (int64_t)h * total_q + qs;
    if (qrank * kBR >= N) return;                       // the tile lies before the sequence
  }
  // Query tiles are aligned to the end of the sequence: tile qrank holds rows
  // N-(qrank+1)*kBR .. N-qrank*kBR-1, so a partial tile (rows below 0 are
  // absent) holds the first rows, which see the fewest keys under the causal
  // mask, and tile 0, the heaviest, is scheduled first.
  const int q0 = N - (qrank + 1) * kBR;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int grp = lane >> 4;                                    // 0..3
  const int wbase = q0 + kRows * wave;                          // first row of the wave
  const int offs = Nk - N;                                      // bottom-right causal offset

  // ---- buffer views: one (batch, head) slice each; reads past the end are 0
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc =
      make_rsrc(q + (q_row0 * Hq + h) * D, (uint32_t)((N - 1) * Hq + 1) * D * 2);
  const uint16_t* k_slice = k + (k_row0 * Hkv + g) * D;
  const uint16_t* v_slice = v + (k_row0 * Hkv + g) * D;
  const uint32_t kv_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * Hkv + 1) * D * 2 : 0u;

  // ---- Q -> registers (B operands of S^T = K Q^T): lane (row j, group c)
  // holds head-dim 32t + 8c..+7 of row 16rb + j; absent rows (below 0) get an
  // offset past any slice (slices are under 2 GiB) and read 0.  Q is read
  // once, so its loads are non-temporal (policy bit NT): it is streamed
  // rather than allocated in the caches that hold the re-read K/V tiles.
  constexpr int kNT = 2;
  bf16x8 qf[kRB][DT];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = wbase + 16 * rb + l16;
    const uint32_t off = row >= 0 ? (uint32_t)row * q_row_bytes + grp * 16 : 0x80000000u;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      qf[rb][t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off + t * 64, 0, kNT));
  }

  // ---- KV tiles this workgroup needs, and where this wave's masked suffix starts
  int n_kv = (Nk + kBC - 1) / kBC;
  if (CAUSAL) {
    const int last_key = N - qrank * kBR - 1 + offs;       // the tile's last row's last key
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kBC + 1);
  }
  // tile j needs no mask for this wave iff j*kBC + kBC-1 < Nk and, when
  // causal, j*kBC + kBC-1 <= max(wbase, 0) + offs (the wave's first present
  // row sees it all; absent rows are never stored, so what they see is moot)
  int n_clean = Nk / kBC;
  if (CAUSAL) {
    const int d0 = max(wbase, 0) + offs - (kBC - 1);
    n_clean = min(n_clean, d0 < 0 ? 0 : d0 / kBC + 1);
  }
  n_clean = min(n_clean, n_kv);

  // ---- copies of K/V tiles into LDS by the 4 waves of group 0: lane l of
  // 1 KB instruction n fills row n*RPI + l/CPR, physical chunk l%CPR.  The
  // per-lane offsets are fixed for the whole kernel: the compiler treats a
  // copy's address register as pending until the copy lands.
  const int dma_wave = wave % (kWaves / 2);
  uint32_t k_voff[DMA_PER_WAVE], v_voff[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int row = (dma_wave * DMA_PER_WAVE + i) * RPI + lane / CPR;
    const int pc = lane % CPR;
    k_voff[i] = (uint32_t)row * kv_row_bytes + (uint32_t)((pc ^ swz_k<CPR>(row)) * 16);
    v_voff[i] = (uint32_t)row * kv_row_bytes + (uint32_t)((pc ^ swz_v<CPR>(row)) * 16);
  }
  // Tile j begins j*kBC rows into the slice.  Every call issues the same
  // number of copies: for a tile that does not exist (j >= n_kv) the view is
  // empty, so the copy writes zeros into a free stage and reads nothing; the
  // waits below count copies.  Each tensor's tiles are copied in order, so a
  // cursor per tensor holds the next tile's index and, where kCursorCopy is
  // set, its first row and the bytes left to the slice end: the descriptor
  // then takes no multiplies and no branches, and the compiler can spread the
  // few scalar instructions of a copy between the MFMAs it sits among.  With
  // d = 128 and with 16-row waves that shortened the copying MFMA block by a
  // measured 1-6%; with 32- and 48-row waves at d = 64 (the block is half as
  // long there) it cost 1-3%, so those keep the address taken from the index.
  constexpr bool kCursorCopy = D == 128 || RW == 16;
  struct Cursor {
    const uint16_t* base;   // the slice
    const uint16_t* ptr;    // first row of tile j (kCursorCopy)
    uint32_t left;          // bytes from ptr to the slice end (kCursorCopy)
    int j;                  // next tile
  };
  Cursor kc{k_slice, k_slice, kv_bytes, 0}, vc{v_slice, v_slice, kv_bytes, 0};
  auto issue = [&](Cursor& cur, const uint32_t* voff, char* stage) __attribute__((always_inline)) {
    const bool real = cur.j < n_kv;
    __amdgpu_buffer_rsrc_t r;
    if constexpr (kCursorCopy) {
      // (the cursor is wave-uniform; said explicitly, so that the descriptor
      // stays in scalar registers)
      const uint64_t pa = reinterpret_cast<uint64_t>(cur.ptr);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
      const uint32_t bytes = __builtin_amdgcn_readfirstlane(real ? cur.left : 0u);
      r = make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), bytes);
      const uint32_t step = (uint32_t)kBC * kv_row_bytes;
      cur.ptr += (int64_t)kBC * Hkv * D;
      cur.left = cur.left > step ? cur.left - step : 0u;
    } else {
      const uint32_t tile_off = real ? (uint32_t)(cur.j * kBC) * kv_row_bytes : 0u;
      r = make_rsrc(cur.base + (real ? (int64_t)cur.j * kBC * Hkv * D : 0), real ? kv_bytes - tile_off : 0u);
    }
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      buffer_load16_to_lds(r, voff[i], 0, (lds_void*)(stage + (dma_wave * DMA_PER_WAVE + i) * 1024));
    ++cur.j;
  };
  constexpr int kCopiesPerBlock = 2 * DMA_PER_WAVE;

  // ---- lane-constant LDS offsets (bytes) for the MFMA operand reads
  // K (A operand of S^T, block kb, step t): row pi16(kb, l16), chunk 4t + grp
  int k_off[2][DT];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = pi16(kb, l16);
#pragma unroll
    for (int t = 0; t < DT; ++t) k_off[kb][t] = row * (2 * D) + (((4 * t + grp) ^ swz_k<CPR>(row)) * 16);
  }
  // V^T (A operand of O^T, transpose read, head-dim block db): lane r of group
  // grp points at key 8grp + r/4 (+4 for the second read) and head-dim
  // 16db + 4(r%4); lane r then receives keys 8grp.. of head-dim 16db + r.
  const int vrow = 8 * grp + (l16 >> 2);
  int v_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 2 * db + ((l16 & 3) >> 1);
    v_off[db] = vrow * (2 * D) + ((chunk ^ swz_v<CPR>(vrow)) * 16) + (l16 & 1) * 8;
  }

  // ---- state
  f32x4 acc_o[kRB][DB];      // O^T: lane (row j, group c) item r = head-dim 16db + 4c + r
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[kRB], nmu[kRB], thr[kRB], l_part[kRB], alpha[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_ref[rb] = -INFINITY;   // reference max of the lane's row (base-2 domain), same in its 4 lanes
    nmu[rb] = 0.0f;          // -m_ref, or 0 while the row has seen no key
    thr[rb] = -INFINITY;     // raw score above which the reference must move
    l_part[rb] = 0.0f;       // fp32 weights of this lane's keys (for LSE)
    alpha[rb] = 1.0f;        // pending rescale of acc_o (applied before the next P.V)
  }
  bool rescale = false;      // wave-uniform: some row of the wave has alpha != 1
  f32x4 s[kRB][2];           // scores of the current tile: item r of block kb = key 8c + 4kb + r
  bf16x8 pf[kRB];            // weights of the current tile, B operands of P.V
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) pf[rb] = bf16x8{};   // the first P.V adds nothing

  // S^T = K Q^T for the K tile at `kst`
  auto stage_s = [&](const char* kst) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, load16(kst + k_off[kb][t]));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rb][t], s[rb][kb], 0, 0, 0);
      }
    }
  };

  // O^T = alpha*O^T + V^T P^T for the V tile at `vst`
  auto stage_pv = [&](const char* vst) {
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc_o[rb][db] *= alpha[rb];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 lo = lds_read_tr16(vst + v_off[db]);
      const u32x2 hi = lds_read_tr16(vst + v_off[db] + 4 * (2 * D));
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc_o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rb], acc_o[rb][db], 0, 0, 0);
    }
  };

  // online softmax of the tile of keys j0..j0+31 -> pf.  `masked`
  // (wave-uniform): some key of the tile is invisible to some row of this wave.
  // Every row that sees any key sees key 0 (the causal limit of a row is a
  // prefix of the keys), so the reference max of every row is set by tile 0
  // and later tiles only compare their max with a fixed threshold: the
  // reference moves (and O, l are rescaled) only when a score exceeds it by
  // more than kRescaleSlack, on a wave-uniform branch that is rarely taken.
  // (c > 0, so s*c > m + slack  <=>  s > (m + slack)/c.)
  auto stage_softmax = [&](const int j0, const bool masked) {
    if (__builtin_expect(masked, 0)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        // last visible key of this lane's row; item r of block kb holds key
        // j0 + 8grp + 4kb + r
        const int lim = CAUSAL ? min(Nk - 1, wbase + 16 * rb + l16 + offs) : Nk - 1;
        const int lim_rel = lim - (j0 + 8 * grp);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[rb][kb][r] = 4 * kb + r <= lim_rel ? s[rb][kb][r] : -INFINITY;
      }
    }
    // (the threshold tests follow the one masking branch in a single block,
    // and each compare is balloted on its own: a ballot of a compare is the
    // compare's lane mask, while a ballot of an OR of compares rebuilds a
    // per-lane bool first)
    float lm[kRB];             // max of this lane's 8 scores of each row block
    uint64_t need = 0;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float m = -INFINITY;     // (a -inf seed keeps the chain to plain v_max3_f32)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, s[rb][i >> 2][i & 3]);
      lm[rb] = m;
      need |= __builtin_amdgcn_ballot_w64(m > thr[rb]);
    }
    // Tile 0 sets every row's reference (thr = -inf there); later tiles move
    // it only when some score exceeds thr, on a wave-uniform branch.  Only
    // then is the row max reduced across the row's 4 lanes.
    rescale = need != 0;
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        // the row's 32 keys sit in lanes j, j+16, j+32, j+48
        const float mx = max_xor32(max_xor16(lm[rb]));
        const bool up = mx > thr[rb];
        const float m_new = up ? mx * c : m_ref[rb];
        // a row's first reference: its sums and O are still 0 (alpha = 0)
        alpha[rb] = up ? (m_ref[rb] == -INFINITY ? 0.0f : fast_exp2(m_ref[rb] - m_new)) : 1.0f;
        m_ref[rb] = m_new;
        nmu[rb] = up ? -m_new : nmu[rb];
        thr[rb] = up ? (m_new + kRescaleSlack) / c : thr[rb];
        l_part[rb] *= alpha[rb];
      }
    }
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float p[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[4 * kb + r] = fast_exp2(fmaf(s[rb][kb][r], c, nmu[rb]));
      l_part[rb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      const u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                       pack_bf16x2(p[6], p[7])};
      pf[rb] = __builtin_bit_cast(bf16x8, w);
    }
  };


  // The MFMA block of tile j: P.V of tile j-1, S of tile j, and (group 0)
  // the copies of K_{j+kPD} and V_{j+kPD-1}.  The read and copy stages are
  // distinct variables, so the compiler does not wait for the copies in
  // flight before the reads (the waits that order copies and reads are the
  // explicit ones below, before the workgroup barriers).
  auto mblock = [&](const char* kread, const char* vread, char* kdst, char* vdst,
                    auto copy_tag) __attribute__((always_inline)) {
    // (tile 0's P.V reads the zero-filled stage of tile -1 with zero weights:
    // no branch, so both products share one scheduling region)
    stage_pv(vread);
    stage_s(kread);
    // LDS operand reads run two MFMA groups ahead of their use
#ifndef PREFILL_READ_AHEAD
#define PREFILL_READ_AHEAD 2
#endif
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PREFILL_READ_AHEAD, 0);   // V^T operands of the first blocks
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // reads two blocks ahead
      __builtin_amdgcn_sched_group_barrier(0x008, kRB, 0);   // MFMAs of block db
    }
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // K operand
      __builtin_amdgcn_sched_group_barrier(0x008, kRB, 0);   // MFMAs of one K operand
    }
    if (decltype(copy_tag)::value) {
      issue(kc, k_voff, kdst);                      // K_{j+kPD}
      issue(vc, v_voff, vdst);                      // V_{j+kPD-1}
    }
  };
  const auto kCopy = std::integral_constant<bool, true>();
  const auto kNoCopy = std::integral_constant<bool, false>();

  // ---- ping-pong schedule.  Group g runs the MFMA block M_j = [P.V of tile
  // j-1, S of tile j] in phase 2j+g and the softmax V_j in phase 2j+1+g;
  // both groups execute 2*n_kv + 2 barriers.  Tile j lives in stage j % kNS
  // of each ring.  Group 0 copies K_0..K_{kPD-1} and V_0..V_{kPD-2} before
  // phase 0 and K_{j+kPD}, V_{j+kPD-1} at the end of M_j; at the end of phase
  // 2j+1 it waits until the copies of K_{j+1} and V_j (issued kPD-1 blocks
  // earlier) have landed, and the barrier publishes them to both groups.  A
  // stage is overwritten only after both groups have finished reading its
  // previous tile (K_{j-1}, V_{j-2}: read by the end of phase 2j-1).
  const int group = wave >= kWaves / 2 ? 1 : 0;
  // Causal: group 0 (the first half of the tile's rows) needs only the first
  // n0 tiles.  It runs its MFMA blocks and softmaxes for those, then, for the
  // last n_kv - n0 tiles, only its P.V of tile n0-1 (in phase 2*n0) and the
  // copies, so that group 1 runs those tiles without a partner on its SIMDs.
  // Every step has two barriers, so both groups execute the same number.
#ifndef PREFILL_EARLY_STOP
#define PREFILL_EARLY_STOP 1
#endif
  int n0 = n_kv;
  if (CAUSAL && PREFILL_EARLY_STOP) {
    const int last_key0 = q0 + kRows * (kWaves / 2) - 1 + offs;   // group 0's last row's last key
    n0 = max(1, min(n_kv, last_key0 < 0 ? 0 : last_key0 / kBC + 1));
  }
  // In a partial tile whose first half is all absent rows (below 0, never
  // stored), group 0 has nothing to compute whatever those rows would see:
  // it stops after one tile, causal or not.
  if (PREFILL_EARLY_STOP && q0 + kRows * (kWaves / 2) <= 0) n0 = min(n0, 1);
  // Rounds of kNS tiles, unrolled so that every stage is named statically.
  // The check after each tile leaves the loop (it never skips ahead to the
  // next round), so at the top of a round, as far as the compiler can tell,
  // the same copies are in flight as at the end of the previous one.
  auto run_group = [&](auto copy_tag, const int n_end) __attribute__((always_inline)) {
    constexpr bool COPY = decltype(copy_tag)::value;
    auto step = [&](const int j, const int st) __attribute__((always_inline)) {   // j % kNS == st
      mblock(kS(st), vS((st + kNS - 1) % kNS), kS((st + kPD) % kNS), vS((st + kPD - 1) % kNS),
             copy_tag);                               // phase 2j+g
      barrier_no_fence();
      stage_softmax(j * kBC, j >= n_clean);           // phase 2j+1+g
      if (COPY) wait_vmem_le<(kPD - 1) * kCopiesPerBlock>();
      barrier_no_fence();
    };
    // one round from tile j0 (< n_end); false once tile n_end-1 is done
    auto round = [&](const int j0) __attribute__((always_inline)) -> bool {
      step(j0, 0);
      if (j0 + 1 >= n_end) return false;
      step(j0 + 1, 1);
      if (j0 + 2 >= n_end) return false;
      if constexpr (kNS > 2) {
        step(j0 + 2, 2);
        if (j0 + 3 >= n_end) return false;
      }
      if constexpr (kNS > 3) {
        step(j0 + 3, 3);
        if (j0 + 4 >= n_end) return false;
      }
      return true;
    };
    for (int j0 = 0; round(j0); j0 += kNS) {
    }
  };
  if (n_kv > 0) {
    // tile -1's V stage (kNS - 1) holds zeros, written by plain stores; the
    // first copy into it is issued in phase 2, after both groups' first P.V
    static_assert(TILE_ELEMS * 2 == kThreads * 16 || TILE_ELEMS * 2 == kThreads * 8, "zero fill layout");
    if (TILE_ELEMS * 2 == kThreads * 16)
      store16(vS(kNS - 1) + tid * 16, u32x4{0u, 0u, 0u, 0u});
    else
      *reinterpret_cast<u32x2*>(vS(kNS - 1) + tid * 8) = u32x2{0u, 0u};
    if (group == 0) {
#pragma unroll
      for (int t = 0; t < kPD; ++t) issue(kc, k_voff, kS(t));
#pragma unroll
      for (int t = 0; t < kPD - 1; ++t) issue(vc, v_voff, vS(t));
    }
    // both groups: the Q registers (and group 0's first copies) have landed.
    // (Waiting in one group only would leave the loads pending, as far as the
    // compiler can tell, where the groups' paths join, and it would then wait
    // for them, and for every copy issued after them, inside the loops.)
    wait_vmem_all();
    barrier_no_fence();
    if (group == 0) {
      run_group(kCopy, n0);
      // group 0's tail (stages named at run time: no LDS reads but one P.V)
      for (int j = n0; j < n_kv; ++j) {
        if (j == n0) stage_pv(vS((j + kNS - 1) % kNS));   // phase 2*n0: P.V of tile n0-1
        issue(kc, k_voff, kS((j + kPD) % kNS));
        issue(vc, v_voff, vS((j + kPD - 1) % kNS));
        barrier_no_fence();
        wait_vmem_le<(kPD - 1) * kCopiesPerBlock>();
        barrier_no_fence();
      }
      wait_vmem_all();                              // no copy may land after the workgroup ends
      if (n0 >= n_kv) stage_pv(vS((n_kv - 1) % kNS));   // phase 2n: M_n (earlier when n0 < n_kv)
      barrier_no_fence();
      barrier_no_fence();                           // phase 2n+1: idle
    } else {
      barrier_no_fence();                           // phase 0: idle
      run_group(kNoCopy, n_kv);
      stage_pv(vS((n_kv - 1) % kNS));               // phase 2n+1: M_n
      barrier_no_fence();
    }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
  // (the last tile's rescale was applied by the final P.V block)
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float lt = l_part[rb] + wave_xor16(l_part[rb]);
    lt += wave_xor32(lt);
    const int row = wbase + 16 * rb + l16;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (row >= 0) {                                  // (every row is below N)
      uint16_t* dst = o + (q_row0 + row) * ((int64_t)Hq * D) + (int64_t)h * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 a = acc_o[rb][db];
        u32x2 w;
        w[0] = pack_bf16x2(a[0] * inv, a[1] * inv);
        w[1] = pack_bf16x2(a[2] * inv, a[3] * inv);
        *reinterpret_cast<u32x2*>(dst + 16 * db) = w;
      }
      if (grp == 0)
        lse[lse_row0 + row] = lt > 0.0f ? (m_ref[rb] + fast_log2(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN, int RW>
hipError_t launch(const PrefillArgs& a) {
  constexpr int kBR = RW * kWaves;
  const int n_qtiles = (a.N + kBR - 1) / kBR;
  const int64_t n_work = (int64_t)a.B * a.Hq * n_qtiles;
  if (n_work == 0) return hipSuccess;
  const int64_t grid = (n_work + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, VARLEN, RW>), dim3((unsigned)grid), dim3(kThreads), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, a.N, a.Nk, a.Hq, a.Hkv, a.scale * kLog2e, n_qtiles, (int)n_work, a.cu_q, a.cu_k,
                     a.total_q);
  return hipGetLastError();
}

// Rows per wave at head dim 64.  32 (two workgroups per CU) wins wherever the
// work is even or short: measured against 48 on one box, B16 H16 N512 44 ->
// 29 us, causal B8 H12 N1024 47 -> 41 us, causal N2048 -23..-26%, full N1024
// and N4096 -33% and -19%.  Causal N4096 ties, and causal B1 H16 N8192 is 19%
// slower with 32: its one round of resident workgroups pairs the long
// diagonal-band tiles on shared CUs, where one workgroup per CU runs them in
// LPT order.  (N is the longest query sequence for varlen.)
//
// 16 rows per wave (128-row workgroups, up to four per CU at head dim 64, two
// at 128) shorten the longest workgroup's chain of key tiles, which bounds a
// causal launch with few query tiles.  Against the sizes above, on one box:
// causal B8 H12 N1024 d64 41.8 -> 37.2 us and B2 H16 N4096 d64 -12%, B1 H16
// N8192 d64 +1% (kept at 48); non-causal B16 H16 N512 d64 +6% (kept at 32).
// At head dim 128 they pay when the 384-row tiling leaves fewer tiles than
// CUs: causal B2 H8 N1000 44.7 -> 23.4 us; B4 H16 N2048 (384 tiles) and B2
// H32 N4096 (704) tie.
template <bool VARLEN>
hipError_t dispatch(const PrefillArgs& a) {
  if (a.d == 64) {
    if (!a.causal) return launch<64, false, VARLEN, 32>(a);
    return a.N > 4096 ? launch<64, true, VARLEN, 48>(a) : launch<64, true, VARLEN, 16>(a);
  }
  if ((int64_t)a.B * a.Hq * ((a.N + 383) / 384) < 256)
    return a.causal ? launch<128, true, VARLEN, 16>(a) : launch<128, false, VARLEN, 16>(a);
  return a.causal ? launch<128, true, VARLEN, 48>(a) : launch<128, false, VARLEN, 48>(a);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a) { return a.cu_q ? dispatch<true>(a) : dispatch<false>(a); }

}  // namespace fa
