// fa_bwd_bf16.hip -- backward of exact attention (dQ, dK, dV), bf16 in and
// out, fp32 accumulation, for gfx950.
//
// The pages give no backward algorithm; the kernels compute the chain rule of
// the forward's definition (S = scale Q K^T, P = softmax(S) over the visible
// keys, O = P V), recomputing P from the forward's LSE rather than storing it:
//   P_ij = exp(scale q_i.k_j - LSE_i),  dV = P^T dO,  dP = dO V^T,
//   dS = P o (dP - D),  D_i = sum_j P_ij dP_ij = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q,
// with the forward's mask (bottom-right causal) and the query heads of a kv
// head summed into its dK and dV.
//
// Three kernels, no atomics (each output row has one owner):
//  * bwd_pre_kernel: per 32-row query tile of each (batch, head), the rows'
//    base-2 LSE (+inf for a row without keys or past N, so that its P is 0)
//    and D, into the workspace;
//  * bwd_dq_kernel: one workgroup per (query tile, query head, batch),
//    streaming K/V tiles: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T;
//  * bwd_dkdv_kernel: one workgroup per (key tile, kv head, batch), streaming
//    the Q and dO tiles of the group's query heads; pairs of waves share 32
//    keys, one computing S = Q K^T, P and dV^T += dO^T P, the other, a tile
//    behind, dP = dO V^T, dS and dK^T += Q^T dS.
// Both use the forward's MFMA layout: with the streamed operand's rows fed in
// the permuted order pi16, a lane of a 16x16x32 result holds 8 consecutive
// entries of one row of P or dS, which is exactly its slice of the next
// product's B operand, so P and dS stay in registers (bwd_dkdv hands P from
// one wave of a pair to the other through LDS in that same lane order).  The
// second operand of each product is either held in registers for the whole
// loop (Q and dO in bwd_dq, K or V in bwd_dkdv) or read from the streamed LDS
// tile: by rows (ds_read_b128) as an A operand, or transposed
// (ds_read_b64_tr_b16) as the A operand of a transposed product.  S and dP
// are computed in both kernels: 7 matrix products in all, against 5 with
// atomics on dQ.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kT = 32;          // rows of a streamed tile (keys in bwd_dq, queries in bwd_dkdv)
constexpr int kThr = 256;       // threads of the staging copies and the pre kernel

__device__ __forceinline__ int pi16(int kb, int i) { return 8 * (i >> 2) + 4 * kb + (i & 3); }

// Rows that exactly one workgroup reads (the dQ kernel's Q and dO rows, the
// dK/dV kernel's K and V rows) are loaded non-temporal (policy bit NT):
// streamed rather than allocated in L2, where they would evict the tiles
// that the other workgroups of the head re-read.
__device__ __forceinline__ u32x4 load16_once(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

// XOR of the 16-byte chunk index by the row (bits b4..b0).  A tile is read
// both ways: by rows (ds_read_b128 of one logical chunk of the 16 rows
// pi16(kb, 0..15)) and transposed (ds_read_b64_tr_b16: chunks 2db, 2db+1 of
// rows 8c + 0..3 (+4)).  Measured with SQ_LDS_BANK_CONFLICT on this chip:
// the row reads are conflict-free when bits 0-2 of the swizzle are a
// bijection of (b0, b1, b3) over the rows of 8 consecutive lanes, and the
// transposed reads when bits 1-3 are, over the rows of 32 lanes (bit 0 then
// tells chunk 2db from 2db+1).  (b0, b1, b3, b0) in bits 0-3 satisfies both
// (0 conflicts in both backward kernels, against 20-28% of the LDS cycles
// with the forward's K swizzle).  At d=64 (8 chunks per row, two rows per 64
// banks) the forward's K swizzle already satisfies both.  The swizzle does
// not depend on b2, so rows r and r+4 of a transposed read share it.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  const int b0 = row & 1, b1 = (row >> 1) & 1, b3 = (row >> 3) & 1, b4 = (row >> 4) & 1;
  if (CPR < 16) return (b0 | (b1 << 1) | (b3 << 2) | (b4 << 3)) & (CPR - 1);
  return b0 | (b1 << 1) | (b3 << 2) | (b0 << 3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---- The workspace ld [B*Hq][ntq][2*kT], ntq = ceil(N / kT): for query tile
// t of (batch, head), lse2 of its rows (LSE log2(e); +inf for LSE = -inf and
// for rows past N) then their D_i = dO_i . O_i (0 past N).  D/8 lanes per
// row; the rows are taken in the BSHD order of O and dO (contiguous reads),
// then the B*Hq*(ntq*kT - N) padding rows, one lane each.
template <int D>
__global__ __launch_bounds__(kThr) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ ld, int B,
                                                       int N, int Hq, int ntq) {
  constexpr int LPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * kThr + threadIdx.x;
  const int64_t row = gid / LPR;
  const int part = (int)(gid % LPR);
  const int64_t nrows = (int64_t)B * N * Hq;
  const int pad = ntq * kT - N;
  float acc = 0.0f;
  if (row < nrows) {
    const u32x4 a = load16(o + row * D + part * 8);
    const u32x4 g = load16(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += bf16_lo(a[w]) * bf16_lo(g[w]) + bf16_hi(a[w]) * bf16_hi(g[w]);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (part != 0) return;
  int64_t bh;
  int i;
  float l2;
  if (row < nrows) {
    const int h = (int)(row % Hq);
    const int64_t bi = row / Hq;
    i = (int)(bi % N);
    bh = (bi / N) * Hq + h;
    const float l = lse[bh * N + i];
    l2 = l == -INFINITY ? INFINITY : l * kLog2e;
  } else {
    const int64_t r = row - nrows;               // padding row r of B*Hq*pad
    if (pad == 0 || r >= (int64_t)B * Hq * pad) return;
    bh = r / pad;
    i = N + (int)(r % pad);
    l2 = INFINITY;
  }
  float* blk = ld + (bh * ntq + i / kT) * (2 * kT);
  blk[i % kT] = l2;
  blk[kT + i % kT] = acc;
}

// Copies of one 32-row tile of a [rows, H, D] tensor slice into LDS by THR
// threads: thread t moves 16-byte chunks t, t + THR, ... (row = chunk / CPR).
template <int D, int THR = kThr>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int CH = kT * CPR / THR;       // chunks per thread
  static_assert(CH >= 1 && kT * CPR % THR == 0, "tile chunks spread evenly over the threads");
  u32x4 r[CH];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int row0, uint32_t row_bytes, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int id = tid + THR * i;
      const int row = id / CPR, col = id % CPR;
      r[i] = buffer_load16(rsrc, (uint32_t)(row0 + row) * row_bytes + col * 16);
    }
  }
  __device__ __forceinline__ void store(char* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int id = tid + THR * i;
      const int row = id / CPR, col = id % CPR;
      store16(tile + row * (2 * D) + ((col ^ swz<CPR>(row)) * 16), r[i]);
    }
  }
};

// ---- dQ.  Workgroup: WQ waves x (16 RB) query rows; tile rows aligned to the
// end of the sequence as in the forward (a partial tile holds the first rows).
#ifndef BWD_OCCQ
#define BWD_OCCQ 2
#endif

template <int D, bool CAUSAL, int WQ, int RB>
__global__ __launch_bounds__(64 * WQ, BWD_OCCQ) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ ld, uint16_t* __restrict__ dq, int N, int Nk,
    int Hq, int Hkv, float c, float scale, int ntq, int n_qtiles, int n_work) {
  static_assert(WQ * 64 >= kThr, "staging copies use the first 256 threads");
  constexpr int DT = D / 32, DB = D / 16, CPR = D / 8;
  constexpr int ROWS_W = 16 * RB, ROWS_G = ROWS_W * WQ;
  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][kT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][kT * D];

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  const int n_batch = n_work / (Hq * n_qtiles);
  int rest = logical;
  const int hig = rest % G;
  rest /= G;
  const int qrank = rest % n_qtiles;                 // 0: the last rows (heaviest causal tile)
  rest /= n_qtiles;
  const int b = rest % n_batch;
  const int g = rest / n_batch;
  const int h = g * G + hig;
  const int q0 = N - (qrank + 1) * ROWS_G;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int wbase = q0 + ROWS_W * wave;
  const int offs = Nk - N;

  // Q and dO rows -> B operands (lane (row j, group c): head-dim 32t + 8c..);
  // rows below 0 read 0 (offset past any slice, which is under 2 GiB)
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const int64_t qs = ((int64_t)b * N * Hq + h) * D;
  const uint32_t q_bytes = (uint32_t)((N - 1) * Hq + 1) * D * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(q + qs, q_bytes);
  const __amdgpu_buffer_rsrc_t d_rsrc = make_rsrc(dout + qs, q_bytes);
  bf16x8 qf[RB][DT], df[RB][DT];
  float l2[RB], ds[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wbase + 16 * rb + l16;
    const uint32_t off = row >= 0 ? (uint32_t)row * q_row_bytes + grp * 16 : 0x80000000u;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      qf[rb][t] = __builtin_bit_cast(bf16x8, load16_once(q_rsrc, off + t * 64));
      df[rb][t] = __builtin_bit_cast(bf16x8, load16_once(d_rsrc, off + t * 64));
    }
    const bool in = row >= 0 && row < N;
    const int ri = in ? row : 0;
    const int64_t li = ((int64_t)(b * Hq + h) * ntq + ri / kT) * (2 * kT) + ri % kT;
    l2[rb] = in ? ld[li] : INFINITY;                  // P = 0 for absent rows
    ds[rb] = in ? ld[li + kT] : 0.0f;
  }

  // key tiles this workgroup needs; tiles below n_clean need no mask for this wave
  int n_kv = (Nk + kT - 1) / kT;
  if (CAUSAL) {
    const int last_key = N - qrank * ROWS_G - 1 + offs;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kT + 1);
  }
  int n_clean = Nk / kT;
  if (CAUSAL) {
    const int d0 = max(wbase, 0) + offs - (kT - 1);
    n_clean = min(n_clean, d0 < 0 ? 0 : d0 / kT + 1);
  }

  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const int64_t ks = ((int64_t)b * Nk * Hkv + g) * D;
  const uint32_t kv_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * Hkv + 1) * D * 2 : 0u;
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(k + ks, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(v + ks, kv_bytes);

  // LDS offsets: row reads (A operand rows pi16(kb, l16), chunk 4t + grp) and
  // transposed reads (lane r of group c: row 8c + r/4 (+4), head-dim 16db + 4(r%4))
  int r_off[2][DT];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = pi16(kb, l16);
#pragma unroll
    for (int t = 0; t < DT; ++t) r_off[kb][t] = row * (2 * D) + (((4 * t + grp) ^ swz<CPR>(row)) * 16);
  }
  const int trow = 8 * grp + (l16 >> 2);
  int t_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 2 * db + ((l16 & 3) >> 1);
    t_off[db] = trow * (2 * D) + ((chunk ^ swz<CPR>(trow)) * 16) + (l16 & 1) * 8;
  }

  f32x4 acc[RB][DB];          // dQ^T: lane (row j, group c) item r = head-dim 16db + 4c + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  TileCopy<D> ck, cv;
  const bool copier = tid < kThr;
  if (n_kv > 0) {
    if (copier) {
      ck.load(k_rsrc, 0, kv_row_bytes, tid);
      cv.load(v_rsrc, 0, kv_row_bytes, tid);
      ck.store(reinterpret_cast<char*>(sK[0]), tid);
      cv.store(reinterpret_cast<char*>(sV[0]), tid);
    }
    __syncthreads();
  }
  for (int j = 0; j < n_kv; ++j) {
    const bool more = j + 1 < n_kv;
    if (more && copier) {
      ck.load(k_rsrc, (j + 1) * kT, kv_row_bytes, tid);
      cv.load(v_rsrc, (j + 1) * kT, kv_row_bytes, tid);
    }
    const char* kt = reinterpret_cast<const char*>(sK[j & 1]);
    const char* vt = reinterpret_cast<const char*>(sV[j & 1]);
    // S^T = K Q^T and dP^T = V dO^T: lane (row j, group c) item r of block kb
    // = key 8c + 4kb + r of the tile
    f32x4 s[RB][2], dp[RB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][kb] = dp[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, load16(kt + r_off[kb][t]));
        const bf16x8 va = __builtin_bit_cast(bf16x8, load16(vt + r_off[kb][t]));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[rb][t], s[rb][kb], 0, 0, 0);
          dp[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, df[rb][t], dp[rb][kb], 0, 0, 0);
        }
      }
    }
    // P = 2^(s c - lse2) (0 where masked), dS = P (dP - D) -> bf16 B operands
    const bool masked = j >= n_clean;
    bf16x8 dsf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float e[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(s[rb][kb][r], c, -l2[rb]));
          e[4 * kb + r] = p * (dp[rb][kb][r] - ds[rb]);
        }
      if (masked) {
        const int row = wbase + 16 * rb + l16;
        const int lim = CAUSAL ? min(Nk - 1, row + offs) : Nk - 1;
        const int rel = lim - (j * kT + 8 * grp);
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = i <= rel ? e[i] : 0.0f;
      }
      const u32x4 w = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                       pack_bf16x2(e[6], e[7])};
      dsf[rb] = __builtin_bit_cast(bf16x8, w);
    }
    // dQ^T += K^T dS^T (K^T: transposed reads of the K tile)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 lo = lds_read_tr16(kt + t_off[db]);
      const u32x2 hi = lds_read_tr16(kt + t_off[db] + 4 * (2 * D));
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dsf[rb], acc[rb][db], 0, 0, 0);
    }
    if constexpr (kDebugSync) __syncthreads();
    if (more && copier) {
      // the other buffers were last read in iteration j-1, before its barrier
      ck.store(reinterpret_cast<char*>(sK[(j + 1) & 1]), tid);
      cv.store(reinterpret_cast<char*>(sV[(j + 1) & 1]), tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wbase + 16 * rb + l16;
    if (row >= 0) {                                  // (every row is below N)
      uint16_t* dst = dq + (((int64_t)b * N + row) * Hq + h) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 a = acc[rb][db];
        u32x2 w;
        w[0] = pack_bf16x2(a[0] * scale, a[1] * scale);
        w[1] = pack_bf16x2(a[2] * scale, a[3] * scale);
        *reinterpret_cast<u32x2*>(dst + 16 * db) = w;
      }
    }
  }
}

// ---- dK and dV.  Workgroup: 8 waves over 128 keys of one kv head, as 4 pairs
// of waves on 32 keys each; the two waves of a pair (waves p and p + 4) run
// on one SIMD.  It streams the 32-row Q and dO tiles of every query head of
// the group, from the last query tile down to the first that sees one of its
// keys, heads innermost: the workgroups of one kv head start on the same tile
// and move through the tiles together, so they share each one in L2.
// Per tile, wave A of a pair computes S = Q K^T, P (masked) and
// dV^T += dO^T P, and leaves P (fp32) in LDS; wave B, half a tile behind,
// computes dP = dO V^T, dS = P o (dP - D) and dK^T += Q^T dS.  Both do the
// same number of MFMAs per tile; a tile has two phases (two workgroup
// barriers), and in each one wave of every SIMD runs its MFMAs while the
// other runs its exponentials or dS arithmetic.  The tiles, with lse2 and D
// of their rows, reach LDS by buffer_load ... lds through a ring of 4
// stages, two tiles ahead.
constexpr int kDkWaves = 8;                         // 4 pairs
constexpr int kDkRB = 2;                            // 16-key blocks per pair
constexpr int kDkKeys = 16 * kDkRB * kDkWaves / 2;  // keys per workgroup
constexpr int kDkNS = 4;                            // stages of the Q/dO ring (copies run 2 tiles ahead)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kDkWaves, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ ld, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int N, int Nk, int Hq, int Hkv, float c, float scale, int ntq, int n_ktiles,
    int n_work) {
  constexpr int DT = D / 32, DB = D / 16, CPR = D / 8, RB = kDkRB;
  constexpr int TILE_BYTES = kT * D * 2;            // one tensor's tile
  constexpr int INSTR_T = TILE_BYTES / 1024;        // 1 KB copies per tensor tile
  constexpr int DMA_PW = 2 * INSTR_T / kDkWaves;    // tile copies per wave
  constexpr int RPI = 1024 / (2 * D);               // rows per copy
  constexpr int LD_PW = 2 * kT * 4 / kDkWaves;      // bytes of lse2/D per wave (2 lanes x 16)
  static_assert(DMA_PW >= 1 && 2 * INSTR_T == DMA_PW * kDkWaves && INSTR_T % DMA_PW == 0,
                "each wave copies whole 1 KB blocks of one tensor");
  static_assert(LD_PW == 32, "two 16-byte lanes of lse2/D per wave");
  // One LDS variable per stage and buffer: the compiler keeps apart the
  // accesses it can attribute to different variables, so a copy in flight
  // into one stage does not make it wait before reads of another (the step
  // loop below is unrolled by 4 so that every stage is named statically).
  __shared__ __attribute__((aligned(1024))) char sQ0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sQ1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sQ2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sQ3[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sO0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sO1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sO2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sO3[TILE_BYTES];
  __shared__ __attribute__((aligned(256))) float sL0[2 * kT];   // lse2[kT], D[kT]
  __shared__ __attribute__((aligned(256))) float sL1[2 * kT];
  __shared__ __attribute__((aligned(256))) float sL2[2 * kT];
  __shared__ __attribute__((aligned(256))) float sL3[2 * kT];
  __shared__ __attribute__((aligned(1024))) f32x4 sP0[kDkWaves / 2][RB][2][64];   // P of a pair, by lane
  __shared__ __attribute__((aligned(1024))) f32x4 sP1[kDkWaves / 2][RB][2][64];
  auto qS = [&](const int st) -> char* { return st == 0 ? sQ0 : st == 1 ? sQ1 : st == 2 ? sQ2 : sQ3; };
  auto oS = [&](const int st) -> char* { return st == 0 ? sO0 : st == 1 ? sO1 : st == 2 ? sO2 : sO3; };
  auto lS = [&](const int st) -> float* { return st == 0 ? sL0 : st == 1 ? sL1 : st == 2 ? sL2 : sL3; };

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  const int n_batch = n_work / (Hkv * n_ktiles);
  int rest = logical;
  const int krank = rest % n_ktiles;                 // 0: the first keys (heaviest causal tile)
  rest /= n_ktiles;
  const int b = rest % n_batch;
  const int g = rest / n_batch;
  const int k0 = krank * kDkKeys;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int pair = wave % (kDkWaves / 2);
  const int role = wave / (kDkWaves / 2);           // 0: S, P, dV;  1: dP, dS, dK
  const int kp = k0 + 16 * RB * pair;               // the pair's first key
  const int offs = Nk - N;

  // K (role 0) or V (role 1) rows -> B operands: lane (key j, group c) holds
  // head-dim 32t + 8c..; keys past Nk read 0 (their dK and dV are not stored)
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const int64_t ks = ((int64_t)b * Nk * Hkv + g) * D;
  const uint32_t kv_bytes = (uint32_t)((Nk - 1) * Hkv + 1) * D * 2;
  const __amdgpu_buffer_rsrc_t kv_rsrc = make_rsrc((role == 0 ? k : v) + ks, kv_bytes);
  bf16x8 kvf[RB][DT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t off = (uint32_t)(kp + 16 * rb + l16) * kv_row_bytes + grp * 16;
#pragma unroll
    for (int t = 0; t < DT; ++t) kvf[rb][t] = __builtin_bit_cast(bf16x8, load16_once(kv_rsrc, off + t * 64));
  }

  // query tiles: causal row i sees key j iff j <= i + offs, so the
  // workgroup's keys are seen from row k0 - offs on.  Iteration `it` takes
  // tile ntq - 1 - it / G of query head g*G + it % G.
  const int qt0 = CAUSAL ? min(ntq, max(0, k0 - offs) / kT) : 0;
  const int n_it = G * (ntq - qt0);

  // ---- copies: wave w moves 1 KB blocks w*DMA_PW.. of the stage's [Q, dO]
  // pair (lane l of a block fills row blk*RPI + l/CPR, physical chunk l%CPR),
  // all of one tensor, and with lanes 0-1 bytes 32w..32w+31 of the tile's
  // lse2/D block.  Every wave issues DMA_PW + 1 copies per tile.
  const int dma_t = wave * DMA_PW / INSTR_T;         // 0: Q, 1: dO
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint16_t* src = (dma_t == 0 ? q : dout) + (int64_t)b * N * Hq * D;
  uint32_t voff[DMA_PW];
#pragma unroll
  for (int i = 0; i < DMA_PW; ++i) {
    const int row = ((wave * DMA_PW + i) % INSTR_T) * RPI + lane / CPR;
    voff[i] = (uint32_t)row * q_row_bytes + (uint32_t)(((lane % CPR) ^ swz<CPR>(row)) * 16);
  }
  const uint32_t ld_voff = (uint32_t)(LD_PW * wave + 16 * lane);
  // Every call issues the same copies: for an iteration past the last, the
  // views are empty, so the copies write zeros into a free stage and read
  // nothing; the waits below count copies.
  // The iteration of the next copy (tile nx_ti of head g*G + nx_h), kept
  // incrementally: the loop's scalar work is a large share of a step, and
  // these need no division.  A view runs from row i0 of its head to row N-1
  // (rows past N read 0), whatever the head.
  int nx_it = 0, nx_h = 0;
  const uint16_t* nx_row = src + ((int64_t)(ntq - 1) * kT * Hq + g * G) * D;   // row i0 of head g*G
  uint32_t nx_bytes = (uint32_t)((N - 1 - (ntq - 1) * kT) * Hq + 1) * D * 2;
  const float* nx_ld = ld + ((int64_t)(b * Hq + g * G) * ntq + ntq - 1) * (2 * kT);
  auto issue = [&](const int st) __attribute__((always_inline)) {
    const bool real = nx_it < n_it;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(nx_row + nx_h * D, real ? nx_bytes : 0u);
    char* dst = dma_t == 0 ? qS(st) : oS(st);
#pragma unroll
    for (int i = 0; i < DMA_PW; ++i)
      buffer_load16_to_lds(r, voff[i], 0, (lds_void*)(dst + ((wave * DMA_PW + i) % INSTR_T) * 1024));
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(nx_ld, real ? 2 * kT * 4 : 0);
    if (lane < 2)
      buffer_load16_to_lds(rl, ld_voff, 0, (lds_void*)(reinterpret_cast<char*>(lS(st)) + LD_PW * wave));
    if (real) {
      ++nx_it;
      nx_ld += (int64_t)ntq * (2 * kT);
      if (++nx_h == G) {                        // next tile down, first head
        nx_h = 0;
        nx_row -= (int64_t)kT * Hq * D;
        nx_bytes += (uint32_t)kT * Hq * D * 2;
        nx_ld -= (int64_t)G * ntq * (2 * kT) + 2 * kT;
      }
    }
  };

  int r_off[2][DT];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = pi16(kb, l16);
#pragma unroll
    for (int t = 0; t < DT; ++t) r_off[kb][t] = row * (2 * D) + (((4 * t + grp) ^ swz<CPR>(row)) * 16);
  }
  const int trow = 8 * grp + (l16 >> 2);
  int t_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 2 * db + ((l16 & 3) >> 1);
    t_off[db] = trow * (2 * D) + ((chunk ^ swz<CPR>(trow)) * 16) + (l16 & 1) * 8;
  }

  f32x4 acc[RB][DB];   // dV^T (role 0) or dK^T (role 1): lane (key j, group c) item r = head-dim 16db + 4c + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The two products of a tile: mm1 computes S = Q K^T (wave A, `rows` = Q)
  // or dP = dO V^T (wave B, `rows` = dO) into x; mm2 adds dO^T P (wave A)
  // or Q^T dS (wave B) to acc, wf holding P or dS as B operands and trf the
  // transposed reads of dO or Q (fetched by prefetch_tr).  x: lane (key j,
  // group c) item r of block kb = query 8c + 4kb + r of the tile.
  f32x4 x[RB][2];
  bf16x8 wf[RB];
  bf16x8 trf[DB];
  bf16x8 ra[2][DT];
  auto read_rows = [&](const char* rows) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < DT; ++t) ra[kb][t] = __builtin_bit_cast(bf16x8, load16(rows + r_off[kb][t]));
  };
  auto mm1 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) x[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          x[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[kb][t], kvf[rb][t], x[rb][kb], 0, 0, 0);
    }
  };
  auto prefetch_tr = [&](const char* trs) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 lo = lds_read_tr16(trs + t_off[db]);
      const u32x2 hi = lds_read_tr16(trs + t_off[db] + 4 * (2 * D));
      trf[db] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };
  auto mm2 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(trf[db], wf[rb], acc[rb][db], 0, 0, 0);
  };
  auto pack = [&](float (*w)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const u32x4 u = {pack_bf16x2(w[rb][0], w[rb][1]), pack_bf16x2(w[rb][2], w[rb][3]),
                       pack_bf16x2(w[rb][4], w[rb][5]), pack_bf16x2(w[rb][6], w[rb][7])};
      wf[rb] = __builtin_bit_cast(bf16x8, u);
    }
  };
  // wave A: P = 2^(s c - lse2) of the tile at row i0 (0 where masked; key
  // kp + 16rb + l16 is visible to query i0 + 8c + i iff key <= i0 + 8c + i +
  // offs), into wf and, in fp32, into the pair's slot of `pbuf`
  auto soft_a = [&](const int i0, const float* ldv, f32x4 (*pbuf)[RB][2][64]) __attribute__((always_inline)) {
    const f32x4 la = *reinterpret_cast<const f32x4*>(&ldv[8 * grp]);
    const f32x4 lb = *reinterpret_cast<const f32x4*>(&ldv[8 * grp + 4]);
    const bool masked = CAUSAL && i0 + offs < kp + 16 * RB - 1;
    f32x4* pslot = &pbuf[pair][0][0][lane];        // [rb][half] at stride 64
    float w[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) w[rb][4 * kb + r] = fast_exp2(fmaf(x[rb][kb][r], c, -(kb == 0 ? la[r] : lb[r])));
      if (masked) {
        const int rel = (i0 + 8 * grp + offs) - (kp + 16 * rb + l16);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[rb][i] = i >= -rel ? w[rb][i] : 0.0f;
      }
      pslot[128 * rb] = f32x4{w[rb][0], w[rb][1], w[rb][2], w[rb][3]};
      pslot[128 * rb + 64] = f32x4{w[rb][4], w[rb][5], w[rb][6], w[rb][7]};
    }
    pack(w);
  };
  // wave B: dS = P o (dP - D), P from wave A's slot in `pbuf`
  auto soft_b = [&](const float* ldv, f32x4 (*pbuf)[RB][2][64]) __attribute__((always_inline)) {
    const f32x4 da = *reinterpret_cast<const f32x4*>(&ldv[kT + 8 * grp]);
    const f32x4 dbv = *reinterpret_cast<const f32x4*>(&ldv[kT + 8 * grp + 4]);
    const f32x4* pslot = &pbuf[pair][0][0][lane];
    float w[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x4 p0 = pslot[128 * rb], p1 = pslot[128 * rb + 64];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[rb][r] = p0[r] * (x[rb][0][r] - da[r]);
        w[rb][4 + r] = p1[r] * (x[rb][1][r] - dbv[r]);
      }
    }
    pack(w);
  };

  // Step t (ST = t % NS) has two phases; in each, one wave of a pair runs its
  // MFMAs while the other (on the same SIMD) runs its exponentials or dS:
  //   phase 2t:   A: dV += dO_{t-1}^T P_{t-1}, S_t = Q_t K^T  |  B: dS_{t-1}
  //   phase 2t+1: B: dK += Q_{t-1}^T dS_{t-1}, dP_t = dO_t V^T  |  A: P_t -> LDS
  // Tile t is read in phases 2t..2t+3; the copies of tile t+PD go out at the
  // start of step t into the stage of tile t+PD-NS (last read in phase
  // 2t-1).
  constexpr int NS = kDkNS, PD = kDkNS - 2;
  int cur_h = 0, cur_i0 = (ntq - 1) * kT;         // wave A: head index and first row of iteration t
  auto step = [&](const int t, const int ST) __attribute__((always_inline)) {
    const int SB = (ST + NS - 1) % NS;              // stage of tile t-1
    f32x4 (*p_cur)[RB][2][64] = (ST & 1) ? sP1 : sP0;
    f32x4 (*p_prev)[RB][2][64] = (ST & 1) ? sP0 : sP1;
    issue((ST + PD) % NS);                  // iteration t + PD
    // (an MFMA phase issues all its LDS reads first: the transposed operands
    // of mm2, then the rows of mm1, which land while mm2 runs)
    if (role == 0) {
      if (t >= 1) prefetch_tr(oS(SB));
      if (t < n_it) read_rows(qS(ST));
      if (t >= 1) mm2();
      if (t < n_it) mm1();
    } else if (t >= 1) {
      soft_b(lS(SB), p_prev);
    }
    barrier_no_fence();
    if (role == 1) {
      if (t >= 1) prefetch_tr(qS(SB));
      if (t < n_it) read_rows(oS(ST));
      if (t >= 1) mm2();
      if (t < n_it) mm1();
    } else if (t < n_it) {
      soft_a(cur_i0, lS(ST), p_cur);
      if (++cur_h == G) {                      // the tile of iteration t+1
        cur_h = 0;
        cur_i0 -= kT;
      }
    }
    wait_vmem_le<(PD - 1) * (DMA_PW + 1)>();   // tile t+1 has landed
    barrier_no_fence();                        // ... for every wave
  };

  if (n_it > 0) {
#pragma unroll
    for (int t = 0; t < PD; ++t) issue(t);
    wait_vmem_le<(PD - 1) * (DMA_PW + 1)>();
    barrier_no_fence();
    // steps 0..n_it, unrolled by NS so that every stage is named statically;
    // the check after each step leaves the loop (it never skips ahead)
    auto round = [&](const int s0) __attribute__((always_inline)) -> bool {
      step(s0, 0);
      if (s0 + 1 > n_it) return false;
      step(s0 + 1, 1);
      if (s0 + 2 > n_it) return false;
      step(s0 + 2, 2);
      if (s0 + 3 > n_it) return false;
      step(s0 + 3, 3);
      if (s0 + 4 > n_it) return false;
      return true;
    };
    for (int s0 = 0; round(s0); s0 += NS) {
    }
  }
  wait_vmem_all();          // no copy may land after the workgroup ends

  uint16_t* dst = role == 0 ? dv : dk;
  const float f = role == 0 ? 1.0f : scale;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int key = kp + 16 * rb + l16;
    if (key < Nk) {
      const int64_t o = (((int64_t)b * Nk + key) * Hkv + g) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 a = acc[rb][db];
        u32x2 u;
        u[0] = pack_bf16x2(a[0] * f, a[1] * f);
        u[1] = pack_bf16x2(a[2] * f, a[3] * f);
        *reinterpret_cast<u32x2*>(dst + o + 16 * db) = u;
      }
    }
  }
}

#ifndef BWD_WQ
#define BWD_WQ 4
#endif
#ifndef BWD_RBQ
#define BWD_RBQ 2
#endif
constexpr int kWQ = BWD_WQ, kRBQ = BWD_RBQ;    // bwd_dq: waves x 16-row blocks per wave

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const float c = a.scale * kLog2e;
  const int ntq = (a.N + kT - 1) / kT;
  if ((int64_t)a.B * a.N * a.Hq > 0) {
    const int64_t threads = ((int64_t)a.B * a.N * a.Hq + (int64_t)a.B * a.Hq * (ntq * kT - a.N)) * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + kThr - 1) / kThr)), dim3(kThr), 0,
                       a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, a.ld, a.B, a.N, a.Hq, ntq);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr int ROWS_G = 16 * kRBQ * kWQ;
    const int n_qtiles = (a.N + ROWS_G - 1) / ROWS_G;
    const int64_t n_work = (int64_t)a.B * a.Hq * n_qtiles;
    const int64_t grid = (n_work + 7) / 8 * 8;
    // (no query rows: no dQ to compute; the dK/dV kernel below still runs and
    // writes dK = dV = 0, since no query sees any key)
    if (grid > 0) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, kWQ, kRBQ>), dim3((unsigned)grid), dim3(64 * kWQ), 0, a.stream,
                         (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                         a.ld, (uint16_t*)a.dq, a.N, a.Nk, a.Hq, a.Hkv, c, a.scale, ntq, n_qtiles, (int)n_work);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (a.Nk > 0) {
    const int n_ktiles = (a.Nk + kDkKeys - 1) / kDkKeys;
    const int64_t n_work = (int64_t)a.B * a.Hkv * n_ktiles;
    const int64_t grid = (n_work + 7) / 8 * 8;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(64 * kDkWaves), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                       a.ld, (uint16_t*)a.dk, (uint16_t*)a.dv, a.N, a.Nk, a.Hq, a.Hkv, c, a.scale, ntq, n_ktiles,
                       (int)n_work);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
