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
//  * bwd_pre_kernel: D and the base-2 LSE (+inf for a row without keys, so
//    that its P is 0) per (batch, head, row), into the workspace;
//  * bwd_dq_kernel: one workgroup per (query tile, query head, batch),
//    streaming K/V tiles: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T;
//  * bwd_dkdv_kernel: one workgroup per (key tile, kv head, batch), streaming
//    the Q and dO tiles of the group's query heads: S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P, dK^T += Q^T dS.
// Both use the forward's MFMA layout: with the streamed operand's rows fed in
// the permuted order pi16, a lane of a 16x16x32 result holds 8 consecutive
// entries of one row of P or dS, which is exactly its slice of the next
// product's B operand, so P and dS never leave registers.  The second
// operand of each product is either held in registers for the whole loop (Q
// and dO in bwd_dq, K and V in bwd_dkdv) or read from the streamed LDS tile:
// by rows (ds_read_b128) as an A operand, or transposed (ds_read_b64_tr_b16)
// as the A operand of a transposed product.  S and dP are computed in both
// kernels: 7 matrix products in all, against 5 with atomics on dQ.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kT = 32;          // rows of a streamed tile (keys in bwd_dq, queries in bwd_dkdv)
constexpr int kThr = 256;       // threads of the staging copies and the pre kernel

__device__ __forceinline__ int pi16(int kb, int i) { return 8 * (i >> 2) + 4 * kb + (i & 3); }

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

// ---- D_i = dO_i . O_i and lse2_i = LSE_i log2(e) (+inf when LSE_i = -inf),
// both [B, Hq, N]; D/8 lanes per (b, i, h) row of the BSHD tensors.
template <int D>
__global__ __launch_bounds__(kThr) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ dsum,
                                                       float* __restrict__ lse2, int B, int N, int Hq) {
  constexpr int LPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * kThr + threadIdx.x;
  const int64_t row = gid / LPR;
  const int part = (int)(gid % LPR);
  const int64_t nrows = (int64_t)B * N * Hq;
  float acc = 0.0f;
  if (row < nrows) {
    const u32x4 a = load16(o + row * D + part * 8);
    const u32x4 g = load16(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += bf16_lo(a[w]) * bf16_lo(g[w]) + bf16_hi(a[w]) * bf16_hi(g[w]);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < nrows && part == 0) {
    const int h = (int)(row % Hq);
    const int64_t bi = row / Hq;
    const int i = (int)(bi % N);
    const int64_t b = bi / N;
    const int64_t idx = (b * Hq + h) * N + i;
    dsum[idx] = acc;
    const float l = lse[idx];
    lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
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
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dsum,
    uint16_t* __restrict__ dq, int N, int Nk, int Hq, int Hkv, float c, float scale, int n_qtiles, int n_work) {
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
      qf[rb][t] = __builtin_bit_cast(bf16x8, buffer_load16(q_rsrc, off + t * 64));
      df[rb][t] = __builtin_bit_cast(bf16x8, buffer_load16(d_rsrc, off + t * 64));
    }
    const bool in = row >= 0 && row < N;
    const int64_t li = ((int64_t)b * Hq + h) * N + (in ? row : 0);
    l2[rb] = in ? lse2[li] : INFINITY;                // P = 0 for absent rows
    ds[rb] = in ? dsum[li] : 0.0f;
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

#ifndef BWD_OCC
#define BWD_OCC 1
#endif
#ifndef BWD_RA
#define BWD_RA 2
#endif


// ---- dK and dV.  Workgroup: WK waves x (16 RB) keys of one kv head; it
// streams 32-row Q and dO tiles (with their lse2 and D) of every query head
// of the group, from the first query tile that sees one of its keys.
template <int D, bool CAUSAL, int WK, int RB>
__global__ __launch_bounds__(64 * WK, BWD_OCC) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dsum,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int Nk, int Hq, int Hkv, float c, float scale,
    int n_ktiles, int n_work) {
  constexpr int DT = D / 32, DB = D / 16, CPR = D / 8;
  constexpr int KEYS_W = 16 * RB, KEYS_G = KEYS_W * WK;
  __shared__ __attribute__((aligned(1024))) uint16_t sQ[2][kT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sO[2][kT * D];
  __shared__ __attribute__((aligned(16))) float sL[2][kT];
  __shared__ __attribute__((aligned(16))) float sD[2][kT];

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  const int n_batch = n_work / (Hkv * n_ktiles);
  int rest = logical;
  const int krank = rest % n_ktiles;                 // 0: the first keys (heaviest causal tile)
  rest /= n_ktiles;
  const int b = rest % n_batch;
  const int g = rest / n_batch;
  const int k0 = krank * KEYS_G;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int kw = k0 + KEYS_W * wave;
  const int offs = Nk - N;

  // K and V rows -> B operands (lane (key j, group c): head-dim 32t + 8c..);
  // keys past Nk read 0 (their dK and dV are not stored)
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const int64_t ks = ((int64_t)b * Nk * Hkv + g) * D;
  const uint32_t kv_bytes = (uint32_t)((Nk - 1) * Hkv + 1) * D * 2;
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(k + ks, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(v + ks, kv_bytes);
  bf16x8 kf[RB][DT], vf[RB][DT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t off = (uint32_t)(kw + 16 * rb + l16) * kv_row_bytes + grp * 16;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      kf[rb][t] = __builtin_bit_cast(bf16x8, buffer_load16(k_rsrc, off + t * 64));
      vf[rb][t] = __builtin_bit_cast(bf16x8, buffer_load16(v_rsrc, off + t * 64));
    }
  }

  // query tiles: causal rows i see key j iff j <= i + offs, so this
  // workgroup's keys are seen from row k0 - offs on
  const int nq = (N + kT - 1) / kT;
  const int qt0 = CAUSAL ? min(nq, max(0, k0 - offs) / kT) : 0;
  const int per_head = nq - qt0;
  const int n_it = G * per_head;
  // the tile at row i0 needs a mask for this wave iff some key of the wave
  // is invisible to its first row: i0 + offs < kw + KEYS_W - 1

  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  // (N = 0: no query tile is loaded, n_it = 0; the view is then empty)
  const uint32_t q_bytes = N > 0 ? (uint32_t)((N - 1) * Hq + 1) * D * 2 : 0u;
  auto head_rsrc = [&](const uint16_t* base, int h) {
    return make_rsrc(base + ((int64_t)b * N * Hq + h) * D, q_bytes);
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

  f32x4 acc_k[RB][DB], acc_v[RB][DB];   // dK^T, dV^T: lane (key j, group c) item r = head-dim 16db + 4c + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_k[rb][db] = acc_v[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging of iteration `it`: Q and dO tiles of head g*G + it/per_head,
  // rows (qt0 + it%per_head)*32..; lse2 (+inf past N) and D for those rows.
  // Their loads mostly miss L2, so they run two tiles ahead: two register
  // sets, tile t in set t % 2; the loads of tile it+2 are issued at the start
  // of iteration it, and tile it+1 is stored to LDS at its end.  (A third set
  // makes the unrolled loop spill at d=128.)  CT threads copy: one 16-byte
  // chunk each per tensor at d=128 with 8 waves.
  constexpr int CT = 64 * WK < kT * CPR ? 64 * WK : kT * CPR;
  struct Stage {
    TileCopy<D, CT> cq, co;
    float l = INFINITY, d = 0.0f;
  };
  Stage st0, st1;
  auto load_it = [&](const int it, Stage& st) {
    const int h = g * G + it / per_head;
    const int i0 = (qt0 + it % per_head) * kT;
    if (tid < CT) {
      st.cq.load(head_rsrc(q, h), i0, q_row_bytes, tid);
      st.co.load(head_rsrc(dout, h), i0, q_row_bytes, tid);
    }
    if (tid < kT) {
      const int row = i0 + tid;
      const int64_t li = ((int64_t)b * Hq + h) * N + (row < N ? row : 0);
      st.l = row < N ? lse2[li] : INFINITY;
      st.d = row < N ? dsum[li] : 0.0f;
    }
  };
  auto store_it = [&](const int buf, const Stage& st) {
    if (tid < CT) {
      st.cq.store(reinterpret_cast<char*>(sQ[buf]), tid);
      st.co.store(reinterpret_cast<char*>(sO[buf]), tid);
    }
    if (tid < kT) {
      sL[buf][tid] = st.l;
      sD[buf][tid] = st.d;
    }
  };

  if (n_it > 0) {
    load_it(0, st0);
    if (n_it > 1) load_it(1, st1);
    store_it(0, st0);
    __syncthreads();
  }
  // iteration `it`: `ld` receives tile it+2, `nx` holds tile it+1
  auto step = [&](const int it, Stage& ld, Stage& nx) __attribute__((always_inline)) {
    if (it + 2 < n_it) load_it(it + 2, ld);
    const int i0 = (qt0 + it % per_head) * kT;
    const char* qt = reinterpret_cast<const char*>(sQ[it & 1]);
    const char* ot = reinterpret_cast<const char*>(sO[it & 1]);
    // S = Q K^T and dP = dO V^T: lane (key j, group c) item r of block kb =
    // query 8c + 4kb + r of the tile
    f32x4 s[RB][2], dp[RB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][kb] = dp[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 qa = __builtin_bit_cast(bf16x8, load16(qt + r_off[kb][t]));
        const bf16x8 oa = __builtin_bit_cast(bf16x8, load16(ot + r_off[kb][t]));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[rb][t], s[rb][kb], 0, 0, 0);
          dp[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[rb][t], dp[rb][kb], 0, 0, 0);
        }
      }
    }
    // LDS reads run BWD_RA steps ahead of the MFMAs that use them
    if constexpr (BWD_RA > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * BWD_RA, 0);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);
      }
    }
    // lse2 and D of this lane's 8 queries (8c..8c+7)
    const f32x4 la = *reinterpret_cast<const f32x4*>(&sL[it & 1][8 * grp]);
    const f32x4 lb = *reinterpret_cast<const f32x4*>(&sL[it & 1][8 * grp + 4]);
    const f32x4 da = *reinterpret_cast<const f32x4*>(&sD[it & 1][8 * grp]);
    const f32x4 dbv = *reinterpret_cast<const f32x4*>(&sD[it & 1][8 * grp + 4]);
    const bool masked = CAUSAL && i0 + offs < kw + KEYS_W - 1;
    bf16x8 pf[RB], dsf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float p[8], e[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float l = kb == 0 ? la[r] : lb[r];
          const float dd = kb == 0 ? da[r] : dbv[r];
          p[4 * kb + r] = fast_exp2(fmaf(s[rb][kb][r], c, -l));
          e[4 * kb + r] = p[4 * kb + r] * (dp[rb][kb][r] - dd);
        }
      if (masked) {
        // key kw + 16rb + l16 is visible to query i0 + 8c + i iff key <= i0 + 8c + i + offs
        const int rel = (i0 + 8 * grp + offs) - (kw + 16 * rb + l16);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = i >= -rel ? p[i] : 0.0f;
          e[i] = i >= -rel ? e[i] : 0.0f;
        }
      }
      const u32x4 wp = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
      const u32x4 we = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                        pack_bf16x2(e[6], e[7])};
      pf[rb] = __builtin_bit_cast(bf16x8, wp);
      dsf[rb] = __builtin_bit_cast(bf16x8, we);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (transposed reads of the dO and Q tiles)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 olo = lds_read_tr16(ot + t_off[db]);
      const u32x2 ohi = lds_read_tr16(ot + t_off[db] + 4 * (2 * D));
      const u32x2 qlo = lds_read_tr16(qt + t_off[db]);
      const u32x2 qhi = lds_read_tr16(qt + t_off[db] + 4 * (2 * D));
      const bf16x8 oa = __builtin_bit_cast(bf16x8, u32x4{olo[0], olo[1], ohi[0], ohi[1]});
      const bf16x8 qa = __builtin_bit_cast(bf16x8, u32x4{qlo[0], qlo[1], qhi[0], qhi[1]});
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc_v[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, pf[rb], acc_v[rb][db], 0, 0, 0);
        acc_k[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, dsf[rb], acc_k[rb][db], 0, 0, 0);
      }
    }
    if constexpr (BWD_RA > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * BWD_RA, 0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);
      }
    }
    if (it + 1 < n_it) store_it((it + 1) & 1, nx);  // last read in iteration it-1, before its barrier
    __syncthreads();
  };
  for (int it = 0; it < n_it; it += 2) {
    step(it, st0, st1);
    if (it + 1 >= n_it) break;
    step(it + 1, st1, st0);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int key = kw + 16 * rb + l16;
    if (key < Nk) {
      const int64_t o = (((int64_t)b * Nk + key) * Hkv + g) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 a = acc_k[rb][db], e = acc_v[rb][db];
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(a[0] * scale, a[1] * scale);
        wk[1] = pack_bf16x2(a[2] * scale, a[3] * scale);
        wv[0] = pack_bf16x2(e[0], e[1]);
        wv[1] = pack_bf16x2(e[2], e[3]);
        *reinterpret_cast<u32x2*>(dk + o + 16 * db) = wk;
        *reinterpret_cast<u32x2*>(dv + o + 16 * db) = wv;
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
#ifndef BWD_WK
#define BWD_WK 8
#endif
#ifndef BWD_RBK
#define BWD_RBK 1
#endif
constexpr int kWQ = BWD_WQ, kRBQ = BWD_RBQ;    // bwd_dq: waves x 16-row blocks per wave
constexpr int kWK = BWD_WK, kRBK = BWD_RBK;    // bwd_dkdv: waves x 16-key blocks per wave

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const float c = a.scale * kLog2e;
  if ((int64_t)a.B * a.N * a.Hq > 0) {
    const int64_t threads = (int64_t)a.B * a.N * a.Hq * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + kThr - 1) / kThr)), dim3(kThr), 0,
                       a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, a.dsum, a.lse2, a.B, a.N,
                       a.Hq);
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
                         a.lse2, a.dsum, (uint16_t*)a.dq, a.N, a.Nk, a.Hq, a.Hkv, c, a.scale, n_qtiles, (int)n_work);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (a.Nk > 0) {
    constexpr int KEYS_G = 16 * kRBK * kWK;
    const int n_ktiles = (a.Nk + KEYS_G - 1) / KEYS_G;
    const int64_t n_work = (int64_t)a.B * a.Hkv * n_ktiles;
    const int64_t grid = (n_work + 7) / 8 * 8;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, kWK, kRBK>), dim3((unsigned)grid), dim3(64 * kWK), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse2, a.dsum, (uint16_t*)a.dk, (uint16_t*)a.dv, a.N, a.Nk, a.Hq,
                       a.Hkv, c, a.scale, n_ktiles, (int)n_work);
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
