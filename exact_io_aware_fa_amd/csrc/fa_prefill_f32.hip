// fa_prefill_f32.hip -- tiled exact attention forward in fp32 throughout, for
// gfx950.  Same method as the bf16 kernel (K/V taken tile by tile, online
// softmax with a running row max and row sum, causal mask inside the tile,
// fully masked tiles skipped; ai6s.net page, sections "FlashAttention
// changes the dataflow, not the algorithm" and "what ops-transformer adds"),
// but every product and sum is an fp32 FMA on the vector ALU: no reduced-
// precision matrix mode is involved, so the result stays within fp32 rounding
// of exact attention.
//
// Mapping: a workgroup owns ROWS = 64 / TPR query rows (TPR = D / 4 lanes
// per row) and splits their key tiles over its kWaves waves: wave w takes
// tiles w, w + kWaves, ..., with its own running max and sum, and the waves'
// partial results are merged at the end (each partial is the softmax of its
// own keys scaled by 2^(its max); the merge rescales them to the common max,
// as the online softmax does between tiles).  Within a wave, a lane holds its
// row's whole q and computes the full dot products of its KPL = 32 / TPR keys
// of the tile, so a tile's row max takes one reduction over the row's lanes;
// for the weighted sum of V a lane owns 4 head-dim entries of the row and
// reads the tile's 32 weights of its row from a per-wave LDS buffer.  Keys
// and rows past the end are read as 0 through bounded buffer views.  A lane's
// loads go out in batches (a key's row, 8 or 16 keys' V slices), so that a
// tile costs a few memory round trips rather than one per key.  Even one
// head of a few hundred rows spreads over many waves with short chains of
// dependent work: the single-head N = 256, d = 64 case (64 workgroups of 8
// waves, one 32-key tile per wave) is bound by the launch and one tile's
// latency.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kTileKeys = 32;
constexpr int kWaves = 8;                 // waves per workgroup (key-tile split)
constexpr int kThreads = 64 * kWaves;
constexpr int kSlice = 4;                 // output head-dim entries per lane

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int N, int Nk, int Hq, int Hkv, float c,
    int n_qtiles, int n_work) {
  constexpr int TPR = D / kSlice;                 // lanes per query row
  constexpr int ROWS = 64 / TPR;                  // query rows per workgroup
  constexpr int KPL = kTileKeys / TPR;            // keys per lane in a tile's dot products
  constexpr int DC = D / 4;                       // 16-byte chunks of a row
  static_assert(ROWS * TPR == 64 && KPL * TPR == kTileKeys, "a row's lanes lie in one wave");
  __shared__ __attribute__((aligned(16))) float sP[kWaves][ROWS][kTileKeys];   // a tile's weights by row
  __shared__ float sM[kWaves][64], sL[kWaves][64];
  __shared__ f32x4 sA[kWaves][64];

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  int rest = logical;
  const int hig = rest % G;
  rest /= G;
  const int qrank = rest % n_qtiles;
  rest /= n_qtiles;
  const int g = rest % Hkv;
  const int b = rest / Hkv;
  const int qt = CAUSAL ? (n_qtiles - 1 - qrank) : qrank;
  const int h = g * G + hig;
  const int q0 = qt * ROWS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane / TPR;                       // row of the lane within the workgroup
  const int part = lane % TPR;
  const int row = q0 + r;
  const int offs = Nk - N;
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 4;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 4;
  // bounded views of this (batch, head) q slice and (batch, kv head) K/V slices
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(q + ((int64_t)b * N * Hq + h) * D,
                                                  (uint32_t)((N - 1) * Hq + 1) * D * 4);
  const uint32_t kv_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * Hkv + 1) * D * 4 : 0u;
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(k + ((int64_t)b * Nk * Hkv + g) * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(v + ((int64_t)b * Nk * Hkv + g) * D, kv_bytes);
  auto ld4 = [](__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  };

  f32x4 qf[DC];                                   // the row's q (0 past N)
#pragma unroll
  for (int t = 0; t < DC; ++t) qf[t] = ld4(q_rsrc, (uint32_t)row * q_row_bytes + t * 16);

  float m_run = -INFINITY;                        // running max of the row (scaled, base 2)
  float l_part = 0.0f;                            // this lane's share of the running row sum
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};               // head-dim entries 4*part.. of the row's output

  int n_kv = (Nk + kTileKeys - 1) / kTileKeys;
  if (CAUSAL) {
    const int last_key = min(q0 + ROWS - 1, N - 1) + offs;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kTileKeys + 1);
  }

  for (int j = wave; j < n_kv; j += kWaves) {
    const int j0 = j * kTileKeys;
    float s[KPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int key = j0 + part * KPL + i;
      // the key's row in batches of up to 16 loads (one memory round trip
      // each; two at d = 128, where the row and q fill half the registers)
      constexpr int KB = DC < 16 ? DC : 16;
      float d4[4] = {0.f, 0.f, 0.f, 0.f};         // four partial sums (independent chains)
#pragma unroll
      for (int t0 = 0; t0 < DC; t0 += KB) {
        f32x4 kr[KB];
#pragma unroll
        for (int t = 0; t < KB; ++t) kr[t] = ld4(k_rsrc, (uint32_t)key * kv_row_bytes + (t0 + t) * 16);
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) d4[e] = fmaf(qf[t0 + t][e], kr[t][e], d4[e]);
      }
      const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      const bool vis = key < Nk && (!CAUSAL || key <= row + offs);
      s[i] = vis ? dot * c : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float m_new = fmaxf(m_run, mx);
    const float mu = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - mu);    // 0 while nothing was visible
    l_part *= alpha;
    acc *= alpha;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const float p = fast_exp2(s[i] - mu);
      l_part += p;
      sP[wave][r][part * KPL + i] = p;
    }
    // (the wave's LDS accesses run in order: the reads below see the writes
    // above, and the next tile's writes follow these reads)
    __builtin_amdgcn_wave_barrier();
    // V in batches of VB keys (one round trip each)
    constexpr int VB = D == 64 ? 16 : 8;
#pragma unroll
    for (int hb = 0; hb < kTileKeys / VB; ++hb) {
      f32x4 vr[VB];
#pragma unroll
      for (int e = 0; e < VB; ++e) vr[e] = ld4(v_rsrc, (uint32_t)(j0 + VB * hb + e) * kv_row_bytes + part * 16);
#pragma unroll
      for (int k4 = 0; k4 < VB / 4; ++k4) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&sP[wave][r][VB * hb + 4 * k4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += p4[e] * vr[4 * k4 + e];
      }
    }
    __builtin_amdgcn_wave_barrier();
    m_run = m_new;
  }
  // the row's sum over its lanes, then the merge of the waves' partials
  float l_run = l_part;
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) l_run += __shfl_xor(l_run, off, 64);
  sM[wave][lane] = m_run;
  sL[wave][lane] = l_run;
  sA[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sM[w][lane]);
  const float mu = m == -INFINITY ? 0.0f : m;
  float l = 0.0f;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = fast_exp2(sM[w][lane] - mu);  // 0 for a wave that saw no key
    l = fmaf(sL[w][lane], f, l);
    a += f * sA[w][lane];
  }

  if (row < N) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* dst = o + ((int64_t)b * N + row) * ((int64_t)Hq * D) + (int64_t)h * D + part * kSlice;
    *reinterpret_cast<f32x4*>(dst) = a * inv;
    if (part == 0)
      lse[((int64_t)b * Hq + h) * N + row] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a) {
  constexpr int ROWS = 64 / (D / kSlice);
  const int n_qtiles = (a.N + ROWS - 1) / ROWS;
  const int64_t n_work = (int64_t)a.B * a.Hq * n_qtiles;
  if (n_work == 0) return hipSuccess;
  const int64_t grid = (n_work + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.N,
                     a.Nk, a.Hq, a.Hkv, a.scale * kLog2e, n_qtiles, (int)n_work);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
