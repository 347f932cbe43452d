// fa_prefill_f32.hip -- tiled exact attention forward in fp32 throughout, for
// gfx950.  Same method as the bf16 kernel (K/V tiles streamed through LDS,
// online softmax with a running row max and row sum, causal mask inside the
// tile, fully masked tiles skipped; ai6s.net page, sections "FlashAttention
// changes the dataflow, not the algorithm" and "what ops-transformer adds"),
// but every product and sum is an fp32 FMA on the vector ALU: no reduced-
// precision matrix mode is involved, so the result stays within fp32 rounding
// of exact attention.
//
// Mapping: a wave owns 64 / TPR query rows; TPR = D / 4 lanes share one row,
// each holding 4 of its head-dim entries of q and of the output accumulator
// (a row's dot products are summed across its lanes by a shuffle tree), so
// that even one head of a few hundred rows spreads over many waves: the
// single-head N = 256, d = 64 case takes 0.038 ms, against 0.153 ms with one
// lane per row.
// K and V tiles of 32 keys are staged in LDS and read as broadcasts.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kTileKeys = 32;
constexpr int kThreads = 64;
constexpr int kSlice = 4;             // head-dim entries per lane

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int N, int Nk, int Hq, int Hkv, float c,
    int n_qtiles, int n_work) {
  constexpr int TPR = D / kSlice;                 // lanes per query row
  constexpr int ROWS = kThreads / TPR;            // query rows per workgroup
  static_assert(TPR <= kThreads && ROWS * TPR == kThreads, "a row's lanes lie in one wave");
  __shared__ __attribute__((aligned(16))) float sK[kTileKeys * D];
  __shared__ __attribute__((aligned(16))) float sV[kTileKeys * D];

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
  const int row = q0 + tid / TPR;
  const int part = tid % TPR;
  const int offs = Nk - N;
  const int64_t q_row_stride = (int64_t)Hq * D;
  const int64_t kv_row_stride = (int64_t)Hkv * D;
  const float* kbase = k + ((int64_t)b * Nk * Hkv + g) * D;
  const float* vbase = v + ((int64_t)b * Nk * Hkv + g) * D;

  float qv[kSlice], acc[kSlice];
  {
    const float* src = q + ((int64_t)b * N + row) * q_row_stride + (int64_t)h * D + part * kSlice;
#pragma unroll
    for (int e = 0; e < kSlice; ++e) {
      qv[e] = row < N ? src[e] : 0.0f;
      acc[e] = 0.0f;
    }
  }
  float m_run = -INFINITY, l_run = 0.0f;

  int n_kv = (Nk + kTileKeys - 1) / kTileKeys;
  if (CAUSAL) {
    const int last_key = min(q0 + ROWS - 1, N - 1) + offs;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kTileKeys + 1);
  }

  for (int j = 0; j < n_kv; ++j) {
    const int j0 = j * kTileKeys;
    __syncthreads();
    for (int idx = tid; idx < kTileKeys * D / 4; idx += kThreads) {
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      const int key = j0 + r;
      f32x4 kw = {0.f, 0.f, 0.f, 0.f}, vw = {0.f, 0.f, 0.f, 0.f};
      if (key < Nk) {
        kw = *reinterpret_cast<const f32x4*>(kbase + (int64_t)key * kv_row_stride + c4 * 4);
        vw = *reinterpret_cast<const f32x4*>(vbase + (int64_t)key * kv_row_stride + c4 * 4);
      }
      *reinterpret_cast<f32x4*>(&sK[r * D + c4 * 4]) = kw;
      *reinterpret_cast<f32x4*>(&sV[r * D + c4 * 4]) = vw;
    }
    __syncthreads();

    float s[kTileKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kTileKeys; ++jj) {
      const float* kr = &sK[jj * D + part * kSlice];
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < kSlice; ++e) dot = fmaf(qv[e], kr[e], dot);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) dot += __shfl_xor(dot, off, 64);
      const int key = j0 + jj;
      const bool vis = key < Nk && (!CAUSAL || key <= row + offs);
      s[jj] = vis ? dot * c : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float mu = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - mu);        // 0 while nothing was visible
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < kSlice; ++e) acc[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kTileKeys; ++jj) {
      const float p = fast_exp2(s[jj] - mu);
      l_run += p;
      const float* vr = &sV[jj * D + part * kSlice];
#pragma unroll
      for (int e = 0; e < kSlice; ++e) acc[e] = fmaf(p, vr[e], acc[e]);
    }
    m_run = m_new;
  }

  if (row < N) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* dst = o + ((int64_t)b * N + row) * q_row_stride + (int64_t)h * D + part * kSlice;
#pragma unroll
    for (int e = 0; e < kSlice; e += 4) {
      f32x4 w = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
      *reinterpret_cast<f32x4*>(dst + e) = w;
    }
    if (part == 0)
      lse[((int64_t)b * Hq + h) * N + row] = l_run > 0.0f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a) {
  constexpr int ROWS = kThreads / (D / kSlice);
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
