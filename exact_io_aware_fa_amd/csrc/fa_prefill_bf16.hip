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
//  * workgroup = 8 waves = 256 query rows of one (batch, query head); a KV
//    tile is 64 keys and is shared by all 8 waves.  Wave w owns query rows
//    32w..32w+31.  With ~170 registers per wave two waves share each SIMD, so
//    one wave's softmax (VALU) runs while the other's MFMAs issue.
//  * K and V tiles go from HBM straight into LDS with buffer_load ... lds
//    (no staging registers); rows past the end of the sequence read as zero.
//    Tile j+1 is in flight while tile j is computed (two LDS stages, one
//    barrier per tile).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K from LDS is the A operand, Q sits in
//    registers as the B operand for the whole kernel.  Lane (i, h) then holds
//    16 keys of query row i and lane i^32 the other 16, so the row max is an
//    in-lane reduction plus one exchange with lane^32, and the row sum is
//    kept per lane and exchanged once at the end.
//  * K rows are fed to the MFMA permuted (pi32) so that lane half h holds keys
//    h*16+0..15: the fp32 scores convert to bf16 in place and already form the
//    B operand of O^T += V^T P^T.
//  * V stays row-major in LDS; its A operand (8 consecutive keys of one
//    head-dim column per lane) is read with ds_read_b64_tr_b16.
//  * LDS rows are XOR-swizzled per 16-byte chunk so that the MFMA operand
//    reads are free of bank conflicts; the DMA writes realise the swizzle by
//    choosing which global chunk each lane fetches.
//  * Two row sums are kept: the fp32 sum of the weights (for LSE) and the sum
//    of the bf16-rounded weights the P.V MFMA actually multiplies (for the
//    normalisation of O), so O is an exact convex combination of the rounded
//    weights and the rounding of P does not bias it.
//  * The softmax runs in the base-2 domain: p = 2^(s*c - m), c = scale*log2(e).
//    The reference max m only moves when a tile's max exceeds it by more than
//    kRescaleSlack (so p <= 2^kRescaleSlack); any consistent reference gives
//    the same O = sum p v / sum p.  The rescale of O is skipped for the whole
//    wave when no row needs it.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBR = 256;            // query rows per workgroup
constexpr int kBC = 64;             // keys per KV tile
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr float kRescaleSlack = 8.0f;

// Accumulator row R of a 32x32 MFMA lives in lane half (R>>2)&1, item
// (R>>3)*4 + (R&3).  Feeding K row pi32(R) as A-operand row R puts key h*16+r
// in item r of lane half h.
__device__ __forceinline__ int pi32(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// Chunk swizzles (XOR on the 16-byte chunk index within a row).
//  K: the eight rows one ds_read_b128 phase touches differ in row bits 0,1,4.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 2) & 4); }
//  V: a 16-lane transpose read touches 4 consecutive rows, 32 bytes each.
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int N, int Nk, int Hq, int Hkv, float c,
    int n_qtiles, int n_work) {
  constexpr int DSTEPS = D / 16;            // MFMA k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;              // 32-wide blocks of the head dim
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPI = 1024 / (2 * D);       // rows per 1 KB wave DMA instruction
  constexpr int TILE_ELEMS = kBC * D;
  constexpr int DMA_PER_WAVE = TILE_ELEMS * 2 / 1024 / kWaves;
  static_assert(DMA_PER_WAVE >= 1, "each wave issues at least one DMA per tensor");

  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][TILE_ELEMS];

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
  const int qt = CAUSAL ? (n_qtiles - 1 - qrank) : qrank;   // heaviest causal tiles first
  const int h = g * G + hig;
  const int q0 = qt * kBR;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int qbase = q0 + 32 * wave;
  const int offs = Nk - N;                                      // bottom-right causal offset

  // ---- buffer views: one (batch, head) slice each; reads past the end are 0
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc =
      make_rsrc(q + ((int64_t)b * N * Hq + h) * D, (uint32_t)((N - 1) * Hq + 1) * D * 2);
  const uint32_t kv_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * Hkv + 1) * D * 2 : 0u;
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(k + ((int64_t)b * Nk * Hkv + g) * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(v + ((int64_t)b * Nk * Hkv + g) * D, kv_bytes);

  // ---- Q tile -> registers (B operand of S^T = K Q^T); rows past N read 0
  bf16x8 qf[DSTEPS];
  {
    const uint32_t off = (uint32_t)(qbase + li) * q_row_bytes + hh * 16;
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) qf[t] = __builtin_bit_cast(bf16x8, buffer_load16(q_rsrc, off + t * 32));
  }

  // ---- number of KV tiles this workgroup needs
  int n_kv = (Nk + kBC - 1) / kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + kBR - 1, N - 1) + offs;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kBC + 1);
  }

  // ---- DMA of one K/V tile into LDS stage `st`: each wave issues
  // DMA_PER_WAVE 1 KB instructions per tensor; lane l of instruction n fills
  // row n*RPI + l/CPR, physical chunk l%CPR.
  const int dma_row_in = lane / CPR;
  const int dma_pc = lane % CPR;
  auto issue_tile = [&](int j, int st) {
    const int j0 = j * kBC;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int n = wave * DMA_PER_WAVE + i;
      const int row = n * RPI + dma_row_in;
      const uint32_t key_off = (uint32_t)(j0 + row) * kv_row_bytes;
      buffer_load16_to_lds(k_rsrc, key_off + (uint32_t)((dma_pc ^ swz_k(row)) * 16), (lds_void*)&sK[st][n * 512]);
      buffer_load16_to_lds(v_rsrc, key_off + (uint32_t)((dma_pc ^ swz_v(row)) * 16), (lds_void*)&sV[st][n * 512]);
    }
  };

  // ---- lane-constant LDS offsets (bytes) for the MFMA operand reads
  // K (A operand of S^T): row kb*32 + pi32(li), chunk 2t + hh swizzled; for
  // t = 4*t1 + t0 the swizzled chunk is 8*t1 + ((2*t0 + hh) ^ swz_k(row)).
  const int krow = pi32(li);
  int k_off[4];
#pragma unroll
  for (int t0 = 0; t0 < 4; ++t0) k_off[t0] = krow * (2 * D) + (((2 * t0 + hh) ^ swz_k(krow)) * 16);
  // V (A operand of O^T, transpose read): 16-lane group (mh, h) of the wave,
  // lane r points at key  h*16 + r/4 (+ kb*32 + u*8 + 4*rho)  and head-dim
  // 16*mh + 4*(r%4) (+ 32*ddb).
  const int r16 = lane & 15;
  const int mh = (lane >> 4) & 1;
  const int vrow = hh * 16 + (r16 >> 2);
  int v_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int chunk = 4 * par + 2 * mh + ((r16 & 3) >> 1);
    v_off[par] = vrow * (2 * D) + ((chunk ^ swz_v(vrow)) * 16) + (r16 & 1) * 8;
  }

  // ---- accumulators
  f32x16 acc_o[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[d][r] = 0.0f;
  float m_ref = -INFINITY;
  float l_part = 0.0f;     // sum of fp32 weights (this lane's keys)
  float l_rnd = 0.0f;      // sum of bf16-rounded weights

  if (n_kv > 0) issue_tile(0, 0);

  // One KV tile.  MASKED = the tile holds keys that some row of this wave
  // must not see (causal diagonal or keys past Nk): every score then goes
  // through the visibility select.  Otherwise the body is straight-line.
  auto tile_step = [&](const int st, const int j0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;

    // ---- S^T = K Q^T
    const char* kst = reinterpret_cast<const char*>(&sK[st][0]);
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, load16(kst + kb * 32 * (2 * D) + (t >> 2) * 128 + k_off[t & 3]));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
        // keep at most a few operand reads in flight (bounds register use)
        if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- online softmax (per lane: one query row, 32 of the tile's 64 keys)
    if (MASKED) {
      const int qi = qbase + li;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + hh * 16 + r;
          const bool vis = key < Nk && (!CAUSAL || key <= qi + offs);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float mt = mx * c;
    const bool need = mt > m_ref + kRescaleSlack;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = need ? fast_exp2(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      l_part *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[d][r] *= alpha;
    }
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(s[kb][r], c, -mu));
        l_part += p[r];
      }
      pf[kb][0] = pack_bf16x8_sum(&p[0], &l_rnd);
      pf[kb][1] = pack_bf16x8_sum(&p[8], &l_rnd);
    }

    // ---- O^T += V^T P^T
    const char* vst = reinterpret_cast<const char*>(&sV[st][0]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
          const char* base = vst + (kb * 32 + u * 8) * (2 * D) + (d >> 1) * 128 + v_off[d & 1];
          const u32x2 lo = lds_read_tr16(base);
          const u32x2 hi = lds_read_tr16(base + 4 * (2 * D));
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][u], acc_o[d], 0, 0, 0);
          if ((d & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
  };

  // keys j0..j0+63 are all visible to every row of this wave iff the tile
  // ends before Nk and (causal) before the first row's diagonal
  for (int j = 0; j < n_kv; ++j) {
    const int st = j & 1;
    const int j0 = j * kBC;
    wait_vmem_all();
    __syncthreads();                                  // tile j is in LDS; stage st^1 is free
    if (j + 1 < n_kv) issue_tile(j + 1, st ^ 1);
    const bool clean = j0 + kBC <= Nk && (!CAUSAL || j0 + kBC - 1 <= qbase + offs);
    if (clean)
      tile_step(st, j0, std::integral_constant<bool, false>());
    else
      tile_step(st, j0, std::integral_constant<bool, true>());
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
  // lane (i, hh) item r holds head-dim 32*d + 8*(r/4) + 4*hh + r%4
  {
    const float lt = l_part + wave_xor32(l_part);
    const float lr = l_rnd + wave_xor32(l_rnd);
    const int row = qbase + li;
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    if (row < N) {
      uint16_t* dst = o + ((int64_t)b * N + row) * ((int64_t)Hq * D) + (int64_t)h * D + hh * 4;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) {
        const f32x16 a = acc_o[d];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 w;
          w[0] = pack_bf16x2(a[4 * q4] * inv, a[4 * q4 + 1] * inv);
          w[1] = pack_bf16x2(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + d * 32 + q4 * 8) = w;
        }
      }
      if (hh == 0)
        lse[((int64_t)b * Hq + h) * N + row] = lt > 0.0f ? (m_ref + fast_log2(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a) {
  const int n_qtiles = (a.N + kBR - 1) / kBR;
  const int64_t n_work = (int64_t)a.B * a.Hq * n_qtiles;
  if (n_work == 0) return hipSuccess;
  const int64_t grid = (n_work + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, a.N, a.Nk, a.Hq, a.Hkv, a.scale * kLog2e, n_qtiles, (int)n_work);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
