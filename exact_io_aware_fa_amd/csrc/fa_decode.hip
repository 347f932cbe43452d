// fa_decode.hip -- split-KV decode attention over a packed, variable-length
// KV cache, bf16 in/out, fp32 accumulation, for gfx950.
//
// One new query token per sequence attends to every row of that sequence's
// cache; only the real cache length is read (ai6s.net page, section "what
// ops-transformer adds", third item).  Work is split along the cache: each
// workgroup reduces one chunk of one (sequence, kv head) with the online
// softmax (ai6s.net page, section "FlashAttention changes the dataflow, not
// the algorithm") and writes a partial output normalised by its own row sum
// plus that chunk's logsumexp.  A second kernel merges the partials of a
// sequence with weights exp(LSE_s - LSE), LSE = log sum_s exp(LSE_s), which is
// the same rescaling the online softmax applies tile by tile.
//
// gfx950 mapping (split kernel)
//  * workgroup = 4 waves; wave w streams 64-key sub-tiles w, w+4, ... of the
//    chunk.  All query heads of one kv group (G = Hq/Hkv <= 16) share each K/V
//    byte, so K and V are read from HBM exactly once.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K is loaded from HBM straight
//    into A-operand registers (16-byte loads), Q^T (G heads padded to 16
//    columns) is the B operand.  The K rows fed to each MFMA are permuted so
//    that every lane ends up holding 8 consecutive keys of one query head,
//    which is exactly its B-operand slice of the following P.V MFMA.
//  * V is transposed through a per-wave LDS tile (4x8 register transpose,
//    8-byte writes) and read back as 16-byte V^T A-operand slices.
//  * The four waves' (max, sum, output) are merged through LDS at the end.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kSub = 64;            // keys per wave sub-tile
constexpr int kGMax = 16;           // query heads per kv head handled by one MFMA column block
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ int swz_d(int row) { return (row & 7) ^ ((row >> 3) & 7); }

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cu, float* __restrict__ part_o, float* __restrict__ part_lse, int Hq,
    int Hkv, int max_splits, int chunk, float c) {
  constexpr int DT = D / 32;          // MFMA k-steps of S^T
  constexpr int DB = D / 16;          // 16-wide head-dim blocks of O^T
  constexpr int KCH = D / 8;          // 16-byte chunks per row
  constexpr int VIT = kSub * KCH / 4 / 64;   // 4-key x 8-dim blocks per lane
  __shared__ __attribute__((aligned(16))) uint16_t sVt[kWaves][D * kSub];
  __shared__ float s_m[kWaves][kGMax], s_l[kWaves][kGMax], s_lr[kWaves][kGMax];

  const int split = blockIdx.x % max_splits;
  const int rest = blockIdx.x / max_splits;
  const int g = rest % Hkv;
  const int b = rest / Hkv;
  const int start = cu[b];
  const int L = cu[b + 1] - start;
  const int ks = split * chunk;
  if (ks >= L) return;                                 // past this sequence's cache
  const int ke = min(L, ks + chunk);
  const int G = Hq / Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int grp = lane >> 4;                           // 0..3
  const int64_t row_stride = (int64_t)Hkv * D;
  const uint16_t* kbase = kc + ((int64_t)start * Hkv + g) * D;
  const uint16_t* vbase = vc + ((int64_t)start * Hkv + g) * D;

  // Q^T as B operand: column n = query head g*G + n (zero for n >= G)
  bf16x8 qf[DT];
  {
    const bool valid = l16 < G;
    const uint16_t* src = q + ((int64_t)b * Hq + g * G + (valid ? l16 : 0)) * D + grp * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid) w = load16(src + t * 32);
      qf[t] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x4 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.0f;   // l_part: fp32 weights, for LSE
  float l_rnd = 0.0f;                        // bf16-rounded weights, for O
  uint16_t* myV = sVt[wave];

  for (int k0 = ks + wave * kSub; k0 < ke; k0 += kWaves * kSub) {
    // K rows as A operand: block e2 = 2p+e, row R -> key 32p + (R/4)*8 + e*4 + R%4
    u32x4 kf[4][DT];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int p = blk >> 1, e = blk & 1;
      const int key = k0 + 32 * p + (l16 >> 2) * 8 + e * 4 + (l16 & 3);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < ke) w = load16(kbase + (int64_t)key * row_stride + t * 32 + grp * 8);
        kf[blk][t] = w;
      }
    }
    // V rows, 4-key x 8-dim blocks
    u32x4 vr[VIT][4];
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int blkid = it * 64 + lane;
      const int dc = blkid % KCH, kq = blkid / KCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + kq * 4 + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < ke) w = load16(vbase + (int64_t)key * row_stride + dc * 8);
        vr[it][r] = w;
      }
    }

    // S^T blocks: lane (n, grp) item r of block 2p+e = key 32p + grp*8 + e*4 + r
    f32x4 s[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DT; ++t)
        s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[blk][t]), qf[t], s[blk], 0, 0, 0);
    }

    // V^T into this wave's LDS tile
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int blkid = it * 64 + lane;
      const int dc = blkid % KCH, kq = blkid / KCH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        u32x2 out;
        if ((e & 1) == 0) {
          out[0] = (vr[it][0][w] & 0xffffu) | (vr[it][1][w] << 16);
          out[1] = (vr[it][2][w] & 0xffffu) | (vr[it][3][w] << 16);
        } else {
          out[0] = (vr[it][0][w] >> 16) | (vr[it][1][w] & 0xffff0000u);
          out[1] = (vr[it][2][w] >> 16) | (vr[it][3][w] & 0xffff0000u);
        }
        const int row = dc * 8 + e;
        *reinterpret_cast<u32x2*>(&myV[row * kSub + (((kq >> 1) ^ swz_d(row)) * 8) + (kq & 1) * 4]) = out;
      }
    }

    // online softmax for query head l16 over this sub-tile's keys
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int p = blk >> 1, e = blk & 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 32 * p + grp * 8 + e * 4 + r;
        s[blk][r] = key < ke ? s[blk][r] : -INFINITY;
        mx = fmaxf(mx, s[blk][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mt = mx * c;
    const bool need = mt > m_ref + kRescaleSlack;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = need ? fast_exp2(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      l_part *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d) acc[d] *= alpha;
    }
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
    float pv[4][4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[blk][r] = fast_exp2(fmaf(s[blk][r], c, -mu));
        l_part += pv[blk][r];
      }
    bf16x8 pf[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float f8[8] = {pv[2 * p][0],     pv[2 * p][1],     pv[2 * p][2],     pv[2 * p][3],
                           pv[2 * p + 1][0], pv[2 * p + 1][1], pv[2 * p + 1][2], pv[2 * p + 1][3]};
      pf[p] = pack_bf16x8_sum(f8, &l_rnd);
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // O^T += V^T P^T: lane (dd row l16, grp) slot s = key 32p + grp*8 + s
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const int row = d * 16 + l16;
        const bf16x8 a = __builtin_bit_cast(bf16x8, load16(&myV[row * kSub + (((4 * p + grp) ^ swz_d(row)) * 8)]));
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[p], acc[d], 0, 0, 0);
      }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves: sum over lane groups, then across waves in LDS
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
  l_rnd += __shfl_xor(l_rnd, 16, 64);
  l_rnd += __shfl_xor(l_rnd, 32, 64);
  __syncthreads();                                     // V^T tiles are free again
  float* s_o = reinterpret_cast<float*>(&sVt[0][0]);   // [kWaves][kGMax][D] fp32 (fits: 4*16*128*4 = 32 KB)
  if (grp == 0) {
    s_m[wave][l16] = m_ref;
    s_l[wave][l16] = l_part;
    s_lr[wave][l16] = l_rnd;
  }
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[(wave * kGMax + l16) * D + d * 16 + grp * 4 + r] = acc[d][r];
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int n = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][n]);
    float Lsum = 0.0f, Lrnd = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = s_m[w][n] == -INFINITY ? 0.0f : fast_exp2(s_m[w][n] - M);
      Lsum += s_l[w][n] * sc;
      Lrnd += s_lr[w][n] * sc;
      O += s_o[(w * kGMax + n) * D + dd] * sc;
    }
    const int h = g * G + n;
    const int64_t slot = ((int64_t)b * Hq + h) * max_splits + split;
    part_o[slot * D + dd] = O / Lrnd;
    if (dd == 0) part_lse[slot] = (M + fast_log2(Lsum)) * kLn2;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           const int32_t* __restrict__ cu,
                                                           uint16_t* __restrict__ o, float* __restrict__ lse,
                                                           int Hq, int max_splits, int chunk) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int L = cu[b + 1] - cu[b];
  const int ns = min((L + chunk - 1) / chunk, max_splits);   // lengths above the bound are a caller error
  const int dd = threadIdx.x;
  const float* pl = part_lse + (int64_t)bh * max_splits;
  const float* po = part_o + (int64_t)bh * max_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pl[s]);
  float wsum = 0.0f, acc = 0.0f;
  if (ns > 0) {
    for (int s = 0; s < ns; ++s) {
      const float w = fast_exp2((pl[s] - M) * kLog2e);
      wsum += w;
      acc = fmaf(w, po[(int64_t)s * D + dd], acc);
    }
  }
  const float out = ns > 0 ? acc / wsum : 0.0f;
  o[(int64_t)bh * D + dd] = __builtin_bit_cast(uint16_t, (__bf16)out);
  if (dd == 0) lse[bh] = ns > 0 ? M + fast_log2(wsum) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch(const DecodeArgs& a) {
  const int64_t nblk = (int64_t)a.B * a.Hkv * a.max_splits;
  if (nblk > 0) {
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)nblk), dim3(kThreads), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.cu,
                       a.part_o, a.part_lse, a.Hq, a.Hkv, a.max_splits, a.chunk, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(D), 0, a.stream,
                     a.part_o, a.part_lse, a.cu, (uint16_t*)a.o, a.lse, a.Hq, a.max_splits, a.chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a) { return a.d == 64 ? launch<64>(a) : launch<128>(a); }

int decode_max_group() { return kGMax; }
int decode_chunk_granule() { return kWaves * kSub; }

}  // namespace fa
