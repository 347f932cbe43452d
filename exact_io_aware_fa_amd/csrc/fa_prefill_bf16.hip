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
//    tile is 64 keys, shared by all 8 waves.  Wave w owns query rows
//    32w..32w+31.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K from LDS is the A operand, Q sits in
//    registers as the B operand for the whole kernel.  Lane (i, h) then holds
//    16 keys of query row i and lane i^32 the other 16.
//  * K rows are fed to the MFMA permuted (pi32) so that lane half h holds keys
//    h*16+0..15: the fp32 scores convert to bf16 in place and already form the
//    B operand of O^T += V^T P^T.  V stays row-major in LDS and its A operand
//    (8 consecutive keys of one head-dim column per lane) is read with
//    ds_read_b64_tr_b16.
//  * LDS rows are XOR-swizzled per 16-byte chunk; the swizzles were chosen by
//    measuring both read patterns on gfx950.  K and V tiles reach LDS by
//    buffer_load ... lds (no staging registers; rows past the end read 0).
//  * Ping-pong schedule.  Waves w and w+4 share a SIMD and belong to
//    different groups.  Per tile a wave runs an MFMA block (P.V of the
//    previous tile, then S of this tile) and a VALU block (softmax of this
//    tile).  Group 1 runs half a tile behind group 0, and workgroup barriers
//    separate the phases, so in every phase one wave of each SIMD issues MFMAs
//    while the other runs its softmax.
//  * Only group 0 moves data: after the last LDS read of its MFMA block it
//    issues the DMA of the next K tile and of the current V tile, and it
//    waits for them at the end of the following phase.  Its softmax has no
//    branches, and the rare rescale of O is applied at the start of the next
//    MFMA block, so nothing between the DMA and its wait makes the compiler
//    drain the copy early.
//  * Softmax in the base-2 domain: p = 2^(s*c - m), c = scale*log2(e).  The
//    reference max m moves only when a tile's max exceeds it by more than
//    kRescaleSlack (so p <= 2^kRescaleSlack); any consistent reference gives
//    the same O = sum p v / sum p.  Two row sums are kept: fp32 weights (for
//    LSE) and the bf16-rounded weights the MFMA multiplies (to normalise O,
//    so the rounding of P does not bias O).
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBR = 256;            // query rows per workgroup
constexpr int kBC = 64;             // keys per KV tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleSlack = 8.0f;
// K/V tiles are copied kPD tiles ahead of their use, through rings of kNS
// LDS stages per tensor (the copy of K_{j+kPD} and V_{j+kPD-1} is issued while
// tile j is computed).
#ifndef PREFILL_PD
#define PREFILL_PD 3
#endif
constexpr int kPD = PREFILL_PD;
constexpr int kNS = kPD + 1;

// Accumulator row R of a 32x32 MFMA lives in lane half (R>>2)&1, item
// (R>>3)*4 + (R&3).  Feeding K row pi32(R) as A-operand row R puts key h*16+r
// in item r of lane half h.
__device__ __forceinline__ int pi32(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// Chunk swizzles (XOR on the 16-byte chunk index within a row of CPR chunks),
// chosen by measuring the two read patterns on gfx950:
//  K (ds_read_b128 of rows pi32(m)): XOR with the row's low bits.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR > 16 ? 15 : CPR - 1); }
//  V (ds_read_b64_tr_b16: 4 consecutive rows, 32 bytes each per 16 lanes).
template <int CPR>
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << (CPR >= 16 ? 2 : 1); }

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
  constexpr int DMA_PER_WAVE = TILE_ELEMS * 2 / 1024 / (kWaves / 2);   // issued by group 0
  static_assert(DMA_PER_WAVE >= 1, "each issuing wave issues at least one DMA per tensor");

  // One LDS variable per stage: the compiler keeps apart the accesses it can
  // attribute to different variables, so a copy in flight into one stage does
  // not make it wait before reads of another (the stage loops below are
  // unrolled so that every stage is named statically).
  static_assert(kNS <= 4, "at most four stages per tensor");
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sK2[kNS > 2 ? TILE_ELEMS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sK3[kNS > 3 ? TILE_ELEMS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sV2[kNS > 2 ? TILE_ELEMS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sV3[kNS > 3 ? TILE_ELEMS : 8];

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
  // K/V: one view per tile (built in issue_k / issue_v), starting at the
  // tile's first row and ending at the slice's last row, so that rows past
  // Nk read as 0.  (The scalar offset of a buffer access is not range
  // checked, so the tile offset goes into the base, not into soffset.)
  const uint16_t* k_slice = k + ((int64_t)b * Nk * Hkv + g) * D;
  const uint16_t* v_slice = v + ((int64_t)b * Nk * Hkv + g) * D;
  const uint32_t kv_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * Hkv + 1) * D * 2 : 0u;

  // ---- Q tile -> registers (B operand of S^T = K Q^T); rows past N read 0
  bf16x8 qf[DSTEPS];
  {
    const uint32_t off = (uint32_t)(qbase + li) * q_row_bytes + hh * 16;
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) qf[t] = __builtin_bit_cast(bf16x8, buffer_load16(q_rsrc, off + t * 32));
  }

  // ---- KV tiles this workgroup needs, and where this wave's masked suffix starts
  int n_kv = (Nk + kBC - 1) / kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + kBR - 1, N - 1) + offs;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kBC + 1);
  }
  // tile j needs no mask for this wave iff j*64 + 63 < Nk and, when causal,
  // j*64 + 63 <= qbase + offs (the wave's first row sees the whole tile)
  int n_clean = Nk / kBC;
  if (CAUSAL) {
    const int d0 = qbase + offs - (kBC - 1);
    n_clean = min(n_clean, d0 < 0 ? 0 : d0 / kBC + 1);
  }
  n_clean = min(n_clean, n_kv);

  // ---- DMA of one K or V tile into LDS stage `st` by the 4 waves of group 0:
  // lane l of 1 KB instruction n fills row n*RPI + l/CPR, physical chunk
  // l%CPR.  The per-lane offsets are fixed for the whole kernel (the tile
  // offset is the scalar soffset), so their registers are never reused: the
  // compiler treats a DMA's address register as pending until the copy lands.
  const int dma_wave = wave % (kWaves / 2);
  uint32_t k_voff[DMA_PER_WAVE], v_voff[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int row = (dma_wave * DMA_PER_WAVE + i) * RPI + lane / CPR;
    const int pc = lane % CPR;
    k_voff[i] = (uint32_t)row * kv_row_bytes + (uint32_t)((pc ^ swz_k<CPR>(row)) * 16);
    v_voff[i] = (uint32_t)row * kv_row_bytes + (uint32_t)((pc ^ swz_v<CPR>(row)) * 16);
  }
  // Tile j begins j*kBC rows (tile_off bytes) into the slice.  Every call
  // issues the same number of copies: for a tile that does not exist (j >=
  // n_kv) the view is empty, so the copy writes zeros into a free stage and
  // reads nothing; the waits below count copies.
  auto tile_view = [&](const uint16_t* slice, const int j) {
    const bool real = j < n_kv;
    const uint32_t tile_off = real ? (uint32_t)(j * kBC) * kv_row_bytes : 0u;
    return make_rsrc(slice + (real ? (int64_t)j * kBC * Hkv * D : 0), real ? kv_bytes - tile_off : 0u);
  };
  auto issue = [&](const uint16_t* slice, const int j, const uint32_t* voff, char* stage) {
    const __amdgpu_buffer_rsrc_t r = tile_view(slice, j);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      buffer_load16_to_lds(r, voff[i], 0, (lds_void*)(stage + (dma_wave * DMA_PER_WAVE + i) * 1024));
  };
  // stage st of each ring (a constant st names one variable)
  auto kS = [&](const int st) -> char* {
    return reinterpret_cast<char*>(st == 0 ? sK0 : st == 1 ? sK1 : st == 2 ? sK2 : sK3);
  };
  auto vS = [&](const int st) -> char* {
    return reinterpret_cast<char*>(st == 0 ? sV0 : st == 1 ? sV1 : st == 2 ? sV2 : sV3);
  };

  // ---- lane-constant LDS offsets (bytes) for the MFMA operand reads
  // K (A operand of S^T): row kb*32 + pi32(li), logical chunk 2t + hh; the
  // swizzle depends only on the row's low bits, so it is the same for kb = 0, 1.
  const int krow = pi32(li);
  int k_off[DSTEPS];
#pragma unroll
  for (int t = 0; t < DSTEPS; ++t) k_off[t] = krow * (2 * D) + (((2 * t + hh) ^ swz_k<CPR>(krow)) * 16);
  // V (A operand of O^T, transpose read): 16-lane group (mh, h) of the wave,
  // lane r points at key h*16 + r/4 (+ kb*32 + u*8 + 4*rho) and head-dim
  // 32*d + 16*mh + 4*(r%4).
  const int r16 = lane & 15;
  const int mh = (lane >> 4) & 1;
  const int vrow = hh * 16 + (r16 >> 2);
  int v_off[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d) {
    const int chunk = 4 * d + 2 * mh + ((r16 & 3) >> 1);
    v_off[d] = vrow * (2 * D) + ((chunk ^ swz_v<CPR>(vrow)) * 16) + (r16 & 1) * 8;
  }

  // ---- state
  f32x16 acc_o[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[d][r] = 0.0f;
  float m_ref = -INFINITY;   // running reference max (base-2 domain), same in both lanes of a row
  float l_part = 0.0f;       // sum of fp32 weights over this lane's keys
  float l_rnd = 0.0f;        // sum of the bf16-rounded weights over this lane's keys
  float alpha = 1.0f;        // pending rescale of acc_o (applied before the next P.V)
  bool rescale = false;      // wave-uniform: some row of the wave has alpha != 1
  f32x16 s[2];               // scores of the current tile (two 32-key blocks)
  bf16x8 pf[2][2];           // weights of the current tile, B operands of P.V

  // S^T = K Q^T for the K tile at `kst`
  auto stage_s = [&](const char* kst) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, load16(kst + kb * 32 * (2 * D) + k_off[t]));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
        // keep at most a few operand reads in flight (bounds register use)
        if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // O^T = alpha*O^T + V^T P^T for the V tile at `vst`
  auto stage_pv = [&](const char* vst) {
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[d][r] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
          const char* base = vst + (kb * 32 + u * 8) * (2 * D) + v_off[d];
          const u32x2 lo = lds_read_tr16(base);
          const u32x2 hi = lds_read_tr16(base + 4 * (2 * D));
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          acc_o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][u], acc_o[d], 0, 0, 0);
          if ((d & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
  };

  // online softmax of the tile of keys j0..j0+63 -> pf.  `masked`
  // (wave-uniform): some key of the tile is invisible to some row of this wave.
  auto stage_softmax = [&](const int j0, const bool masked) {
    if (__builtin_expect(masked, 0)) {
      // last visible key of this lane's row; item r of block kb holds key
      // j0 + kb*32 + hh*16 + r
      const int lim = CAUSAL ? min(Nk - 1, qbase + li + offs) : Nk - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int thr = lim - (j0 + kb * 32 + hh * 16);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = r <= thr ? s[kb][r] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_xor32(mx);                        // the row's other 32 keys sit in lane^32
    const float mt = mx * c;
    const bool need = mt > m_ref + kRescaleSlack;
    const float m_new = need ? mt : m_ref;
    alpha = need ? fast_exp2(m_ref - m_new) : 1.0f;   // 0 when m_ref was -inf
    rescale = __builtin_amdgcn_ballot_w64(need) != 0;
    m_ref = m_new;
    l_part *= alpha;
    l_rnd *= alpha;
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
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
  };

  // The MFMA block of tile j: P.V of tile j-1, S of tile j, and (group 0)
  // the copies of K_{j+kPD} and V_{j+kPD-1}.  The read and copy stages are
  // distinct; passing them as restrict pointers of one inlined call lets the
  // compiler see that, so it does not wait for the copies in flight before
  // the reads (the waits that order copies and reads are the explicit ones
  // below, before the workgroup barriers).
  auto mblock = [&](const int j, const char* __restrict__ kread, const char* __restrict__ vread,
                    char* __restrict__ kdst, char* __restrict__ vdst, auto copy_tag) __attribute__((always_inline)) {
    if (j >= 1) stage_pv(vread);
    stage_s(kread);
    if (decltype(copy_tag)::value) {
      issue(k_slice, j + kPD, k_voff, kdst);
      issue(v_slice, j + kPD - 1, v_voff, vdst);
    }
  };
  const auto kCopy = std::integral_constant<bool, true>();
  const auto kNoCopy = std::integral_constant<bool, false>();
  constexpr int kCopiesPerBlock = 2 * DMA_PER_WAVE;

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
  // Rounds of kNS tiles, unrolled so that every stage is named statically.
  // The check after each tile leaves the loop (it never skips ahead to the
  // next round), so at the top of a round, as far as the compiler can tell,
  // the same copies are in flight as at the end of the previous one.
  auto run_group = [&](auto copy_tag) __attribute__((always_inline)) {
    constexpr bool COPY = decltype(copy_tag)::value;
    auto step = [&](const int j, const int st) __attribute__((always_inline)) {   // j % kNS == st
      mblock(j, kS(st), vS((st + kNS - 1) % kNS), kS((st + kPD) % kNS), vS((st + kPD - 1) % kNS),
             copy_tag);                               // phase 2j+g
      barrier_no_fence();
      stage_softmax(j * kBC, j >= n_clean);           // phase 2j+1+g
      if (COPY) wait_vmem_le<(kPD - 1) * kCopiesPerBlock>();
      barrier_no_fence();
    };
    // one round from tile j0 (< n_kv); false once the last tile is done
    auto round = [&](const int j0) __attribute__((always_inline)) -> bool {
      step(j0, 0);
      if (j0 + 1 >= n_kv) return false;
      step(j0 + 1, 1);
      if (j0 + 2 >= n_kv) return false;
      if constexpr (kNS > 2) {
        step(j0 + 2, 2);
        if (j0 + 3 >= n_kv) return false;
      }
      if constexpr (kNS > 3) {
        step(j0 + 3, 3);
        if (j0 + 4 >= n_kv) return false;
      }
      return true;
    };
    for (int j0 = 0; round(j0); j0 += kNS) {
    }
  };
  if (n_kv > 0) {
    if (group == 0) {
#pragma unroll
      for (int t = 0; t < kPD; ++t) issue(k_slice, t, k_voff, kS(t));
#pragma unroll
      for (int t = 0; t < kPD - 1; ++t) issue(v_slice, t, v_voff, vS(t));
    }
    // both groups: the Q registers (and group 0's first copies) have landed.
    // (Waiting in one group only would leave the loads pending, as far as the
    // compiler can tell, where the groups' paths join, and it would then wait
    // for them, and for every copy issued after them, inside the loops.)
    wait_vmem_all();
    barrier_no_fence();
    if (group == 0) {
      run_group(kCopy);
      wait_vmem_all();                              // no copy may land after the workgroup ends
      stage_pv(vS((n_kv - 1) % kNS));               // phase 2n: M_n
      barrier_no_fence();
      barrier_no_fence();                           // phase 2n+1: idle
    } else {
      barrier_no_fence();                           // phase 0: idle
      run_group(kNoCopy);
      stage_pv(vS((n_kv - 1) % kNS));               // phase 2n+1: M_n
      barrier_no_fence();
    }
  }

  // ---- epilogue: O = acc / l_rnd, LSE = (m + log2 l) * ln 2
  // lane (i, hh) item r holds head-dim 32*d + 8*(r/4) + 4*hh + r%4
  // (the last tile's rescale was applied by the final P.V block)
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
