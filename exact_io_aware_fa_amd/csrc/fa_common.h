// fa_common.h -- device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// FA_DEBUG_SYNC builds (the library's race check) run every pipeline in
// order: each buffer->LDS copy is waited for as soon as it is issued, every
// workgroup barrier first waits for all of the wave's memory operations, and
// register-staged tiles get a barrier before they are stored.  The arithmetic
// is the same instruction for instruction, so a debug build's results must
// equal the fast build's bit for bit; a missing or short wait in the fast
// pipelines would show as a difference.
#ifdef FA_DEBUG_SYNC
constexpr bool kDebugSync = true;
#else
constexpr bool kDebugSync = false;
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// log2(e) and ln(2) as fp32 values; the kernels work in the base-2 exponent
// domain (p = 2^(s*scale*log2e - m)) and convert LSE back to natural log.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// MI355X dispatches workgroup b to XCD (b mod 8).  Grids are padded to a
// multiple of 8 and this maps the hardware id to a logical work index such
// that each XCD receives one contiguous range of logical work (and so keeps
// the K/V that range shares in its own L2).
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks_padded) {
  const int per_xcd = nblocks_padded >> 3;
  return (bid & 7) * per_xcd + (bid >> 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32;
// `lo` lands in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// acc + lo + hi of a packed bf16 pair (one v_dot2 against (1, 1)).  Callers
// pass scalar words: extracting the words from a vector first is avoided on
// purpose (the compiler folds such extracts feeding v_dot2 into word 0).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Eight fp32 -> bf16x8 MFMA operand; *sum += the eight rounded values.
__device__ __forceinline__ bf16x8 pack_bf16x8_sum(const float* f, float* sum) {
  const uint32_t w0 = pack_bf16x2(f[0], f[1]);
  const uint32_t w1 = pack_bf16x2(f[2], f[3]);
  const uint32_t w2 = pack_bf16x2(f[4], f[5]);
  const uint32_t w3 = pack_bf16x2(f[6], f[7]);
  *sum = add_bf16x2(w3, add_bf16x2(w2, add_bf16x2(w1, add_bf16x2(w0, *sum))));
  const u32x4 w = {w0, w1, w2, w3};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float wave_xor16(float x) { return __shfl_xor(x, 16, 64); }

// max(x[l], x[l ^ 32]) without touching LDS: v_permlane32_swap_b32 a, b swaps
// lanes 32..63 of a with lanes 0..31 of b, so with a = b = x, a and b hold the
// two halves of the wave in opposite order.  (__shfl_xor goes through
// ds_bpermute, an LDS instruction, and the compiler then waits for every
// outstanding buffer->LDS copy first.)  The nops keep the VALU write of the
// operands and the read of the results clear of the swap.
// The max is taken inside the same asm block: a compiler-issued max of an
// asm result would first quiet possible signalling NaNs (one more VALU op per
// operand), which the swap of plain scores never produces.
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return a;
}

// The same for lanes l and l ^ 16: v_permlane16_swap_b32 a, b swaps the odd
// 16-lane rows of a with the even rows of b.
__device__ __forceinline__ float max_xor16(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return a;
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// (and DMA writes of such lanes into LDS write 0), so tile loads need no
// per-lane bounds branches.  Only the per-lane (VGPR) offset is range
// checked; the scalar offset of an access is not, so an offset that may run
// past the end must go into the per-lane offset or into the base.  Word 3 is
// the gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from the buffer straight into LDS: lane l of the wave
// writes lds_wave_base + 16*l (lds_wave_base must be wave-uniform).
// The byte offset is voff (per lane, range checked) + soff (wave-uniform,
// an SGPR, not range checked).
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                     lds_void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voff, soff, 0, 0);
  if constexpr (kDebugSync) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// Wait until at most N of this wave's vector-memory operations (including
// buffer->LDS copies) are outstanding: s_waitcnt vmcnt(N), 0 <= N < 16.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  // gfx9 s_waitcnt: vmcnt is bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
  static_assert(N >= 0 && N < 64, "vmcnt field");
  constexpr int M = kDebugSync ? 0 : N;
  // the fence keeps the scheduler from hoisting the wait above register-only
  // work that precedes it (it would then wait for the copies too early)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(((M >> 4) << 14) | 0x0F70 | (M & 15));
}
__device__ __forceinline__ void wait_vmem_all() { wait_vmem_le<0>(); }

// Workgroup barrier without a memory fence.  __syncthreads() fences, which
// makes every wave wait for all of its outstanding buffer->LDS copies at every
// barrier; kernels that track their copies with wait_vmem_le use this one.
// The empty asm statements keep the compiler from moving memory accesses
// across it; LDS reads issued before it have been consumed (and so completed)
// before the wave reaches it, which the lgkmcnt wait makes explicit.
// The scheduling fences keep the instructions of a phase on their side of the
// barrier (without them register-only work is moved across it freely).
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kDebugSync ? 0x0070 : 0xC07F);   // lgkmcnt(0); vmcnt, expcnt left open (debug: vmcnt(0))
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane r receives element j
// (j = 0..3) from offset r%4 of the 8-byte row addressed by lane 4j + r/4.
// `p` must point into LDS (a __shared__ array).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

}  // namespace fa
