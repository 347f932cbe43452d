// fa_kernels.h -- internal launch interface between the C ABI layer
// (fa_api.cpp) and the HIP kernels.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, Nk, d;   // N, Nk: the lengths, or (varlen) upper bounds of them
  bool causal;
  float scale;
  hipStream_t stream;
  // varlen (bf16 only): packed sequences given by device cu_seqlens; null for
  // the fixed-length [B, N, H, d] layout
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int total_q = 0;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu;
  void* o;
  float* lse;
  float* part_o;      // [(ranges + B) * Hq, d] fp32 partial outputs
  float* part_lse;    // [(ranges + B) * Hq] fp32 partial logsumexps
  int B, Hq, Hkv, d;
  int ranges;         // key ranges of the split (0: no keys to attend)
  float scale;
  hipStream_t stream;
  // paged cache (launch_decode_paged_bf16 only): k_cache/v_cache are
  // [num_blocks, 1 << bs_log2, Hkv, d]; sequence b has seqlens[b] cached rows,
  // row i in block block_table[b * max_blocks + (i >> bs_log2)]; when k_new is
  // set its rows [B, Hkv, d] (and v_new's) are appended first.  cu is then the
  // workspace array [B+1] that receives the prefix sums of 32-key tiles.
  const int32_t* block_table = nullptr;
  const int32_t* seqlens = nullptr;
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int32_t* cu_tiles = nullptr;
  int max_blocks = 0, bs_log2 = 0, num_blocks = 0;
};

// Backward (bf16): dq [B,N,Hq,d], dk/dv [B,Nk,Hkv,d] from q, k, v, o, dout and
// the forward's lse [B,Hq,N].  ld is the workspace [B*Hq][ceil(N/32)][64]
// fp32: per 32-row query tile, the rows' base-2 LSE then their D.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* ld;
  int B, Hq, Hkv, N, Nk, d;
  bool causal;
  float scale;
  hipStream_t stream;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);
hipError_t launch_prefill_f32(const PrefillArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);
hipError_t launch_decode_paged_bf16(const DecodeArgs& a);

int decode_max_group();       // largest Hq/Hkv the decode kernel handles

// Device address (valid on the current device) and size of the decode
// kernels' static scratch array; the address is looked up once per device.
hipError_t decode_scratch(void** ptr, size_t* bytes);
constexpr int kDecodeTile = 32;   // keys per decode tile (paged blocks hold whole tiles)

}  // namespace fa
