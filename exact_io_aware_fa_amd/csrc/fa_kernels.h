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
  int B, Hq, Hkv, N, Nk, d;
  bool causal;
  float scale;
  hipStream_t stream;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu;
  void* o;
  float* lse;
  float* part_o;      // [B, Hq, max_splits, d] fp32
  float* part_lse;    // [B, Hq, max_splits] fp32
  int B, Hq, Hkv, d;
  int max_splits, chunk;
  float scale;
  hipStream_t stream;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a);
hipError_t launch_prefill_f32(const PrefillArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);

int decode_max_group();       // largest Hq/Hkv the decode kernel handles
int decode_chunk_granule();   // split sizes are multiples of this many keys

}  // namespace fa
