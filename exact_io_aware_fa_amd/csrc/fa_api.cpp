// fa_api.cpp -- the C ABI of libfa.so (declared in include/fa.h): argument
// validation, split planning for decode, and dispatch to the HIP kernels.
// Nothing here touches the device before every argument has been checked.
#include "fa.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fa_kernels.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512];

fa_status_t fail(fa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

fa_status_t ok() {
  g_last_error[0] = '\0';
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p+bytes) overlaps [r, r+rbytes)?
bool overlaps(const void* p, size_t bytes, const void* r, size_t rbytes) {
  if (!p || !r || bytes == 0 || rbytes == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), c = reinterpret_cast<uintptr_t>(r);
  return a < c + rbytes && c < a + bytes;
}

// Decode work plan: the cache's (sequence, key) units are shared evenly by
// `ranges` key ranges; the split kernel runs one workgroup per (key range,
// group of kv heads), one wave per kv head, so the waves of a workgroup read
// whole cache rows together.  In total one round of resident waves (2 per
// SIMD on the 256 CUs of an MI355X is 2048): every wave then streams for the
// whole launch, with no second round starting behind a first (measured on the
// varlen decode workload: 1 round 0.353 ms, 2 rounds 0.361 ms, 1.5 rounds
// 0.377 ms).  Fewer ranges when the caches are short, so that a range gets at
// least kMinKeysPerRange keys.
#ifndef FA_DECODE_WAVES
#define FA_DECODE_WAVES 2048
#endif
constexpr int64_t kDecodeWaves = FA_DECODE_WAVES;
constexpr int64_t kMinKeysPerRange = 256;

int plan_ranges(int B, int Hkv, int max_seqlen_k) {
  if (B <= 0 || Hkv <= 0 || max_seqlen_k <= 0) return 0;
  const int64_t units = (int64_t)B * max_seqlen_k;
  const int64_t r = (units + kMinKeysPerRange - 1) / kMinKeysPerRange;
  return (int)std::min(std::max<int64_t>(1, kDecodeWaves / Hkv), std::max<int64_t>(1, r));
}

struct DecodeLayout {
  int ranges;
  int64_t rows;           // partial-result rows: (ranges + B) * Hq
  size_t lse_offset;      // byte offset of part_lse in the workspace
  size_t bytes;
};

DecodeLayout decode_layout(int B, int Hq, int Hkv, int d, int max_seqlen_k) {
  DecodeLayout l{plan_ranges(B, Hkv, max_seqlen_k), 0, 0, 0};
  if (l.ranges == 0) return l;
  l.rows = ((int64_t)l.ranges + B) * Hq;
  l.lse_offset = ((size_t)l.rows * d * sizeof(float) + 255) / 256 * 256;
  l.bytes = l.lse_offset + (size_t)l.rows * sizeof(float);
  return l;
}

}  // namespace

FA_EXPORT int fa_abi_version(void) { return FA_ABI_VERSION; }

FA_EXPORT const char* fa_status_str(fa_status_t status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

FA_EXPORT const char* fa_last_error(void) { return g_last_error; }

FA_EXPORT fa_status_t fa_fwd(fa_dtype_t dtype, const void* q, const void* k, const void* v, void* o,
                             float* lse, int B, int Hq, int Hkv, int N, int Nk, int d, int causal,
                             float scale, void* stream) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || N < 0 || Nk < 0) return fail(FA_ERR_INVALID_ARG, "negative size (B=%d N=%d Nk=%d)", B, N, Nk);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d <= 0) return fail(FA_ERR_INVALID_ARG, "head dim d=%d", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive (got %g)", (double)scale);
  if (B == 0 || N == 0) return ok();
  // the kernels index rows and work items with 32-bit integers
  if ((int64_t)B * N > INT32_MAX || (int64_t)B * Nk > INT32_MAX ||
      (int64_t)B * Hq * ((N + 63) / 64) > INT32_MAX - 8)
    return fail(FA_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
  // tiles address one (batch, head) slice through 32-bit buffer offsets,
  // including up to one tile of rows past the end
  const int64_t es64 = dtype == FA_BF16 ? 2 : 4;
  if (((int64_t)N + 256) * Hq * d * es64 >= INT32_MAX || ((int64_t)Nk + 256) * Hkv * d * es64 >= INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "one batch of q or k/v exceeds 2 GiB");
  if (!q || !o || !lse) return fail(FA_ERR_INVALID_ARG, "null q, o or lse pointer");
  if (Nk > 0 && (!k || !v)) return fail(FA_ERR_INVALID_ARG, "null k or v pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t es = dtype == FA_BF16 ? 2 : 4;
  const size_t q_bytes = (size_t)B * N * Hq * d * es;
  const size_t kv_bytes = (size_t)B * Nk * Hkv * d * es;
  const size_t lse_bytes = (size_t)B * Hq * N * sizeof(float);
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) || overlaps(o, q_bytes, v, kv_bytes) ||
      overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
      overlaps(lse, lse_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, o, q_bytes))
    return fail(FA_ERR_INVALID_ARG, "outputs alias inputs or each other");

  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, N, Nk, d, causal != 0, scale,
                    reinterpret_cast<hipStream_t>(stream)};
  const hipError_t e = dtype == FA_BF16 ? fa::launch_prefill_bf16(a) : fa::launch_prefill_f32(a);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

FA_EXPORT fa_status_t fa_fwd_varlen(fa_dtype_t dtype, const void* q, const void* k, const void* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int max_seqlen_q,
                                    int max_seqlen_k, int total_q, int total_k, void* o, float* lse, int B, int Hq,
                                    int Hkv, int d, int causal, float scale, void* stream) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d max_seqlen_q=%d max_seqlen_k=%d total_q=%d total_k=%d)", B,
                max_seqlen_q, max_seqlen_k, total_q, total_k);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d <= 0) return fail(FA_ERR_INVALID_ARG, "head dim d=%d", d);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive (got %g)", (double)scale);
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "varlen prefill supports bf16 only");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (B == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  // work items and per-sequence buffer views use 32-bit integers
  if ((int64_t)B * Hq * ((max_seqlen_q + 63) / 64) > INT32_MAX - 8)
    return fail(FA_ERR_UNSUPPORTED, "problem too large for 32-bit work indexing");
  if (((int64_t)max_seqlen_q + 256) * Hq * d * 2 >= INT32_MAX ||
      ((int64_t)max_seqlen_k + 256) * Hkv * d * 2 >= INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "one sequence of q or k/v exceeds 2 GiB");
  if (!q || !o || !lse || !cu_seqlens_q || !cu_seqlens_k)
    return fail(FA_ERR_INVALID_ARG, "null q, o, lse or cu_seqlens pointer");
  if (total_k > 0 && (!k || !v)) return fail(FA_ERR_INVALID_ARG, "null k or v pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
  const size_t q_bytes = (size_t)total_q * Hq * d * 2;
  const size_t kv_bytes = (size_t)total_k * Hkv * d * 2;
  const size_t lse_bytes = (size_t)Hq * total_q * sizeof(float);
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) || overlaps(o, q_bytes, v, kv_bytes) ||
      overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
      overlaps(lse, lse_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, o, q_bytes))
    return fail(FA_ERR_INVALID_ARG, "outputs alias inputs or each other");

  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, causal != 0, scale,
                    reinterpret_cast<hipStream_t>(stream), cu_seqlens_q, cu_seqlens_k, total_q};
  const hipError_t e = fa::launch_prefill_bf16(a);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

FA_EXPORT size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_seqlen_k) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_seqlen_k <= 0 || Hq % Hkv != 0) return 0;
  return decode_layout(B, Hq, Hkv, d, max_seqlen_k).bytes;
}

namespace {

// fa_decode and fa_decode_noalloc: the same checks and launch; the second takes
// its workspace from the library's static device array (scratch != false).
fa_status_t decode_impl(fa_dtype_t dtype, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cu_seqlens_k, int max_seqlen_k, void* o, float* lse, int B, int Hq, int Hkv,
                        int d, float scale, void* workspace, size_t workspace_bytes, void* stream, bool scratch) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || max_seqlen_k < 0) return fail(FA_ERR_INVALID_ARG, "negative size (B=%d max_seqlen_k=%d)", B, max_seqlen_k);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d <= 0) return fail(FA_ERR_INVALID_ARG, "head dim d=%d", d);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive (got %g)", (double)scale);
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "decode supports bf16 only");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (Hq / Hkv > fa::decode_max_group())
    return fail(FA_ERR_UNSUPPORTED, "Hq/Hkv=%d above %d", Hq / Hkv, fa::decode_max_group());
  if (B == 0) return ok();
  if (((int64_t)B + kDecodeWaves) * Hq > INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "B*Hq too large");
  if (!q || !o || !lse || !cu_seqlens_k) return fail(FA_ERR_INVALID_ARG, "null q, o, lse or cu_seqlens_k pointer");
  if (max_seqlen_k > 0 && (!k_cache || !v_cache)) return fail(FA_ERR_INVALID_ARG, "null cache pointer");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return fail(FA_ERR_INVALID_ARG, "tensor and workspace pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens_k must be 4-byte aligned");
  const size_t need = fa_decode_workspace_bytes(B, Hq, Hkv, d, max_seqlen_k);
  const size_t qo_bytes = (size_t)B * Hq * d * 2;
  const size_t lse_bytes = (size_t)B * Hq * sizeof(float);
  if (scratch) {
    workspace = nullptr;
    if (need > FA_DECODE_SCRATCH_BYTES)
      return fail(FA_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; the static array holds %zu "
                  "(use fa_decode with a caller-owned workspace)", need, (size_t)FA_DECODE_SCRATCH_BYTES);
  } else if (need > 0 && (!workspace || workspace_bytes < need)) {
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                need);
  }
  if (overlaps(o, qo_bytes, q, qo_bytes) || overlaps(lse, lse_bytes, q, qo_bytes) ||
      overlaps(lse, lse_bytes, o, qo_bytes) || overlaps(workspace, need, o, qo_bytes) ||
      overlaps(workspace, need, lse, lse_bytes) || overlaps(workspace, need, q, qo_bytes))
    return fail(FA_ERR_INVALID_ARG, "outputs or workspace alias inputs or each other");
  // every argument checked: only now the static array's address (the one
  // device call before the launch)
  if (scratch && need > 0) {
    const hipError_t e = fa::decode_scratch(&workspace, &workspace_bytes);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "no address for the static scratch array: %s", hipGetErrorString(e));
  }

  const DecodeLayout lay = decode_layout(B, Hq, Hkv, d, max_seqlen_k);
  float* part_o = lay.ranges > 0 ? static_cast<float*>(workspace) : nullptr;
  float* part_lse =
      lay.ranges > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.lse_offset) : nullptr;
  fa::DecodeArgs a{q, k_cache, v_cache, cu_seqlens_k, o, lse, part_o, part_lse, B, Hq, Hkv, d,
                   lay.ranges, scale, reinterpret_cast<hipStream_t>(stream)};
  const hipError_t e = fa::launch_decode_bf16(a);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

FA_EXPORT fa_status_t fa_decode(fa_dtype_t dtype, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cu_seqlens_k, int max_seqlen_k, void* o, float* lse, int B,
                                int Hq, int Hkv, int d, float scale, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_impl(dtype, q, k_cache, v_cache, cu_seqlens_k, max_seqlen_k, o, lse, B, Hq, Hkv, d, scale, workspace,
                     workspace_bytes, stream, false);
}

FA_EXPORT fa_status_t fa_decode_noalloc(fa_dtype_t dtype, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* cu_seqlens_k, int max_seqlen_k, void* o, float* lse, int B,
                                        int Hq, int Hkv, int d, float scale, void* stream) {
  return decode_impl(dtype, q, k_cache, v_cache, cu_seqlens_k, max_seqlen_k, o, lse, B, Hq, Hkv, d, scale, nullptr, 0,
                     stream, true);
}

namespace {

// Paged decode workspace: the tile prefix sums [B+1] int32 (256-byte padded),
// then the split's partial results, planned for up to max_seqlen_k + 1 keys
// per sequence (room for an appended row).
struct PagedLayout {
  DecodeLayout dec;
  size_t part_offset;
  size_t bytes;
};

PagedLayout paged_layout(int B, int Hq, int Hkv, int d, int max_seqlen_k) {
  PagedLayout p{decode_layout(B, Hq, Hkv, d, max_seqlen_k + 1), 0, 0};
  p.part_offset = ((size_t)(B + 1) * sizeof(int32_t) + 255) / 256 * 256;
  p.bytes = p.part_offset + p.dec.bytes;
  return p;
}

}  // namespace

FA_EXPORT size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int d, int max_seqlen_k) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_seqlen_k < 0 || max_seqlen_k == INT_MAX || Hq % Hkv != 0)
    return 0;
  return paged_layout(B, Hq, Hkv, d, max_seqlen_k).bytes;
}

FA_EXPORT fa_status_t fa_decode_paged(fa_dtype_t dtype, const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* block_table,
                                      const int32_t* seqlens_k, int num_blocks, int block_size,
                                      int max_blocks_per_seq, int max_seqlen_k, void* o, float* lse, int B,
                                      int Hq, int Hkv, int d, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || max_seqlen_k < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d max_seqlen_k=%d num_blocks=%d max_blocks_per_seq=%d)", B,
                max_seqlen_k, num_blocks, max_blocks_per_seq);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d <= 0) return fail(FA_ERR_INVALID_ARG, "head dim d=%d", d);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive (got %g)", (double)scale);
  if (block_size < fa::kDecodeTile || (block_size & (block_size - 1)) != 0 || block_size > (1 << 24))
    return fail(FA_ERR_INVALID_ARG, "block_size=%d must be a power of two from %d to 2^24", block_size,
                fa::kDecodeTile);
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(FA_ERR_INVALID_ARG, "k_new and v_new must both be given or both be null");
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "decode supports bf16 only");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (Hq / Hkv > fa::decode_max_group())
    return fail(FA_ERR_UNSUPPORTED, "Hq/Hkv=%d above %d", Hq / Hkv, fa::decode_max_group());
  if (B == 0) return ok();
  const int append = k_new ? 1 : 0;
  if (max_seqlen_k == INT_MAX) return fail(FA_ERR_UNSUPPORTED, "max_seqlen_k too large");
  if ((int64_t)max_seqlen_k + append > (int64_t)max_blocks_per_seq * block_size)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_k=%d (+%d appended) exceeds the table's %d blocks of %d rows",
                max_seqlen_k, append, max_blocks_per_seq, block_size);
  if (((int64_t)B + kDecodeWaves) * Hq > INT32_MAX || (int64_t)B * max_blocks_per_seq > ((int64_t)1 << 62) ||
      (int64_t)B * (((int64_t)max_seqlen_k + 1 + fa::kDecodeTile - 1) / fa::kDecodeTile) > INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "B, max_blocks_per_seq or max_seqlen_k too large");
  if (!q || !o || !lse || !block_table || !seqlens_k)
    return fail(FA_ERR_INVALID_ARG, "null q, o, lse, block_table or seqlens_k pointer");
  if (num_blocks > 0 && (!k_cache || !v_cache)) return fail(FA_ERR_INVALID_ARG, "null cache pointer");
  if (max_blocks_per_seq < 1) return fail(FA_ERR_INVALID_ARG, "max_blocks_per_seq must be at least 1");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace) || !aligned16(k_new) || !aligned16(v_new))
    return fail(FA_ERR_INVALID_ARG, "tensor and workspace pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 || (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0)
    return fail(FA_ERR_INVALID_ARG, "block_table and seqlens_k must be 4-byte aligned");
  const size_t need = fa_decode_paged_workspace_bytes(B, Hq, Hkv, d, max_seqlen_k);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  const size_t qo_bytes = (size_t)B * Hq * d * 2;
  const size_t lse_bytes = (size_t)B * Hq * sizeof(float);
  const size_t new_bytes = (size_t)B * Hkv * d * 2;
  const size_t cache_bytes = (size_t)num_blocks * block_size * Hkv * d * 2;
  const size_t table_bytes = (size_t)B * max_blocks_per_seq * sizeof(int32_t);
  const size_t len_bytes = (size_t)B * sizeof(int32_t);
  // written: o, lse, workspace, and (appending) both caches; none may overlap
  // anything else the call reads or writes
  struct Span { const void* p; size_t n; bool written; };
  const Span spans[] = {{q, qo_bytes, false},          {k_new, new_bytes, false},
                        {v_new, new_bytes, false},      {block_table, table_bytes, false},
                        {seqlens_k, len_bytes, false},  {k_cache, cache_bytes, append != 0},
                        {v_cache, cache_bytes, append != 0}, {o, qo_bytes, true},
                        {lse, lse_bytes, true},         {workspace, need, true}};
  const int ns = (int)(sizeof spans / sizeof spans[0]);
  for (int i = 0; i < ns; ++i)
    for (int j = i + 1; j < ns; ++j)
      if ((spans[i].written || spans[j].written) && overlaps(spans[i].p, spans[i].n, spans[j].p, spans[j].n))
        return fail(FA_ERR_INVALID_ARG, "outputs, workspace or written caches alias other arguments");

  const PagedLayout lay = paged_layout(B, Hq, Hkv, d, max_seqlen_k);
  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws + lay.part_offset);
  float* part_lse = reinterpret_cast<float*>(ws + lay.part_offset + lay.dec.lse_offset);
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  fa::DecodeArgs a{q, k_cache, v_cache, nullptr, o, lse, part_o, part_lse, B, Hq, Hkv, d,
                   lay.dec.ranges, scale, reinterpret_cast<hipStream_t>(stream)};
  a.block_table = block_table;
  a.seqlens = seqlens_k;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cu_tiles = reinterpret_cast<int32_t*>(ws);
  a.max_blocks = max_blocks_per_seq;
  a.bs_log2 = bs_log2;
  a.num_blocks = num_blocks;
  const hipError_t e = fa::launch_decode_paged_bf16(a);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

FA_EXPORT size_t fa_bwd_workspace_bytes(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  // per (batch, head) and 32-row query tile: the rows' base-2 LSE, then D (fp32)
  return (size_t)B * Hq * ((N + 31) / 32) * 64 * sizeof(float);
}

FA_EXPORT fa_status_t fa_bwd(fa_dtype_t dtype, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int Hq,
                             int Hkv, int N, int Nk, int d, int causal, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || N < 0 || Nk < 0) return fail(FA_ERR_INVALID_ARG, "negative size (B=%d N=%d Nk=%d)", B, N, Nk);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d <= 0) return fail(FA_ERR_INVALID_ARG, "head dim d=%d", d);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive (got %g)", (double)scale);
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "the backward supports bf16 only");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (B == 0 || (N == 0 && Nk == 0)) return ok();
  if ((int64_t)B * N > INT32_MAX || (int64_t)B * Nk > INT32_MAX ||
      (int64_t)B * Hq * ((N + 63) / 64) > INT32_MAX - 8 || (int64_t)B * Hkv * ((Nk + 63) / 64) > INT32_MAX - 8 ||
      (int64_t)B * N * Hq * (d / 8) > ((int64_t)1 << 40))
    return fail(FA_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
  if (((int64_t)N + 256) * Hq * d * 2 >= INT32_MAX || ((int64_t)Nk + 256) * Hkv * d * 2 >= INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "one batch of q or k/v exceeds 2 GiB");
  if (N > 0 && (!q || !o || !lse || !dout || !dq)) return fail(FA_ERR_INVALID_ARG, "null q, o, lse, dout or dq pointer");
  if (Nk > 0 && (!k || !v || !dk || !dv)) return fail(FA_ERR_INVALID_ARG, "null k, v, dk or dv pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return fail(FA_ERR_INVALID_ARG, "tensor and workspace pointers must be 16-byte aligned");
  const size_t need = fa_bwd_workspace_bytes(B, Hq, N);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  const size_t q_bytes = (size_t)B * N * Hq * d * 2;
  const size_t kv_bytes = (size_t)B * Nk * Hkv * d * 2;
  const size_t lse_bytes = (size_t)B * Hq * N * sizeof(float);
  struct Span { const void* p; size_t n; bool written; };
  const Span spans[] = {{q, q_bytes, false},   {k, kv_bytes, false},  {v, kv_bytes, false},
                        {o, q_bytes, false},   {lse, lse_bytes, false}, {dout, q_bytes, false},
                        {dq, q_bytes, true},   {dk, kv_bytes, true},  {dv, kv_bytes, true},
                        {workspace, need, true}};
  const int ns = (int)(sizeof spans / sizeof spans[0]);
  for (int i = 0; i < ns; ++i)
    for (int j = i + 1; j < ns; ++j)
      if ((spans[i].written || spans[j].written) && overlaps(spans[i].p, spans[i].n, spans[j].p, spans[j].n))
        return fail(FA_ERR_INVALID_ARG, "gradients or workspace alias other arguments");

  fa::BwdArgs a{q,  k,  v,  o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, Hq, Hkv, N, Nk, d,
                causal != 0, scale, reinterpret_cast<hipStream_t>(stream)};
  const hipError_t e = fa::launch_bwd_bf16(a);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}
