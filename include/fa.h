/*
 * fa.h -- C ABI of the exact, IO-aware attention forward library (libfa.so)
 * for AMD MI355X (gfx950).
 *
 * The library computes, for every query row i of every (batch b, query head h),
 *
 *     O[i] = sum_j softmax_j(scale * q_i . k_j) * v_j     over visible keys j
 *     LSE[i] = ln sum_j exp(scale * q_i . k_j)             (natural log)
 *
 * without ever writing the N x Nk score matrix to device memory: Q, K and V
 * are tiled along the sequence axis, K/V tiles stream through on-chip memory
 * and a running row max and row sum rescale the partial output (ai6s.net page,
 * section "FlashAttention changes the dataflow, not the algorithm").  The
 * result is exact attention up to floating-point rounding order (same section;
 * effectstory.com page, section "What is FlashAttention").
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, owned by the caller, contiguous,
 *    16-byte aligned, and must stay valid until the enqueued work completes.
 *    Outputs must not alias inputs.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the default
 *    stream).  Calls return without synchronising; the library never
 *    allocates device memory, copies between host and device or synchronises.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error no kernel is launched and no output is touched.  Faults that occur
 *    while a kernel runs surface at the caller's next synchronisation.
 *  - Grouped-query attention: Hq must be a multiple of Hkv and query head h
 *    reads kv head h / (Hq / Hkv) (contiguous groups).
 *  - head dimension d must be 64 or 128.
 *  - scale must be finite and positive.
 *  - The only mutable state is a per-thread copy of the last error's detail
 *    text (fa_last_error); calls from several threads and on different
 *    streams may run concurrently.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 5

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, Hq % Hkv != 0, bad scale, misalignment */
    FA_ERR_UNSUPPORTED = 2,   /* valid but not implemented: head dim, dtype for this entry point */
    FA_ERR_WORKSPACE = 3,     /* decode workspace missing or smaller than fa_decode_workspace_bytes */
    FA_ERR_HIP = 4            /* the HIP runtime rejected a launch */
} fa_status_t;

typedef enum {
    FA_F32 = 0,               /* fp32 in, fp32 out, fp32 arithmetic */
    FA_BF16 = 1               /* bf16 in, bf16 out (round to nearest even), fp32 accumulation */
} fa_dtype_t;

/*
 * Prefill / full-sequence forward.
 *
 * Computes attention of N query rows against Nk keys for every (b, h)
 * (ai6s.net page, sections "standard attention's fatal flaw ..." for the
 * definition and "what ops-transformer adds", second item, for the causal mask
 * fused into the blockwise softmax).
 *
 *   q    [B, N,  Hq,  d]  dtype   (BSHD, row-major, contiguous)
 *   k, v [B, Nk, Hkv, d]  dtype
 *   o    [B, N,  Hq,  d]  dtype   output
 *   lse  [B, Hq, N]       fp32    output, natural-log logsumexp of scale*q.k
 *                                 over the keys visible to the row
 *   causal != 0: bottom-right alignment, key j is visible to query i iff
 *                j <= i + (Nk - N)  (j <= i when N == Nk).  Key tiles that are
 *                entirely masked are never loaded.
 *   A row with no visible key (possible only when causal and Nk < N) gets
 *   O = 0 and LSE = -inf.
 *   B == 0, N == 0 are no-ops returning FA_OK.  Nk == 0 gives O = 0, LSE = -inf.
 *
 * Returns FA_OK or an error status (see above); nothing is enqueued on error.
 */
fa_status_t fa_fwd(fa_dtype_t dtype,
                   const void *q, const void *k, const void *v,
                   void *o, float *lse,
                   int B, int Hq, int Hkv, int N, int Nk, int d,
                   int causal, float scale, void *stream);

/*
 * Variable-length and chunked prefill: B packed sequences, sequence b having
 * N_b query rows and Nk_b keys, N_b <= Nk_b typical for a chunk of new tokens
 * appended to a cache of Nk_b - N_b earlier ones (ai6s.net page, section
 * "what ops-transformer adds", third item: attend to the real lengths only;
 * second item: the causal mask inside the blockwise softmax).
 *
 *   q            [total_q, Hq,  d]  bf16, sequence b owns rows
 *                                   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   k, v         [total_k, Hkv, d]  bf16, sequence b owns rows
 *                                   cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *   cu_seqlens_q,
 *   cu_seqlens_k [B+1]              int32, DEVICE pointers; cu[0] == 0,
 *                                   non-decreasing, cu_seqlens_q[B] == total_q,
 *                                   cu_seqlens_k[B] == total_k.  These cannot be
 *                                   checked without a synchronisation, so they
 *                                   are preconditions, and so are
 *                                   N_b <= max_seqlen_q and Nk_b <= max_seqlen_k.
 *   max_seqlen_q,
 *   max_seqlen_k                    host-side upper bounds on the lengths
 *   o            [total_q, Hq, d]   bf16 output
 *   lse          [Hq, total_q]      fp32 output, natural-log logsumexp
 *   causal != 0: bottom-right alignment within each sequence, key j of
 *                sequence b is visible to its query i iff j <= i + (Nk_b - N_b).
 *   A row with no visible key gets O = 0 and LSE = -inf; a sequence with no
 *   query rows writes nothing.  B == 0 or total_q == 0 is a no-op.
 *   dtype must be FA_BF16 (FA_F32 returns FA_ERR_UNSUPPORTED).
 *
 * Returns FA_OK or an error status (see above); nothing is enqueued on error.
 */
fa_status_t fa_fwd_varlen(fa_dtype_t dtype,
                          const void *q, const void *k, const void *v,
                          const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                          int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                          void *o, float *lse,
                          int B, int Hq, int Hkv, int d,
                          int causal, float scale, void *stream);

/*
 * Decode forward over a packed, variable-length KV cache (one new query token
 * per sequence).  Only the real cache length of each sequence is read: no
 * work is done for keys beyond it (ai6s.net page, section "what
 * ops-transformer adds", third item).
 *
 *   q            [B, Hq, d]       bf16
 *   k_cache,
 *   v_cache      [total, Hkv, d]  bf16, sequence b occupies rows
 *                                 cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *   cu_seqlens_k [B+1]            int32, DEVICE pointer; cu[0] == 0,
 *                                 non-decreasing.  This cannot be checked
 *                                 without a synchronisation, so it is a
 *                                 precondition: every length must be
 *                                 <= max_seqlen_k and rows must lie inside
 *                                 the caches.
 *   max_seqlen_k                  host-side upper bound on every length
 *   o            [B, Hq, d]       bf16 output
 *   lse          [B, Hq]          fp32 output (natural log)
 *   workspace                     device scratch of at least
 *                                 fa_decode_workspace_bytes(B, Hq, Hkv, d,
 *                                 max_seqlen_k) bytes, 16-byte aligned, owned
 *                                 by the caller; its contents on entry do not
 *                                 matter and on exit are unspecified.  Calls
 *                                 that share a workspace must be ordered on
 *                                 one stream.
 *   Every key of the sequence is visible (for one query at the end of the
 *   sequence, bottom-right causal alignment shows it all).  A sequence of
 *   length 0 gets O = 0, LSE = -inf.
 *   dtype must be FA_BF16 (FA_F32 returns FA_ERR_UNSUPPORTED).
 */
fa_status_t fa_decode(fa_dtype_t dtype,
                      const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *cu_seqlens_k, int max_seqlen_k,
                      void *o, float *lse,
                      int B, int Hq, int Hkv, int d, float scale,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace fa_decode needs for these sizes (0 when no work). */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_seqlen_k);

/* fa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, layouts, preconditions, results and errors as fa_decode,
 * without the workspace: the partial results live in a static device array of
 * FA_DECODE_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends (its address is looked up once per device, on the
 * first call with that device current).  The call allocates nothing and frees
 * nothing.  Returns FA_ERR_WORKSPACE when fa_decode_workspace_bytes(B, Hq,
 * Hkv, d, max_seqlen_k) exceeds FA_DECODE_SCRATCH_BYTES (the varlen decode of
 * 32 sequences, Hq 64, Hkv 8, d 128, caches up to 32768 rows needs about
 * 9.5 MB), and FA_ERR_HIP when the array's address cannot be obtained.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (no part of it needs to start at zero: every partial result read is
 * written by the same call first).  Calls that overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race on
 * the array; order them on one stream.
 */
#define FA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

fa_status_t fa_decode_noalloc(fa_dtype_t dtype,
                              const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *cu_seqlens_k, int max_seqlen_k,
                              void *o, float *lse,
                              int B, int Hq, int Hkv, int d, float scale, void *stream);

/* Decode on a paged KV cache, with the new token's K/V row appended first.
 *
 * Each sequence's cache grows by one row per generated token, and the token
 * attends to every row of its sequence's cache (ai6s.net page, section "what
 * ops-transformer adds", third item).  This call does both steps: when k_new
 * and v_new are given, the new token's key and value rows of sequence b are
 * written into the cache as its logical row L_b = seqlens_k[b], and the
 * token's query then attends to the L_b + 1 rows 0..L_b; when both are null
 * it attends to the L_b cached rows only.  Per (b, query head h, kv head
 * g = h / (Hq/Hkv)): O[b,h,:] and LSE[b,h] as in fa_decode.
 *
 * Layouts (all contiguous, bf16 unless noted):
 *   q                [B, Hq, d]
 *   k_new, v_new     [B, Hkv, d]   the new token's rows, or both NULL
 *   k_cache, v_cache [num_blocks, block_size, Hkv, d]: logical row i of
 *                    sequence b is row i % block_size of physical block
 *                    block_table[b * max_blocks_per_seq + i / block_size]
 *   block_table      int32 [B, max_blocks_per_seq], device memory
 *   seqlens_k        int32 [B], device memory: cached rows before the append
 *   o                [B, Hq, d];  lse  fp32 [B, Hq]
 * block_size is a power of two from 32 to 2^24; any number of blocks and any
 * cache size (no 4 GiB limit: every block is addressed on its own).
 *
 * Preconditions on device data (not checked, since that needs a sync):
 * 0 <= seqlens_k[b] <= max_seqlen_k; the table entries of the blocks holding
 * rows 0..L_b (0..L_b - 1 without an append) lie in [0, num_blocks); no two
 * sequences append into the same block row.  The kernels stay inside the
 * cache when an entry breaks this: rows in such a block are neither read nor
 * written, and they count as absent keys (a sequence left with no key gets
 * O = 0 and LSE = -inf).
 *
 * The cache is updated in place; the caller advances seqlens_k afterwards.
 * Ownership and errors as for fa_decode; the appended rows are written before
 * any row is read, in stream order.  The workspace holds
 * fa_decode_paged_workspace_bytes(B, Hq, Hkv, d, max_seqlen_k) bytes.  Returns
 * FA_ERR_INVALID_ARG when max_seqlen_k (+1 with an append) exceeds
 * max_blocks_per_seq * block_size, or when a written buffer (o, lse, the
 * workspace, the caches when appending) overlaps any other argument.
 */
fa_status_t fa_decode_paged(fa_dtype_t dtype,
                            const void *q, const void *k_new, const void *v_new,
                            void *k_cache, void *v_cache,
                            const int32_t *block_table, const int32_t *seqlens_k,
                            int num_blocks, int block_size, int max_blocks_per_seq, int max_seqlen_k,
                            void *o, float *lse,
                            int B, int Hq, int Hkv, int d, float scale,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace fa_decode_paged needs (0 when B is 0); the same size
 * serves calls with and without an append. */
size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int d, int max_seqlen_k);

/* Backward of fa_fwd: gradients dq, dk, dv of a loss whose gradient with
 * respect to O is dout (bf16).
 *
 * The pages state no backward algorithm; this is the chain rule of the
 * forward's definition (ai6s.net page, section "standard attention's fatal
 * flaw is data movement, not compute"), with P recomputed from the forward's
 * LSE (P_ij = exp(scale q_i.k_j - LSE_i) over the visible keys):
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D) with D_i = dO_i . O_i,
 *   dQ = scale dS K,  dK = scale dS^T Q;
 * the same mask as fa_fwd (bottom-right when causal), and for grouped heads
 * dk, dv of kv head g sum over query heads g*(Hq/Hkv) .. (g+1)*(Hq/Hkv)-1.
 *
 * Layouts (contiguous BSHD, bf16): q, o, dout, dq [B, N, Hq, d]; k, v, dk, dv
 * [B, Nk, Hkv, d]; lse [B, Hq, N] fp32 as written by fa_fwd for the same
 * q, k, v, causal and scale (o as well: D uses it).  Rows without a visible
 * key (LSE = -inf) get dq = 0 and add nothing to dk, dv.
 * Workspace: fa_bwd_workspace_bytes(B, Hq, N) bytes, caller-owned.
 * Ownership, asynchrony and errors as for fa_fwd; FA_ERR_UNSUPPORTED for
 * fp32 or d not in {64, 128}; FA_ERR_INVALID_ARG when a gradient or the
 * workspace overlaps another argument.  Deterministic: no atomics.
 */
fa_status_t fa_bwd(fa_dtype_t dtype,
                   const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv,
                   int B, int Hq, int Hkv, int N, int Nk, int d, int causal, float scale,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace fa_bwd needs (0 when there are no query rows). */
size_t fa_bwd_workspace_bytes(int B, int Hq, int N);

/* Static, human-readable name of a status code. */
const char *fa_status_str(fa_status_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *fa_last_error(void);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
