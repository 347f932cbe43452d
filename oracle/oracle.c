/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and
 * the benchmark's CPU-baseline leg may load or call this code.  The GPU path
 * never links it and shares no code, header or constant with it.
 *
 * What it computes (the plain definition, not the tiled method):
 *
 *   S = scale * Q K^T                      (one row of S per query row)
 *   S[i][j] = -inf where key j is not visible to query i
 *   P = softmax(S) along keys,  O = P V,   LSE_i = m_i + ln(sum_j exp(S_ij - m_i))
 *
 * Sources:
 *  - ai6s.net page, section "standard attention's fatal flaw is data movement,
 *    not compute": the four steps Q*K^T -> scale -> softmax -> *V.
 *  - ai6s.net page, section "FlashAttention changes the dataflow, not the
 *    algorithm": the method is exact, so its result is this definition.
 *  - ai6s.net page, section "what ops-transformer adds", second item (causal
 *    mask inside softmax) and third item (variable-length KV cache: attend to
 *    the real cache length only).
 *  - effectstory.com page, section "What is FlashAttention": exact, not an
 *    approximation.
 *
 * Readings taken where the pages are silent:
 *  - causal alignment is bottom-right: key j is visible to query i iff
 *    j <= i + (Nk - N); with N == Nk this is j <= i;
 *  - LSE is the natural log of sum_j exp(S_ij) over visible keys, scale included;
 *  - grouped-query attention uses contiguous groups: kv head g = h / (Hq / Hkv);
 *  - a row with no visible key has O = 0 and LSE = -inf;
 *  - in decode every one of the L_b cache rows of sequence b is visible.
 *
 * Layouts: prefill q,o [B,N,Hq,d], k,v [B,Nk,Hkv,d]; decode q [B,Hq,d],
 * k/v cache [total,Hkv,d] with cu_seqlens [B+1].  Inputs may be f64, f32 or
 * bf16 bit patterns; they are widened exactly to fp64 before any arithmetic
 * (bf16 -> f32 by a 16-bit left shift of the bits, f32 -> f64 exactly).
 * All arithmetic is fp64; sums run sequentially in index order.
 *
 * Row work is spread over POSIX threads; each row is computed the same way
 * whatever thread runs it, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORC_F64 0
#define ORC_F32 1
#define ORC_BF16 2

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENORM 2   /* softmax row did not sum to 1 within 1e-12 */
#define ORC_ENOMEM 3

/* Exact widening of one stored element to fp64. */
static double widen(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORC_F64)
        return ((const double *)base)[idx];
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    /* bf16: the 16 stored bits are the high half of an fp32 pattern */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One query row against one set of keys.
 *   q_off      element offset of the query row (d contiguous elements)
 *   k_off      element offset of key 0; key j starts at k_off + j*kv_stride
 *   nk         number of keys in the set
 *   nvis       keys 0..nvis-1 are visible, the rest are masked (0 <= nvis <= nk)
 * Writes d outputs to o_row and the row's LSE to *lse.
 * srow/prow are caller scratch of nk doubles each.
 */
static int attend_row(int dtype, const void *q, const void *k, const void *v,
                      int64_t q_off, int64_t k_off, int64_t kv_stride,
                      int nk, int nvis, int d, double scale,
                      double *srow, double *prow, double *o_row, double *lse)
{
    /* step 1: the row of S = scale * q . k_j, dot product summed over d in order */
    for (int j = 0; j < nk; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += widen(q, dtype, q_off + c) * widen(k, dtype, k_off + (int64_t)j * kv_stride + c);
        srow[j] = scale * dot;
    }
    /* step 2: the mask, applied as -inf by selection */
    for (int j = nvis; j < nk; ++j)
        srow[j] = -INFINITY;
    /* step 3: softmax along the row */
    double m = -INFINITY;
    for (int j = 0; j < nk; ++j)
        if (srow[j] > m)
            m = srow[j];
    if (m == -INFINITY) {            /* no visible key */
        for (int c = 0; c < d; ++c)
            o_row[c] = 0.0;
        *lse = -INFINITY;
        return ORC_OK;
    }
    double l = 0.0;
    for (int j = 0; j < nk; ++j) {
        prow[j] = exp(srow[j] - m);   /* exp(-inf) == 0 for masked keys */
        l += prow[j];
    }
    double psum = 0.0;
    for (int j = 0; j < nk; ++j) {
        prow[j] /= l;
        psum += prow[j];
    }
    if (!(fabs(psum - 1.0) <= 1e-12))
        return ORC_ENORM;
    /* step 4: O = P V */
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < nk; ++j)
            acc += prow[j] * widen(v, dtype, k_off + (int64_t)j * kv_stride + c);
        o_row[c] = acc;
    }
    /* step 5: LSE in natural log */
    *lse = m + log(l);
    return ORC_OK;
}

/* ---------------------------------------------------------------- threading */

typedef struct {
    /* shared, read-only */
    int mode;                 /* 0 = prefill, 1 = decode */
    int dtype;
    const void *q, *k, *v;
    const int32_t *cu;        /* decode only */
    int B, Hq, Hkv, N, Nk, d, causal;
    double scale;
    int64_t nrows;
    const int32_t *rb, *rh, *ri;
    double *o_out, *lse_out;
    int max_nk;
    /* shared, mutable */
    pthread_mutex_t lock;
    int64_t next;
    int status;
} job_t;

static int64_t grab(job_t *J, int64_t chunk, int64_t *end)
{
    pthread_mutex_lock(&J->lock);
    int64_t s = J->next;
    J->next = s + chunk < J->nrows ? s + chunk : J->nrows;
    *end = J->next;
    pthread_mutex_unlock(&J->lock);
    return s;
}

static void set_status(job_t *J, int st)
{
    pthread_mutex_lock(&J->lock);
    if (J->status == ORC_OK)
        J->status = st;
    pthread_mutex_unlock(&J->lock);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *srow = (double *)malloc(sizeof(double) * (size_t)(J->max_nk > 0 ? J->max_nk : 1));
    double *prow = (double *)malloc(sizeof(double) * (size_t)(J->max_nk > 0 ? J->max_nk : 1));
    if (!srow || !prow) {
        set_status(J, ORC_ENOMEM);
        free(srow);
        free(prow);
        return NULL;
    }
    const int group = J->Hq / J->Hkv;
    for (;;) {
        int64_t end;
        int64_t r = grab(J, 16, &end);
        if (r >= end)
            break;
        for (; r < end; ++r) {
            const int b = J->rb[r], h = J->rh[r];
            const int g = h / group;                       /* contiguous query-head groups */
            int64_t q_off, k_off;
            int nk, nvis;
            if (J->mode == 0) {
                const int i = J->ri[r];
                q_off = (((int64_t)b * J->N + i) * J->Hq + h) * J->d;
                k_off = ((int64_t)b * J->Nk * J->Hkv + g) * J->d;
                nk = J->Nk;
                if (J->causal) {
                    /* bottom-right alignment: query i sits at key position i + Nk - N */
                    int64_t last = (int64_t)i + J->Nk - J->N;   /* last visible key */
                    nvis = last < 0 ? 0 : (last + 1 > nk ? nk : (int)(last + 1));
                } else {
                    nvis = nk;
                }
            } else {
                q_off = ((int64_t)b * J->Hq + h) * J->d;
                const int64_t start = J->cu[b];
                k_off = (start * J->Hkv + g) * J->d;
                nk = (int)(J->cu[b + 1] - start);
                nvis = nk;                                   /* whole real cache length */
            }
            int st = attend_row(J->dtype, J->q, J->k, J->v, q_off, k_off,
                                (int64_t)J->Hkv * J->d, nk, nvis, J->d, J->scale,
                                srow, prow, J->o_out + r * J->d, J->lse_out + r);
            if (st != ORC_OK)
                set_status(J, st);
        }
    }
    free(srow);
    free(prow);
    return NULL;
}

static int run_job(job_t *J, int nthreads)
{
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 1024)
        nthreads = 1024;
    pthread_mutex_init(&J->lock, NULL);
    J->next = 0;
    J->status = ORC_OK;
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tids)
        return ORC_ENOMEM;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, worker, J) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(J);
    for (int t = 0; t < started; ++t)
        pthread_join(tids[t], NULL);
    free(tids);
    pthread_mutex_destroy(&J->lock);
    return J->status;
}

/* ------------------------------------------------------------- entry points */

int oracle_version(void) { return 1; }

/*
 * Prefill attention for an explicit list of query rows (b, h, i).
 * o_out [nrows, d] and lse_out [nrows] receive fp64 results.
 */
int oracle_attn_rows(int dtype, const void *q, const void *k, const void *v,
                     int B, int Hq, int Hkv, int N, int Nk, int d, int causal,
                     double scale, int64_t nrows,
                     const int32_t *rb, const int32_t *rh, const int32_t *ri,
                     double *o_out, double *lse_out, int nthreads)
{
    if (dtype < ORC_F64 || dtype > ORC_BF16 || B < 0 || Hq <= 0 || Hkv <= 0 ||
        Hq % Hkv != 0 || N < 0 || Nk < 0 || d <= 0 || nrows < 0)
        return ORC_EINVAL;
    for (int64_t r = 0; r < nrows; ++r)
        if (rb[r] < 0 || rb[r] >= B || rh[r] < 0 || rh[r] >= Hq || ri[r] < 0 || ri[r] >= N)
            return ORC_EINVAL;
    job_t J;
    memset(&J, 0, sizeof J);
    J.mode = 0; J.dtype = dtype; J.q = q; J.k = k; J.v = v;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.Nk = Nk; J.d = d; J.causal = causal != 0;
    J.scale = scale; J.nrows = nrows; J.rb = rb; J.rh = rh; J.ri = ri;
    J.o_out = o_out; J.lse_out = lse_out; J.max_nk = Nk;
    return run_job(&J, nthreads);
}

/*
 * Decode attention (one query token per sequence) over a packed cache for an
 * explicit list of (sequence b, query head h) pairs.  Keys of sequence b are
 * cache rows cu[b] .. cu[b+1]-1.  o_out [nrows, d], lse_out [nrows].
 */
int oracle_decode_rows(int dtype, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *cu, int B, int Hq, int Hkv, int d, double scale,
                       int64_t nrows, const int32_t *rb, const int32_t *rh,
                       double *o_out, double *lse_out, int nthreads)
{
    if (dtype < ORC_F64 || dtype > ORC_BF16 || B < 0 || Hq <= 0 || Hkv <= 0 ||
        Hq % Hkv != 0 || d <= 0 || nrows < 0)
        return ORC_EINVAL;
    if (B > 0 && cu[0] != 0)
        return ORC_EINVAL;
    int max_nk = 0;
    for (int b = 0; b < B; ++b) {
        int64_t len = (int64_t)cu[b + 1] - cu[b];
        if (len < 0)
            return ORC_EINVAL;
        if (len > max_nk)
            max_nk = (int)len;
    }
    for (int64_t r = 0; r < nrows; ++r)
        if (rb[r] < 0 || rb[r] >= B || rh[r] < 0 || rh[r] >= Hq)
            return ORC_EINVAL;
    job_t J;
    memset(&J, 0, sizeof J);
    J.mode = 1; J.dtype = dtype; J.q = q; J.k = k_cache; J.v = v_cache; J.cu = cu;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = 1; J.d = d; J.scale = scale;
    J.nrows = nrows; J.rb = rb; J.rh = rh; J.ri = NULL;
    J.o_out = o_out; J.lse_out = lse_out; J.max_nk = max_nk;
    return run_job(&J, nthreads);
}
