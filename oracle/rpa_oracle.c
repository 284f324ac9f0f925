/*
 * rpa_oracle.c -- plain fp64 CPU oracle for batched attention over a paged
 * KV cache with a ragged batch of sequences.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two are independent
 * implementations of the same definition.
 *
 * What it computes (written out directly from the definition, no blocking,
 * no online softmax, no splitting):
 *
 *   For each sequence b of the batch:
 *     q_len  = qo_indptr[b+1] - qo_indptr[b]
 *     n_pg   = kv_page_indptr[b+1] - kv_page_indptr[b]
 *     kv_len = n_pg == 0 ? 0 : (n_pg - 1) * page_size + kv_last_page_len[b]
 *   Token t < kv_len of sequence b lives in physical page
 *     kv_page_indices[kv_page_indptr[b] + t / page_size], slot t % page_size,
 *   of a cache laid out [num_pages][2][page_size][num_kv_heads][head_dim]
 *   ("NHD" per page; index 0 of the size-2 axis is K, 1 is V).
 *   (flashinfer issue #323, "How are prefill and decode kernels different?":
 *   the repro's kv_cache shape and the kv_page_indptr / kv_page_indices /
 *   kv_last_page_len tensors.)
 *
 *   Query i < q_len of sequence b is packed at row qo_indptr[b] + i of
 *   q[total_q][num_qo_heads][head_dim] (same issue: qo_indptr of the prefill
 *   wrapper).  The queries are the LAST q_len tokens of the sequence: query i
 *   sits at position pos = kv_len - q_len + i and, when causal, sees keys
 *   0..pos; otherwise it sees all kv_len keys (llama.cpp discussion #15958,
 *   "Pad for prefill stage?": prompts are real tokens followed by padding,
 *   and the FlashAttention kernel's mask hides the tail).  A causal sequence
 *   needs q_len <= kv_len; a non-causal one may have more queries than keys
 *   (the shared-prefix segment of a cascade: every request's queries against
 *   one prefix, vLLM issue #227, "Question about efficient memory sharing"),
 *   but at least one key when it has queries.
 *
 *   Query head h reads kv head h / (num_qo_heads / num_kv_heads) (grouped
 *   query attention with contiguous groups; flashinfer issue #323 uses
 *   64/8 qo heads over 8/8 kv heads).
 *
 *   With s_j = sm_scale * <q, K_j> over the n visible keys:
 *     m = max_j s_j,  l = sum_j exp(s_j - m),
 *     O   = sum_j exp(s_j - m) * V_j / l,
 *     LSE = m + ln(l)            (natural logarithm).
 *
 * Inputs are raw 16-bit patterns (binary16 or bfloat16), decoded exactly to
 * binary64 by the decoders below, written from the two formats' bit-field
 * definitions.  All arithmetic is binary64, in a fixed order per output, so
 * results are deterministic for any thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_OK = 0, ORC_E_ARG = 1, ORC_E_INDPTR = 2, ORC_E_LAST_PAGE_LEN = 3,
       ORC_E_QLEN_GT_KVLEN = 4, ORC_E_PAGE_OOB = 5, ORC_E_NOMEM = 6 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_binary16(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);  /* (1.f) * 2^(e-15), scaled */
    return sign ? -v : v;
}

/* bfloat16: the upper half of an IEEE 754 binary32: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits. */
static double decode_bfloat16(uint16_t b)
{
    int sign = b >> 15;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);             /* subnormal: f * 2^(1-127-7) */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 128), e - 134);  /* (1.f) * 2^(e-127), scaled */
    return sign ? -v : v;
}

static double decode(uint16_t x, int dtype) { return dtype == 0 ? decode_binary16(x) : decode_bfloat16(x); }

/* Exported so tests can pin the decoders against independent libraries. */
void rpa_oracle_decode(int32_t dtype, int64_t n, const uint16_t* in, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode(in[i], dtype);
}

typedef struct {
    int32_t batch;
    const int32_t *qo_indptr, *kv_page_indptr, *kv_page_indices, *kv_last_page_len;
    int32_t num_qo_heads, num_kv_heads, head_dim, page_size, dtype, causal;
    double sm_scale;
    const uint16_t *q, *kv_cache;
    double *o, *lse;
    const int64_t* rows;   /* token rows to compute, or NULL for all */
    int64_t n_rows;
    int64_t total_q;
    int32_t nthreads, tid;
    int32_t max_kv;
} job_t;

static int32_t seq_kv_len(const job_t* J, int32_t b)
{
    int32_t np = J->kv_page_indptr[b + 1] - J->kv_page_indptr[b];
    return np == 0 ? 0 : (np - 1) * J->page_size + J->kv_last_page_len[b];
}

/* Element d of K (kv = 0) or V (kv = 1) of token t, kv head hk, sequence b. */
static double kv_elem(const job_t* J, int32_t b, int32_t t, int32_t kv, int32_t hk, int32_t d)
{
    int64_t page = J->kv_page_indices[J->kv_page_indptr[b] + t / J->page_size];
    int64_t slot = t % J->page_size;
    int64_t idx = (((page * 2 + kv) * J->page_size + slot) * J->num_kv_heads + hk) * J->head_dim + d;
    return decode(J->kv_cache[idx], J->dtype);
}

/* One output row: query token row r (belonging to sequence b, index i),
 * query head h.  Two passes over the visible keys, as in the definition. */
static void one_row(const job_t* J, int32_t b, int64_t r, int32_t h, double* s)
{
    const int32_t D = J->head_dim;
    const int32_t group = J->num_qo_heads / J->num_kv_heads;
    const int32_t hk = h / group;
    const int32_t q_len = J->qo_indptr[b + 1] - J->qo_indptr[b];
    const int32_t kv_len = seq_kv_len(J, b);
    const int32_t i = (int32_t)(r - J->qo_indptr[b]);
    const int32_t pos = kv_len - q_len + i;
    const int32_t n = J->causal ? pos + 1 : kv_len;
    const uint16_t* qrow = J->q + (r * J->num_qo_heads + h) * (int64_t)D;

    double m = -INFINITY;
    for (int32_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += decode(qrow[d], J->dtype) * kv_elem(J, b, j, 0, hk, d);
        s[j] = J->sm_scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int32_t j = 0; j < n; ++j) l += exp(s[j] - m);
    double* orow = J->o + (r * J->num_qo_heads + h) * (int64_t)D;
    for (int32_t d = 0; d < D; ++d) orow[d] = 0.0;
    for (int32_t j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        for (int32_t d = 0; d < D; ++d) orow[d] += w * kv_elem(J, b, j, 1, hk, d);
    }
    for (int32_t d = 0; d < D; ++d) orow[d] /= l;
    if (J->lse) J->lse[r * J->num_qo_heads + h] = m + log(l);
}

/* Sequence owning token row r: the b with qo_indptr[b] <= r < qo_indptr[b+1]. */
static int32_t seq_of_row(const job_t* J, int64_t r)
{
    int32_t lo = 0, hi = J->batch;  /* invariant: answer in [lo, hi) */
    while (hi - lo > 1) {
        int32_t mid = (lo + hi) / 2;
        if (J->qo_indptr[mid] <= r) lo = mid; else hi = mid;
    }
    while (lo < J->batch && J->qo_indptr[lo + 1] <= r) ++lo;  /* skip empty sequences */
    return lo;
}

static void* worker(void* arg)
{
    const job_t* J = (const job_t*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->max_kv > 0 ? J->max_kv : 1));
    if (!s) return (void*)1;
    int64_t n_units = (J->rows ? J->n_rows : J->total_q) * J->num_qo_heads;
    for (int64_t u = J->tid; u < n_units; u += J->nthreads) {
        int64_t k = u / J->num_qo_heads;
        int32_t h = (int32_t)(u % J->num_qo_heads);
        int64_t r = J->rows ? J->rows[k] : k;
        one_row(J, seq_of_row(J, r), r, h, s);
    }
    free(s);
    return NULL;
}

/*
 * Validate the page table and lengths, then compute O (and LSE if lse != NULL)
 * for all token rows, or only for `rows[0..n_rows)` when rows != NULL (other
 * rows of `o` / `lse` are left untouched).  Returns 0 or a positive error code.
 *
 *   q        : [qo_indptr[batch]][num_qo_heads][head_dim] raw 16-bit values
 *   kv_cache : [num_pages][2][page_size][num_kv_heads][head_dim] raw 16-bit
 *   o        : [qo_indptr[batch]][num_qo_heads][head_dim] binary64
 *   lse      : [qo_indptr[batch]][num_qo_heads] binary64, or NULL
 *   dtype    : 0 = binary16, 1 = bfloat16
 */
int rpa_oracle_run(int32_t batch, const int32_t* qo_indptr, const int32_t* kv_page_indptr,
                   const int32_t* kv_page_indices, const int32_t* kv_last_page_len, int64_t num_pages,
                   int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                   int32_t dtype, int32_t causal, double sm_scale, const uint16_t* q,
                   const uint16_t* kv_cache, double* o, double* lse, const int64_t* rows,
                   int64_t n_rows, int32_t nthreads)
{
    if (batch < 0 || !qo_indptr || !kv_page_indptr || num_qo_heads <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || page_size <= 0 || (dtype != 0 && dtype != 1) || !o ||
        num_qo_heads % num_kv_heads != 0)
        return ORC_E_ARG;
    if (qo_indptr[0] != 0 || kv_page_indptr[0] != 0) return ORC_E_INDPTR;
    int32_t max_kv = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (qo_indptr[b + 1] < qo_indptr[b] || kv_page_indptr[b + 1] < kv_page_indptr[b]) return ORC_E_INDPTR;
        int32_t np = kv_page_indptr[b + 1] - kv_page_indptr[b];
        if (np > 0 && (kv_last_page_len[b] < 1 || kv_last_page_len[b] > page_size)) return ORC_E_LAST_PAGE_LEN;
        int32_t kv_len = np == 0 ? 0 : (np - 1) * page_size + kv_last_page_len[b];
        int32_t q_len = qo_indptr[b + 1] - qo_indptr[b];
        /* Causal queries are the last q_len of kv_len positions, so q_len <= kv_len;
         * non-causal queries see all kv_len keys, any number of them, but need at
         * least one key. */
        if (causal ? q_len > kv_len : (q_len > 0 && kv_len == 0)) return ORC_E_QLEN_GT_KVLEN;
        for (int32_t p = kv_page_indptr[b]; p < kv_page_indptr[b + 1]; ++p)
            if (kv_page_indices[p] < 0 || kv_page_indices[p] >= num_pages) return ORC_E_PAGE_OOB;
        if (kv_len > max_kv) max_kv = kv_len;
    }
    int64_t total_q = qo_indptr[batch];
    if (total_q > 0 && (!q || !kv_cache)) return ORC_E_ARG;
    if (rows)
        for (int64_t k = 0; k < n_rows; ++k)
            if (rows[k] < 0 || rows[k] >= total_q) return ORC_E_ARG;
    if (nthreads < 1) nthreads = 1;

    job_t base = {batch, qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len,
                  num_qo_heads, num_kv_heads, head_dim, page_size, dtype, causal, sm_scale,
                  q, kv_cache, o, lse, rows, n_rows, total_q, nthreads, 0, max_kv};
    job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int8_t* started = (int8_t*)calloc((size_t)nthreads, 1);
    if (!jobs || !th || !started) { free(jobs); free(th); free(started); return ORC_E_NOMEM; }
    int failed = 0;
    for (int32_t t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].tid = t;
    }
    for (int32_t t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&th[t], NULL, worker, &jobs[t]) == 0;
    /* Units of a thread that could not be started are done on this thread. */
    for (int32_t t = 0; t < nthreads; ++t)
        if (t == 0 || !started[t]) failed |= worker(&jobs[t]) != NULL;
    for (int32_t t = 1; t < nthreads; ++t) {
        if (!started[t]) continue;
        void* ret = NULL;
        pthread_join(th[t], &ret);
        failed |= ret != NULL;
    }
    free(jobs);
    free(th);
    free(started);
    if (failed) return ORC_E_NOMEM;
    return ORC_OK;
}
