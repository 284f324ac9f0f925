/* Sanitizer test program for the oracle (test infrastructure): random small ragged batches,
 * valid and invalid, through rpa_oracle_run on 1 and 3 threads, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Exits 0 when every call behaved
 * and outputs of the two thread counts agree bit for bit. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int rpa_oracle_run(int32_t batch, const int32_t* qo_indptr, const int32_t* kv_page_indptr,
                   const int32_t* kv_page_indices, const int32_t* kv_last_page_len, int64_t num_pages,
                   int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                   int32_t dtype, int32_t causal, double sm_scale, const uint16_t* q,
                   const uint16_t* kv_cache, double* o, double* lse, const int64_t* rows,
                   int64_t n_rows, int32_t nthreads);

static uint32_t state = 12345;
static uint32_t rnd(void) {
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    return state;
}

int main(void) {
    int failures = 0, ran = 0, refused = 0;
    for (int it = 0; it < 200; ++it) {
        const int H = 1 + (int)(rnd() % 4) * 2, Hk = (rnd() % 2) ? 1 : H, D = 8 + 8 * (int)(rnd() % 3), ps = 16;
        const int B = 1 + (int)(rnd() % 5), causal = (int)(rnd() % 3 != 0), dtype = (int)(rnd() % 2);
        int32_t qo[8] = {0}, kp[8] = {0}, kl[8];
        for (int b = 0; b < B; ++b) {
            int q = (int)(rnd() % 6), kv = causal ? q + (int)(rnd() % 40) : (int)(rnd() % 40) + (q ? 1 : 0);
            if (rnd() % 30 == 0) kv = 0;
            qo[b + 1] = qo[b] + q;
            int np = (kv + ps - 1) / ps;
            kp[b + 1] = kp[b] + np;
            kl[b] = np ? (kv - 1) % ps + 1 : 1;
        }
        if (rnd() % 20 == 0) kl[rnd() % B] = 0;
        const int64_t pool = kp[B] + 3;
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(kp[B] + 1));
        for (int i = 0; i < kp[B]; ++i) idx[i] = (int32_t)(rnd() % (uint32_t)pool);
        if (kp[B] > 0 && rnd() % 20 == 0) idx[rnd() % (uint32_t)kp[B]] = (int32_t)pool;  /* out of range */
        const int64_t T = qo[B];
        const size_t nq = (size_t)(T * H * D), nkv = (size_t)(pool * 2 * ps * Hk * D);
        uint16_t* q = (uint16_t*)malloc(2 * (nq + 1));
        uint16_t* kv = (uint16_t*)malloc(2 * (nkv + 1));
        for (size_t i = 0; i < nq; ++i) q[i] = (uint16_t)(0x3000 + rnd() % 0x0c00 + (rnd() % 2) * 0x8000);
        for (size_t i = 0; i < nkv; ++i) kv[i] = (uint16_t)(0x3000 + rnd() % 0x0c00 + (rnd() % 2) * 0x8000);
        double* o1 = (double*)malloc(8 * (nq + 1));
        double* o3 = (double*)malloc(8 * (nq + 1));
        double* l1 = (double*)malloc(8 * (size_t)(T * H + 1));
        double* l3 = (double*)malloc(8 * (size_t)(T * H + 1));
        const int r1 = rpa_oracle_run(B, qo, kp, idx, kl, pool, H, Hk, D, ps, dtype, causal, 0.0, q, kv, o1, l1,
                                      NULL, 0, 1);
        const int r3 = rpa_oracle_run(B, qo, kp, idx, kl, pool, H, Hk, D, ps, dtype, causal, 0.0, q, kv, o3, l3,
                                      NULL, 0, 3);
        if (r1 != r3) ++failures;
        if (r1 == 0) {
            ++ran;
            if (memcmp(o1, o3, 8 * nq) != 0 || memcmp(l1, l3, 8 * (size_t)(T * H)) != 0) ++failures;
            if (T > 0) {  /* a row subset computes those rows only */
                int64_t row = (int64_t)(rnd() % (uint32_t)T);
                if (rpa_oracle_run(B, qo, kp, idx, kl, pool, H, Hk, D, ps, dtype, causal, 0.0, q, kv, o3, l3, &row,
                                   1, 2) != 0)
                    ++failures;
            }
        } else {
            ++refused;
        }
        free(idx); free(q); free(kv); free(o1); free(o3); free(l1); free(l3);
    }
    printf("oracle fuzz: %d batches run, %d refused, %d failures\n", ran, refused, failures);
    return failures == 0 ? 0 : 1;
}
