// Sanitizer test program for the library's host code: random ragged batches (and invalid
// ones) through rpa_plan_create(_shared) / info / tiles / update / destroy,
// rpa_workspace_bytes, rpa_trim_page_table, rpa_validate_page_table and the size
// check of rpa_run_noalloc, built with AddressSanitizer and UndefinedBehaviorSanitizer.
// Exits 0 when every call behaved; any sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "rpa.h"

extern int g_hip_calls;

static int failures = 0;
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 400;
    std::mt19937 rng(1234);
    auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
    int64_t plans = 0, refused = 0;
    for (int it = 0; it < iters; ++it) {
        rpa_params p{};
        const int shapes[][3] = {{8, 1, 128}, {32, 8, 128}, {64, 8, 128}, {8, 8, 64}, {12, 1, 128}, {16, 2, 64}};
        const auto& sh = shapes[rng() % 6];
        p.num_qo_heads = sh[0];
        p.num_kv_heads = sh[1];
        p.head_dim = sh[2];
        p.page_size = 16;
        p.dtype = int(rng() % 2);
        p.causal = int(rng() % 4 != 0);
        p.max_kv_splits = pick({0, 0, 1, 2, 5});
        p.num_cus = pick({0, 0, 4, 64, 2048});
        p.narrow_kernel = int(rng() % 3 == 0);
        p.kv_shared = int(rng() % 2);
        const int B = 1 + int(rng() % 40);
        std::vector<int32_t> qo(B + 1, 0), kp(B + 1, 0), kl(B, 1), newlen(B);
        for (int b = 0; b < B; ++b) {
            const int q = pick({0, 1, 1, 2, 5, 17, 33, 130, 300});
            const int extra = pick({0, 1, 15, 16, 255, 257, 1000, 4000});
            int kv = p.causal ? q + extra : (q ? 1 + extra : extra);
            if (rng() % 50 == 0) kv = 0;  // a sequence without pages (invalid if it has queries)
            qo[b + 1] = qo[b] + q;
            const int np = (kv + 15) / 16;
            kp[b + 1] = kp[b] + np;
            kl[b] = np ? (kv - 1) % 16 + 1 : 1;
            newlen[b] = kv ? int(rng() % (kv + 1)) : 0;
        }
        if (rng() % 25 == 0) kl[rng() % B] = 17;  // invalid last-page length
        rpa_plan* plan = nullptr;
        const int shared_pages = rng() % 3 == 0 ? int(rng() % 20) : 0;  // a declared common prefix
        const rpa_status st = shared_pages
                                  ? rpa_plan_create_shared(&p, B, qo.data(), kp.data(), kl.data(), shared_pages, &plan)
                                  : rpa_plan_create(&p, B, qo.data(), kp.data(), kl.data(), &plan);
        size_t bound = 0;
        const rpa_status bs = rpa_workspace_bytes(&p, B, qo[B], kp[B], &bound);
        CHECK(bs == RPA_OK);
        if (st != RPA_OK) {
            CHECK(plan == nullptr && rpa_last_error()[0] != 0);
            ++refused;
            continue;
        }
        ++plans;
        rpa_plan_info_t info{};
        CHECK(rpa_plan_info(plan, &info) == RPA_OK);
        CHECK(info.workspace_bytes <= bound);
        std::vector<int32_t> tiles(size_t(info.num_tiles) * 16 + 16);
        int64_t n = -1;
        CHECK(rpa_plan_tiles(plan, tiles.data(), info.num_tiles, &n) == RPA_OK && n == info.num_tiles);
        CHECK(rpa_plan_tiles(plan, tiles.data(), 1, &n) == RPA_OK);
        // one decode step: every sequence with pages one token longer
        std::vector<int32_t> kp2(B + 1, 0), kl2(B);
        for (int b = 0; b < B; ++b) {
            int np = kp[b + 1] - kp[b];
            int last = kl[b];
            if (np > 0 && last == 16) {
                ++np;
                last = 1;
            } else if (np > 0) {
                ++last;
            }
            kp2[b + 1] = kp2[b] + np;
            kl2[b] = last;
        }
        const rpa_status us = rpa_plan_update(plan, qo.data(), kp2.data(), kl2.data());
        CHECK(us == RPA_OK || us == RPA_E_UNSUPPORTED);
        CHECK(rpa_plan_info(plan, &info) == RPA_OK);
        // an unbound plan: run is refused before any HIP call; run_noalloc refuses only
        // by size here (a fitting plan would launch)
        CHECK(rpa_run(plan, &p, &p, &p, nullptr, nullptr) == RPA_E_ARG);
        if (info.workspace_bytes > (size_t(16) << 20)) {
            CHECK(rpa_run_noalloc(plan, kp.data(), 1, &p, &p, &p, nullptr, nullptr, nullptr) == RPA_E_WORKSPACE);
        }
        // page-table edits and checks on the host
        std::vector<int32_t> idx(kp[B] + 1), oip(B + 1), oix(kp[B] + 1), okl(B);
        for (int i = 0; i < kp[B]; ++i) idx[i] = int32_t(rng() % 100000);
        CHECK(rpa_trim_page_table(B, kp.data(), idx.data(), kl.data(), newlen.data(), oip.data(), oix.data(),
                                  okl.data()) == RPA_OK);
        CHECK(oip[B] <= kp[B]);
        const rpa_status vs = rpa_validate_page_table(B, kp.data(), idx.data(), 50000);
        CHECK(vs == RPA_OK || vs == RPA_E_PAGE_OOB);
        rpa_plan_destroy(plan);
    }
    // NULL and out-of-range arguments
    rpa_plan* plan = nullptr;
    CHECK(rpa_plan_create(nullptr, 0, nullptr, nullptr, nullptr, &plan) == RPA_E_ARG);
    rpa_params p{8, 1, 128, 16, 0, 1, 0.f, 0, 0, 0, 0};
    CHECK(rpa_plan_create(&p, -1, nullptr, nullptr, nullptr, &plan) != RPA_OK);
    size_t bytes = 0;
    CHECK(rpa_workspace_bytes(&p, 4, -1, 0, &bytes) == RPA_E_ARG);
    rpa_plan_destroy(nullptr);
    CHECK(g_hip_calls == 0);
    std::printf("planner fuzz: %lld plans, %lld refused, %d failures, %d HIP calls\n", (long long)plans,
                (long long)refused, failures, g_hip_calls);
    return failures == 0 ? 0 : 1;
}
