// rpa_api.cpp -- the C ABI declared in include/rpa.h: argument checks, plan
// lifecycle, schedule upload into the caller's workspace, kernel launches and
// error reporting.  Host code only; the kernels live in rpa_kernels.hip.
#include "rpa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "rpa_launch.h"
#include "rpa_schedule.h"


struct rpa_plan {
    rpa_params params{};
    int32_t batch = 0;
    int32_t shared_pages = 0;  // declared shared prefix (rpa_plan_create_shared)
    int32_t tail_skip = 1;     // RPA_DISABLE_TAIL_SKIP at create time, kept by update
    rpa::Schedule sched;
    rpa::WorkspaceLayout ws_layout{};  // byte offsets within the workspace
    // bound state
    const int32_t* page_idx_d = nullptr;
    int64_t num_pages = 0;
    char* ws = nullptr;
    void* staging = nullptr;  // pinned host image of the schedule
    size_t staging_bytes = 0;
    bool bound = false;
};

namespace {

thread_local std::string g_err;

rpa_status set_err(rpa_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

rpa_status hip_err(hipError_t e, const char* what) {
    return set_err(RPA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---- kernel timing (benchmarks only) ----
std::mutex g_prof_mu;
bool g_prof_on = false;
struct ProfEv { hipEvent_t a, b; int kind; };
std::vector<ProfEv> g_prof_events;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Test and measurement switches, read from the environment when a plan is created.
//   RPA_DISABLE_TAIL_SKIP=1  causal query tiles walk every key up to kv_len and mask
//                            the tail instead of skipping it: the same results, at the
//                            cost the skip saves (for A/B timing)
//   RPA_LOG=1                one line per created or updated plan on stderr
bool env_on(const char* name) {
    const char* v = std::getenv(name);
    return v && v[0] && std::strcmp(v, "0") != 0;
}

rpa::PlanParams plan_params(const rpa_params& P, int32_t shared_pages, int32_t tail_skip) {
    rpa::PlanParams pp{P.num_qo_heads, P.num_kv_heads, P.head_dim,      P.page_size,  P.causal,
                       P.max_kv_splits,  P.num_cus,      P.narrow_kernel, shared_pages};
    pp.tail_skip = tail_skip;
    return pp;
}

void log_plan(const char* what, const rpa_plan* plan) {
    if (!env_on("RPA_LOG")) return;
    const auto& S = plan->sched;
    std::fprintf(stderr,
                 "rpa: %s batch=%d total_q=%lld tiles=%zu (wide %lld, narrow %lld, group %lld%s) "
                 "split_groups=%zu max_splits=%d partial_rows=%lld workspace=%zu B tail_skip=%d\n",
                 what, plan->batch, (long long)S.total_q, S.tiles.size(), (long long)S.wide_tiles,
                 (long long)S.narrow_tiles, (long long)S.group_tiles, S.fused ? ", one mixed launch" : "",
                 S.merges.size(), S.max_splits, (long long)S.partial_rows, plan->ws_layout.bytes, plan->tail_skip);
}

// The schedule's part of a workspace image: tile records and the sequence table (the
// counters and error word after them stay zero).
void write_image(const rpa_plan* plan, char* img) {
    const auto& S = plan->sched;
    if (!S.tiles.empty())
        std::memcpy(img + plan->ws_layout.off_tiles, S.tiles.data(), S.tiles.size() * sizeof(rpa::Tile));
    if (!S.seqtab.empty())
        std::memcpy(img + plan->ws_layout.off_seqtab, S.seqtab.data(), S.seqtab.size() * sizeof(int32_t));
}

// Enqueue the plan's attention kernels over a workspace image at `ws` (tiles, split
// counters and partials at the offsets of plan->ws_layout); error bits go to err_flag.
rpa_status launch_plan(const rpa_plan* plan, char* ws, const int32_t* page_idx, int64_t num_pages, int32_t* err_flag,
                       const void* q, const void* kv_cache, void* o, float* lse, hipStream_t st) {
    const auto& S = plan->sched;
    const rpa_params& P = plan->params;
    const float scale = P.sm_scale > 0.f ? P.sm_scale : 1.f / std::sqrt(float(P.head_dim));
    rpa::LaunchAttn L{};
    const rpa::WorkspaceLayout& WL = plan->ws_layout;
    L.a.tiles = reinterpret_cast<const rpa::Tile*>(ws + WL.off_tiles);
    L.a.page_idx = page_idx;
    L.a.num_pages = int32_t(num_pages);
    L.a.q = static_cast<const uint16_t*>(q);
    L.a.kv = static_cast<const uint16_t*>(kv_cache);
    L.a.o = static_cast<uint16_t*>(o);
    L.a.lse = lse;
    L.a.part_o = reinterpret_cast<float*>(ws + WL.off_part_o);
    L.a.part_lse = reinterpret_cast<float*>(ws + WL.off_part_lse);
    L.a.H = P.num_qo_heads;
    L.a.Hkv = P.num_kv_heads;
    L.a.G = P.num_qo_heads / P.num_kv_heads;
    L.a.c_log2 = float(double(scale) * 1.4426950408889634);
    L.a.causal = P.causal;
    L.a.err_flag = err_flag;
    L.a.counters = reinterpret_cast<int32_t*>(ws + WL.off_counters);
    L.a.seqtab = reinterpret_cast<const int32_t*>(ws + WL.off_seqtab);
    L.head_dim = P.head_dim;
    L.bf16 = P.dtype == RPA_BF16;
    L.n_tiles = int64_t(S.tiles.size());

    // One kernel for the wide tiles (tiles[0, wide)), one for the narrow tiles after them,
    // or, for a plan with both kinds, one mixed kernel over the interleaved tiles.
    // Profiling: an event pair stamped by each dispatch itself (start and end of the kernel).
    const bool prof = g_prof_on;
    ProfEv e0{nullptr, nullptr, 0}, e1{nullptr, nullptr, 1};
    hipError_t e = hipSuccess;
    // Split key ranges put each narrow tile's last step on the latency-critical path of
    // the merge, where the extra LDS round trip of row-wise K loads costs more than their
    // better coalescing gains; unsplit (many-tile) decode is throughput-bound.
    L.k_rows = !S.narrow_split;
    // Pages read by one sequence only are streamed past L2 (non-temporal), which keeps the
    // schedule, page indices and Q resident; shared pages stay cached.
    L.kv_stream = P.kv_shared == 0;
    L.group = S.group_tiles > 0;
    if (S.fused) {  // wide and narrow tiles interleaved in one launch (timed as "wide")
        if (prof) {
            e0.a = prof_event();
            e0.b = prof_event();
        }
        e = rpa::launch_mixed(L, st, e0.a, e0.b);
        if (e != hipSuccess) return hip_err(e, "mixed attention kernel launch");
    } else if (S.wide_tiles > 0) {
        if (prof) {
            e0.a = prof_event();
            e0.b = prof_event();
        }
        L.n_tiles = S.wide_tiles;
        e = rpa::launch_wide(L, st, e0.a, e0.b);
        if (e != hipSuccess) return hip_err(e, "wide attention kernel launch");
    }
    if (!S.fused && S.narrow_tiles > 0) {
        if (prof) {
            e1.a = prof_event();
            e1.b = prof_event();
        }
        rpa::LaunchAttn N = L;
        N.a.tiles = L.a.tiles + S.wide_tiles;
        N.n_tiles = S.narrow_tiles;
        e = P.narrow_kernel == 1 ? rpa::launch_narrow_valu(N, S.narrow_max_rows, st, e1.a, e1.b)
                                 : rpa::launch_narrow(N, st, e1.a, e1.b);
        if (e != hipSuccess) return hip_err(e, "narrow attention kernel launch");
    }
    if (prof) {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (e0.a && e0.b) g_prof_events.push_back(e0);
        if (e1.a && e1.b) g_prof_events.push_back(e1);
    }
    return RPA_OK;
}

}  // namespace

extern "C" {

const char* rpa_last_error(void) { return g_err.c_str(); }

const char* rpa_version(void) { return "0.1.0"; }

rpa_status rpa_plan_create(const rpa_params* params, int32_t batch, const int32_t* qo_indptr_h,
                           const int32_t* kv_page_indptr_h, const int32_t* kv_last_page_len_h,
                           rpa_plan** out) {
    return rpa_plan_create_shared(params, batch, qo_indptr_h, kv_page_indptr_h, kv_last_page_len_h, 0, out);
}

rpa_status rpa_plan_create_shared(const rpa_params* params, int32_t batch, const int32_t* qo_indptr_h,
                                  const int32_t* kv_page_indptr_h, const int32_t* kv_last_page_len_h,
                                  int32_t shared_pages, rpa_plan** out) {
    if (!params || !out) return set_err(RPA_E_ARG, "params and out must be non-NULL");
    *out = nullptr;
    if (params->dtype != RPA_F16 && params->dtype != RPA_BF16)
        return set_err(RPA_E_ARG, "dtype must be RPA_F16 (0) or RPA_BF16 (1)");
    if (params->causal != 0 && params->causal != 1) return set_err(RPA_E_ARG, "causal must be 0 or 1");
    if (!std::isfinite(params->sm_scale)) return set_err(RPA_E_ARG, "sm_scale must be finite");
    if (params->narrow_kernel != 0 && params->narrow_kernel != 1)
        return set_err(RPA_E_ARG, "narrow_kernel must be 0 (MFMA) or 1 (VALU)");
    if (params->kv_shared != 0 && params->kv_shared != 1) return set_err(RPA_E_ARG, "kv_shared must be 0 or 1");
    if (shared_pages < 0) return set_err(RPA_E_ARG, "shared_pages must be >= 0");
    const int32_t tail_skip = env_on("RPA_DISABLE_TAIL_SKIP") ? 0 : 1;
    const rpa::PlanParams pp = plan_params(*params, shared_pages, tail_skip);
    rpa_plan* plan = new (std::nothrow) rpa_plan();
    if (!plan) return set_err(RPA_E_ARG, "out of host memory");
    std::string err;
    int rc = 0;
    try {
        rc = rpa::build_schedule(pp, batch, qo_indptr_h, kv_page_indptr_h, kv_last_page_len_h, &plan->sched, &err);
    } catch (const std::bad_alloc&) {
        rc = RPA_E_ARG;
        err = "out of host memory while planning";
    }
    if (rc != 0) {
        delete plan;
        return set_err(rpa_status(rc), err);
    }
    plan->params = *params;
    plan->batch = batch;
    plan->shared_pages = shared_pages;
    plan->tail_skip = tail_skip;
    const auto& S = plan->sched;
    plan->ws_layout = rpa::workspace_layout(int64_t(S.tiles.size()), int64_t(S.seqtab.size()),
                                            int64_t(S.merges.size()), S.partial_rows, params->head_dim);
    plan->staging_bytes = plan->ws_layout.off_part_lse;  // tiles, then the zeroed counters and error word
    log_plan("create", plan);
    *out = plan;
    return RPA_OK;
}

rpa_status rpa_plan_info(const rpa_plan* plan, rpa_plan_info_t* out) {
    if (!plan || !out) return set_err(RPA_E_ARG, "plan and out must be non-NULL");
    const auto& S = plan->sched;
    out->num_tiles = int64_t(S.tiles.size());
    out->num_split_groups = int64_t(S.merges.size());
    out->max_splits = S.max_splits;
    out->block_m = S.block_m;
    out->block_n = S.block_n;
    out->tokens_per_tile = S.tokens_per_tile;
    out->partial_rows = S.partial_rows;
    out->workspace_bytes = plan->ws_layout.bytes;
    out->total_q = S.total_q;
    out->visible_pairs = S.visible_pairs;
    out->kv_tokens = S.kv_tokens;
    return RPA_OK;
}

rpa_status rpa_workspace_bytes(const rpa_params* params, int32_t batch, int64_t total_q, int64_t total_pages,
                               size_t* bytes_out) {
    if (!params || !bytes_out) return set_err(RPA_E_ARG, "params and bytes_out must be non-NULL");
    *bytes_out = 0;
    const rpa::PlanParams pp = plan_params(*params, 0, 1);
    rpa::ScheduleBound B{};
    std::string err;
    const int rc = rpa::schedule_bound(pp, batch, total_q, total_pages, &B, &err);
    if (rc != 0) return set_err(rpa_status(rc), err);
    *bytes_out = rpa::workspace_layout(B.tiles, B.seqtab, B.merges, B.partial_rows, params->head_dim).bytes;
    return RPA_OK;
}

rpa_status rpa_plan_tiles(const rpa_plan* plan, int32_t* out_h, int64_t cap, int64_t* n_out) {
    if (!plan || !n_out || cap < 0 || (cap > 0 && !out_h))
        return set_err(RPA_E_ARG, "plan and n_out must be non-NULL, cap >= 0");
    const auto& tiles = plan->sched.tiles;
    *n_out = int64_t(tiles.size());
    const int64_t n = std::min<int64_t>(cap, int64_t(tiles.size()));
    if (n > 0) std::memcpy(out_h, tiles.data(), size_t(n) * sizeof(rpa::Tile));
    return RPA_OK;
}

rpa_status rpa_plan_bind(rpa_plan* plan, const int32_t* kv_page_indices_d, int64_t num_pages, void* workspace_d,
                         size_t workspace_bytes, void* stream) {
    if (!plan) return set_err(RPA_E_ARG, "plan must be non-NULL");
    const auto& S = plan->sched;
    if (num_pages < 0 || num_pages > INT32_MAX) return set_err(RPA_E_ARG, "num_pages outside [0, 2^31)");
    if (!S.tiles.empty() && !kv_page_indices_d) return set_err(RPA_E_ARG, "kv_page_indices must be non-NULL");
    if (!S.tiles.empty() && num_pages < 1) return set_err(RPA_E_ARG, "num_pages must be >= 1 for a non-empty batch");
    if (!workspace_d) return set_err(RPA_E_ARG, "workspace must be non-NULL");
    if (reinterpret_cast<uintptr_t>(workspace_d) % 256 != 0)
        return set_err(RPA_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < plan->ws_layout.bytes) {
        char buf[160];
        std::snprintf(buf, sizeof(buf), "workspace of %zu bytes is too small: this plan needs %zu bytes",
                      workspace_bytes, plan->ws_layout.bytes);
        return set_err(RPA_E_WORKSPACE, buf);
    }
    if (!plan->staging) {
        hipError_t e = hipHostMalloc(&plan->staging, plan->staging_bytes, hipHostMallocDefault);
        if (e != hipSuccess) {
            plan->staging = nullptr;
            return hip_err(e, "hipHostMalloc(schedule staging)");
        }
        std::memset(plan->staging, 0, plan->staging_bytes);
        write_image(plan, static_cast<char*>(plan->staging));
    }
    hipError_t e = hipMemcpyAsync(workspace_d, plan->staging, plan->staging_bytes, hipMemcpyHostToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(schedule upload)");
    plan->page_idx_d = kv_page_indices_d;
    plan->num_pages = num_pages;
    plan->ws = static_cast<char*>(workspace_d);
    plan->bound = true;
    return RPA_OK;
}

rpa_status rpa_plan_update(rpa_plan* plan, const int32_t* qo_indptr_h, const int32_t* kv_page_indptr_h,
                           const int32_t* kv_last_page_len_h) {
    if (!plan) return set_err(RPA_E_ARG, "plan must be non-NULL");
    const rpa_params& P = plan->params;
    const rpa::PlanParams pp = plan_params(P, plan->shared_pages, plan->tail_skip);
    rpa::Schedule S;
    std::string err;
    int rc = 0;
    try {
        rc = rpa::build_schedule(pp, plan->batch, qo_indptr_h, kv_page_indptr_h, kv_last_page_len_h, &S, &err);
    } catch (const std::bad_alloc&) {
        return set_err(RPA_E_ARG, "out of host memory while planning");
    }
    if (rc != 0) return set_err(rpa_status(rc), err);
    const auto& O = plan->sched;
    // The launch a captured graph replays was configured from the old schedule: the
    // grid (tile counts), the kernel (wide / narrow / mixed, K loads for split narrow
    // tiles) and, on the VALU kernel, its row capacity.  All must stay.
    auto valu_rows = [](int32_t r) { return r <= 2 ? 2 : r <= 4 ? 4 : 8; };
    const bool same_kernel = S.narrow_split == O.narrow_split && S.group_tiles == O.group_tiles &&
                             (P.narrow_kernel != 1 || S.narrow_tiles == 0 ||
                              valu_rows(S.narrow_max_rows) == valu_rows(O.narrow_max_rows));
    if (S.tiles.size() != O.tiles.size() || S.wide_tiles != O.wide_tiles || S.fused != O.fused ||
        S.narrow_tiles != O.narrow_tiles || S.merges.size() != O.merges.size() || !same_kernel ||
        S.partial_rows > O.partial_rows)
        return set_err(RPA_E_UNSUPPORTED,
                       "the new lengths need another launch shape (" + std::to_string(S.tiles.size()) + " tiles, " +
                           std::to_string(S.merges.size()) + " split groups instead of " +
                           std::to_string(O.tiles.size()) + ", " + std::to_string(O.merges.size()) +
                           (same_kernel ? "" : "; another kernel configuration") +
                           "): create and bind a new plan");
    S.partial_rows = O.partial_rows;  // the workspace layout stays as bound
    std::swap(plan->sched, S);
    rpa::recycle_schedule(&S);  // the previous schedule's buffers serve the next update
    if (plan->staging) write_image(plan, static_cast<char*>(plan->staging));
    log_plan("update", plan);
    return RPA_OK;
}

rpa_status rpa_plan_upload(const rpa_plan* plan, void* stream) {
    if (!plan) return set_err(RPA_E_ARG, "plan must be non-NULL");
    if (!plan->bound) return set_err(RPA_E_ARG, "plan is not bound to a workspace (rpa_plan_bind)");
    // tiles and zeroed split counters; the error word after them is left as it is
    hipError_t e = hipMemcpyAsync(plan->ws, plan->staging, plan->ws_layout.off_flags, hipMemcpyHostToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(schedule upload)");
    return RPA_OK;
}

rpa_status rpa_run(const rpa_plan* plan, const void* q, const void* kv_cache, void* o, float* lse, void* stream) {
    if (!plan) return set_err(RPA_E_ARG, "plan must be non-NULL");
    if (!plan->bound) return set_err(RPA_E_ARG, "plan is not bound to a workspace (rpa_plan_bind)");
    if (plan->sched.tiles.empty()) return RPA_OK;
    if (!q || !kv_cache || !o) return set_err(RPA_E_ARG, "q, kv_cache and o must be non-NULL");
    return launch_plan(plan, plan->ws, plan->page_idx_d, plan->num_pages,
                       reinterpret_cast<int32_t*>(plan->ws + plan->ws_layout.off_flags), q, kv_cache, o, lse,
                       static_cast<hipStream_t>(stream));
}

rpa_status rpa_run_noalloc(const rpa_plan* plan, const int32_t* kv_page_indices_d, int64_t num_pages, const void* q,
                           const void* kv_cache, void* o, float* lse, int32_t* err_flag_d, void* stream) {
    if (!plan) return set_err(RPA_E_ARG, "plan must be non-NULL");
    const auto& S = plan->sched;
    const rpa::WorkspaceLayout& WL = plan->ws_layout;
    // size first: a plan too large for the static scratch is refused before any HIP call
    if (WL.bytes > rpa::kStaticScratchBytes) {
        char buf[200];
        std::snprintf(buf, sizeof(buf),
                      "this plan needs %zu bytes of scratch; rpa_run_noalloc has %zu: use rpa_plan_bind and "
                      "rpa_run with a workspace", WL.bytes, size_t(rpa::kStaticScratchBytes));
        return set_err(RPA_E_WORKSPACE, buf);
    }
    if (num_pages < 0 || num_pages > INT32_MAX) return set_err(RPA_E_ARG, "num_pages outside [0, 2^31)");
    if (S.tiles.empty()) return RPA_OK;
    if (!kv_page_indices_d) return set_err(RPA_E_ARG, "kv_page_indices must be non-NULL");
    if (num_pages < 1) return set_err(RPA_E_ARG, "num_pages must be >= 1 for a non-empty batch");
    if (!q || !kv_cache || !o) return set_err(RPA_E_ARG, "q, kv_cache and o must be non-NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* scratch = nullptr;
    hipError_t e = rpa::static_scratch(&scratch);
    if (e != hipSuccess) return hip_err(e, "locating the static scratch (hipGetSymbolAddress)");
    char* ws = static_cast<char*>(scratch);
    // the schedule, from the plan's host memory; then counters and error word cleared by a
    // kernel (what the previous call left there is not zero)
    e = hipMemcpyAsync(ws + WL.off_tiles, S.tiles.data(), S.tiles.size() * sizeof(rpa::Tile),
                       hipMemcpyHostToDevice, st);
    if (e == hipSuccess && !S.seqtab.empty())
        e = hipMemcpyAsync(ws + WL.off_seqtab, S.seqtab.data(), S.seqtab.size() * sizeof(int32_t),
                           hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(schedule into the static scratch)");
    int32_t* cleared = reinterpret_cast<int32_t*>(ws + WL.off_counters);
    e = rpa::launch_clear(cleared, int64_t((WL.off_part_lse - WL.off_counters) / sizeof(int32_t)), st);
    if (e != hipSuccess) return hip_err(e, "clear kernel launch");
    int32_t* flag = err_flag_d ? err_flag_d : reinterpret_cast<int32_t*>(ws + WL.off_flags);
    return launch_plan(plan, ws, kv_page_indices_d, num_pages, flag, q, kv_cache, o, lse, st);
}

rpa_status rpa_plan_check(const rpa_plan* plan, void* stream, int32_t* flag_out) {
    if (!plan || !flag_out) return set_err(RPA_E_ARG, "plan and flag_out must be non-NULL");
    if (!plan->bound) return set_err(RPA_E_ARG, "plan is not bound");
    int32_t flag = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* word = plan->ws + plan->ws_layout.off_flags;
    hipError_t e = hipMemcpyAsync(&flag, word, sizeof(flag), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess && flag != 0) {  // read and clear: the next check covers later runs
        static const int32_t zero = 0;
        e = hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
    }
    if (e != hipSuccess) return hip_err(e, "reading the error flag");
    *flag_out = flag;
    if (flag & rpa::kErrPage)
        return set_err(RPA_E_PAGE_OOB, "a page index outside [0, num_pages) was met; its keys read as zero");
    if (flag & rpa::kErrVRange)
        return set_err(RPA_E_V_RANGE, "a bf16 V value above 65504 (the largest fp16 value) was met; the P V "
                                      "product saturated it, so the rows that read it are wrong");
    return RPA_OK;
}

void rpa_plan_destroy(rpa_plan* plan) {
    if (!plan) return;
    if (plan->staging) (void)hipHostFree(plan->staging);
    delete plan;
}

rpa_status rpa_validate_page_table(int32_t batch, const int32_t* kv_page_indptr_h, const int32_t* kv_page_indices_h,
                                   int64_t num_pages) {
    if (batch < 0 || (batch > 0 && !kv_page_indptr_h)) return set_err(RPA_E_ARG, "bad batch or NULL indptr");
    if (batch > 0 && kv_page_indptr_h[0] != 0) return set_err(RPA_E_INDPTR, "kv_page_indptr[0] must be 0");
    for (int32_t b = 0; b < batch; ++b) {
        if (kv_page_indptr_h[b + 1] < kv_page_indptr_h[b])
            return set_err(RPA_E_INDPTR, "kv_page_indptr decreases at " + std::to_string(b));
    }
    const int32_t nnz = batch > 0 ? kv_page_indptr_h[batch] : 0;
    if (nnz > 0 && !kv_page_indices_h) return set_err(RPA_E_ARG, "kv_page_indices must be non-NULL");
    for (int32_t i = 0; i < nnz; ++i)
        if (kv_page_indices_h[i] < 0 || kv_page_indices_h[i] >= num_pages)
            return set_err(RPA_E_PAGE_OOB, "kv_page_indices[" + std::to_string(i) + "] = " +
                                               std::to_string(kv_page_indices_h[i]) + " outside [0, " +
                                               std::to_string(num_pages) + ")");
    return RPA_OK;
}

rpa_status rpa_append_kv(int32_t batch, int64_t n_new, int32_t num_kv_heads, int32_t head_dim,
                         const int32_t* append_indptr_d, const int32_t* kv_page_indptr_d,
                         const int32_t* kv_page_indices_d, const int32_t* kv_last_page_len_d, const void* new_kv_d,
                         void* kv_cache_d, int64_t num_pages, int32_t* err_flag_d, void* stream) {
    if (batch < 0 || n_new < 0) return set_err(RPA_E_ARG, "batch and n_new must be >= 0");
    if (num_kv_heads < 1) return set_err(RPA_E_SHAPE, "num_kv_heads must be >= 1");
    if (head_dim != 64 && head_dim != 128)
        return set_err(RPA_E_SHAPE, "head_dim " + std::to_string(head_dim) + " not supported (64 or 128)");
    if (num_pages < 0 || num_pages > INT32_MAX) return set_err(RPA_E_ARG, "num_pages outside [0, 2^31)");
    if (n_new == 0) return RPA_OK;
    if (batch == 0) return set_err(RPA_E_ARG, "new tokens need at least one sequence");
    if (n_new > INT32_MAX) return set_err(RPA_E_ARG, "too many new tokens");
    if (!append_indptr_d || !kv_page_indptr_d || !kv_page_indices_d || !kv_last_page_len_d || !new_kv_d ||
        !kv_cache_d)
        return set_err(RPA_E_ARG, "device arrays must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(new_kv_d) | reinterpret_cast<uintptr_t>(kv_cache_d)) & 15)
        return set_err(RPA_E_ARG, "new_kv and kv_cache must be 16-byte aligned");
    rpa::AppendArgs A{};
    A.append_indptr = append_indptr_d;
    A.kv_page_indptr = kv_page_indptr_d;
    A.kv_page_indices = kv_page_indices_d;
    A.kv_last_page_len = kv_last_page_len_d;
    A.new_kv = static_cast<const uint16_t*>(new_kv_d);
    A.kv = static_cast<uint16_t*>(kv_cache_d);
    A.n_new = n_new;
    A.batch = batch;
    A.Hkv = num_kv_heads;
    A.D = head_dim;
    A.num_pages = int32_t(num_pages);
    A.err_flag = err_flag_d;
    const hipError_t e = rpa::launch_append(A, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_err(e, "append kernel launch");
    return RPA_OK;
}

rpa_status rpa_trim_page_table(int32_t batch, const int32_t* kv_page_indptr_h, const int32_t* kv_page_indices_h,
                               const int32_t* kv_last_page_len_h, const int32_t* new_kv_len_h,
                               int32_t* out_kv_page_indptr_h, int32_t* out_kv_page_indices_h,
                               int32_t* out_kv_last_page_len_h) {
    if (batch < 0) return set_err(RPA_E_ARG, "batch must be >= 0");
    if (batch > 0 && (!kv_page_indptr_h || !kv_last_page_len_h || !new_kv_len_h || !out_kv_page_indptr_h ||
                      !out_kv_last_page_len_h))
        return set_err(RPA_E_ARG, "host arrays must be non-NULL");
    if (out_kv_page_indptr_h && batch >= 0) out_kv_page_indptr_h[0] = 0;
    if (batch == 0) return RPA_OK;
    if (kv_page_indptr_h[0] != 0) return set_err(RPA_E_INDPTR, "kv_page_indptr[0] must be 0");
    if (kv_page_indptr_h[batch] > 0 && (!kv_page_indices_h || !out_kv_page_indices_h))
        return set_err(RPA_E_ARG, "kv_page_indices and out_kv_page_indices must be non-NULL");
    const int P = rpa::kPageSize;
    int32_t w = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t np = kv_page_indptr_h[b + 1] - kv_page_indptr_h[b];
        if (np < 0) return set_err(RPA_E_INDPTR, "kv_page_indptr decreases at " + std::to_string(b));
        if (np > 0 && (kv_last_page_len_h[b] < 1 || kv_last_page_len_h[b] > P))
            return set_err(RPA_E_LAST_PAGE_LEN, "kv_last_page_len[" + std::to_string(b) + "] outside [1, 16]");
        const int64_t kv_len = np == 0 ? 0 : int64_t(np - 1) * P + kv_last_page_len_h[b];
        const int32_t nl = new_kv_len_h[b];
        if (nl < 0 || nl > kv_len)
            return set_err(RPA_E_ARG, "new_kv_len[" + std::to_string(b) + "] = " + std::to_string(nl) +
                                          " outside [0, " + std::to_string(kv_len) + "]");
        const int32_t keep = (nl + P - 1) / P;
        for (int32_t i = 0; i < keep; ++i) out_kv_page_indices_h[w + i] = kv_page_indices_h[kv_page_indptr_h[b] + i];
        w += keep;
        out_kv_page_indptr_h[b + 1] = w;
        out_kv_last_page_len_h[b] = nl == 0 ? 0 : (nl - 1) % P + 1;
    }
    return RPA_OK;
}

rpa_status rpa_merge_states(int64_t rows, int32_t num_heads, int32_t head_dim, int32_t dtype, const void* o_a,
                            const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                            void* stream) {
    if (rows < 0 || num_heads < 1) return set_err(RPA_E_ARG, "rows must be >= 0 and num_heads >= 1");
    if (head_dim != 64 && head_dim != 128)
        return set_err(RPA_E_SHAPE, "head_dim " + std::to_string(head_dim) + " not supported (64 or 128)");
    if (dtype != RPA_F16 && dtype != RPA_BF16) return set_err(RPA_E_ARG, "dtype must be RPA_F16 or RPA_BF16");
    if (rows == 0) return RPA_OK;
    if (!o_a || !lse_a || !o_b || !lse_b || !o)
        return set_err(RPA_E_ARG, "o_a, lse_a, o_b, lse_b and o must be non-NULL");
    auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
    if (misaligned(o_a) || misaligned(o_b) || misaligned(o))
        return set_err(RPA_E_ARG, "o_a, o_b and o must be 16-byte aligned");
    rpa::MergeArgs M{};
    M.o_a = static_cast<const uint16_t*>(o_a);
    M.lse_a = lse_a;
    M.o_b = static_cast<const uint16_t*>(o_b);
    M.lse_b = lse_b;
    M.o = static_cast<uint16_t*>(o);
    M.lse = lse;
    M.items = rows * num_heads * (head_dim / 8);
    M.head_dim = head_dim;
    const hipError_t e = rpa::launch_merge(M, dtype == RPA_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_err(e, "merge kernel launch");
    return RPA_OK;
}

rpa_status rpa_prof_start(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = true;
    return RPA_OK;
}

rpa_status rpa_prof_stop(int64_t counts_out[2], double ms_out[2]) {
    std::vector<ProfEv> evs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof_on = false;
        evs.swap(g_prof_events);
    }
    if (counts_out) counts_out[0] = counts_out[1] = 0;
    if (ms_out) ms_out[0] = ms_out[1] = 0.0;
    rpa_status st = RPA_OK;
    for (auto& ev : evs) {
        hipError_t e = hipEventSynchronize(ev.b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev.a, ev.b);
        if (e != hipSuccess) st = hip_err(e, "kernel timing event");
        else {
            if (counts_out) counts_out[ev.kind] += 1;
            if (ms_out) ms_out[ev.kind] += ms;
        }
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof_pool.push_back(ev.a);
        g_prof_pool.push_back(ev.b);
    }
    return st;
}

}  // extern "C"
