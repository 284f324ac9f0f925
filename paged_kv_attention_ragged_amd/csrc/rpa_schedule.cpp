// rpa_schedule.cpp -- host planner: ragged lengths in, work tiles and the
// split-KV schedule out.  Plain C++17, no HIP: it builds and runs anywhere.
//
// The plan is the host half of the pages' begin_forward (flashinfer issue
// #323, "How are prefill and decode kernels different?": auxiliary data built
// once per batch and reused by every forward call).  It depends only on the
// lengths, never on page ids, so two batches with equal lengths get the same
// schedule and therefore the same rounding.
#include "rpa_schedule.h"

#include <algorithm>
#include <cstdio>
#include <map>
#include <numeric>

namespace rpa {
namespace {

enum { OK = 0, E_ARG = 1, E_SHAPE = 2, E_INDPTR = 3, E_LAST_PAGE_LEN = 4, E_QLEN_GT_KVLEN = 5 };

int fail(std::string* err, int code, const char* fmt, long a = 0, long b = 0, long c = 0) {
    char buf[256];
    std::snprintf(buf, sizeof(buf), fmt, a, b, c);
    if (err) *err = buf;
    return code;
}

struct QTile {
    int32_t seq, kv_head, q_row0, q_count, pos0, kv_len, page_base, kv_end, kind;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Piece { Tile t; int64_t cost; };

// Wide tiles re-read the keys of their (sequence, kv head) -- a "stream" -- once per
// query tile, so they are ordered for the L2 caches: workgroup i of a launch runs on
// XCD i % kXcds, and each XCD has its own L2.  Streams are laid out one after the
// other (largest total cost first; within a stream, longest tile first) and the
// list is cut into kXcds runs of about equal cost; run x fills the launch slots
// x, x + kXcds, x + 2 kXcds, ...  An XCD thus works through few streams at a time,
// and concurrent tiles of a stream share its K/V blocks in that XCD's L2.  Runs are
// padded with empty tiles (q_count 0: the kernel returns at once) so that every
// tile lands on its run's XCD.  Small launches keep plain longest-first order.
void order_wide_for_xcds(std::vector<Piece>& wide) {
    auto lpt = [](const Piece& a, const Piece& b) { return a.cost > b.cost; };
    if (wide.size() < size_t(4 * kXcds)) {
        std::stable_sort(wide.begin(), wide.end(), lpt);
        return;
    }
    std::map<std::pair<int32_t, int32_t>, int64_t> stream_cost;
    int64_t total = 0;
    for (const auto& pc : wide) {
        stream_cost[{pc.t.seq, pc.t.kv_head}] += pc.cost;
        total += pc.cost;
    }
    std::stable_sort(wide.begin(), wide.end(), [&](const Piece& a, const Piece& b) {
        const auto ka = std::make_pair(a.t.seq, a.t.kv_head), kb = std::make_pair(b.t.seq, b.t.kv_head);
        if (ka != kb) {
            const int64_t ca = stream_cost[ka], cb = stream_cost[kb];
            return ca != cb ? ca > cb : ka < kb;
        }
        return a.cost > b.cost;
    });
    std::vector<std::vector<Piece>> run(kXcds);
    int64_t acc = 0;
    for (const auto& pc : wide) {
        // the run whose share of the total cost holds this tile's midpoint
        const int64_t mid = acc + pc.cost / 2;
        const int x = int(std::min<int64_t>(kXcds - 1, mid * kXcds / std::max<int64_t>(total, 1)));
        run[x].push_back(pc);
        acc += pc.cost;
    }
    size_t len = 0;
    for (const auto& r : run) len = std::max(len, r.size());
    Piece empty{};
    empty.t.kind = kWide;
    empty.t.part = -1;
    empty.t.group = -1;
    empty.t.seq = -1;
    empty.t.n_splits = 1;
    std::vector<Piece> out;
    out.reserve(len * kXcds);
    for (size_t k = 0; k < len; ++k)
        for (int x = 0; x < kXcds; ++x) out.push_back(k < run[x].size() ? run[x][k] : empty);
    while (!out.empty() && out.back().t.q_count == 0) out.pop_back();  // not launched
    wide.swap(out);
}

// Work vectors of the calling thread, kept between calls: a plan is rebuilt for every
// decode step (rpa_plan_update), and fresh multi-page buffers each time would cost more
// in page faults than the planning itself.
// (build_schedule binds them to references once per call: in the shared library each
// access to a thread_local goes through the TLS lookup call.)
thread_local Schedule t_sched;
thread_local std::vector<QTile> t_base;
thread_local std::vector<Piece> t_wide, t_narrow, t_group;
thread_local std::vector<std::pair<int32_t, int32_t>> t_elig;  // (sequence, kv_len) of groupable decode rows

}  // namespace

namespace {
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

WorkspaceLayout workspace_layout(int64_t tiles, int64_t seqtab_entries, int64_t merges, int64_t partial_rows,
                                 int head_dim) {
    WorkspaceLayout L{};
    L.off_tiles = 0;
    L.off_seqtab = align256(size_t(tiles) * sizeof(Tile));
    L.off_counters = L.off_seqtab + align256(size_t(seqtab_entries) * sizeof(int32_t));
    L.off_flags = L.off_counters + align256(size_t(merges) * sizeof(int32_t));
    L.off_part_lse = L.off_flags + 256;
    L.off_part_o = L.off_part_lse + align256(size_t(partial_rows) * sizeof(float));
    L.bytes = L.off_part_o + align256(size_t(partial_rows) * size_t(head_dim) * sizeof(float));
    return L;
}

// Bounds (see build_schedule for the rules they follow):
//  * query tiles: sequence b has ceil(q_b / TQ) <= floor(q_b / TQ) + 1 of them per kv
//    head, and at most min(batch, total_q) sequences have queries, so there are at
//    most H_kv (floor(total_q / TQ) + min(batch, total_q));
//  * key ranges are split only when the query tiles number fewer than the target, at
//    most 2 N (N compute units).  The piece size C is then 256 keys if that gives fewer
//    pieces than the target, else the largest multiple of 256 still giving at least the
//    target; since ceil(k / C) <= 2 ceil(k / (C + 256)) for C >= 256, that is fewer
//    than twice the target, so fewer than 4 N pieces (the bound below takes 2 N).
//    Pieces therefore number at most max(query tiles, 4 N - 1), split groups fewer
//    than 2 N, and partial rows at most (pieces) x (rows of the largest tile);
//  * XCD padding lays the wide tiles out in 8 runs padded to the longest, so the launch
//    has at most 8 slots per piece.
int schedule_bound(const PlanParams& p, int32_t batch, int64_t total_q, int64_t total_pages, ScheduleBound* out,
                   std::string* err) {
    if (!out || batch < 0 || total_q < 0 || total_pages < 0)
        return fail(err, E_ARG, "batch, total_q and total_pages must be >= 0 and out non-NULL");
    if (p.num_qo_heads < 1 || p.num_kv_heads < 1 || p.num_qo_heads % p.num_kv_heads != 0)
        return fail(err, E_SHAPE, "num_qo_heads (%ld) must be a positive multiple of num_kv_heads (%ld)",
                    p.num_qo_heads, p.num_kv_heads);
    if (p.head_dim != 64 && p.head_dim != 128)
        return fail(err, E_SHAPE, "head_dim %ld not supported (64 or 128)", p.head_dim);
    if (p.page_size != kPageSize) return fail(err, E_SHAPE, "page_size %ld not supported (16)", p.page_size);
    const int32_t G = p.num_qo_heads / p.num_kv_heads;
    if (G > kMaxGroup) return fail(err, E_SHAPE, "query group %ld exceeds %ld heads per kv head", G, kMaxGroup);
    if (p.max_kv_splits < 0) return fail(err, E_ARG, "max_kv_splits must be >= 0");
    const int64_t TQ = block_m_for(p.head_dim) / G;
    const int64_t seqs = std::min<int64_t>(batch, total_q);
    const int64_t base = int64_t(p.num_kv_heads) * (total_q / TQ + seqs);
    const int64_t n_cus = p.num_cus > 0 ? p.num_cus : 256;
    const int64_t target = 2 * n_cus;
    // no sequence has more than 16 total_pages keys, so no tile more than this many pieces
    const int64_t max_chunks = (total_pages * kPageSize + kChunkKeys - 1) / kChunkKeys;
    int64_t pieces = base, merges = 0, partial = 0;
    if (p.max_kv_splits != 1 && base > 0 && max_chunks > 1) {
        const int64_t split_tiles = std::min(base, target - 1);  // query tiles of a split plan
        int64_t per_tile = max_chunks;
        if (p.max_kv_splits > 1) per_tile = std::min<int64_t>(per_tile, p.max_kv_splits);
        const int64_t split_pieces = std::min(2 * target - 1, split_tiles * per_tile);
        pieces = std::max(base, split_pieces);
        merges = split_tiles;
        const int64_t max_rows = std::min<int64_t>(block_m_for(p.head_dim), G * std::min(total_q, TQ));
        partial = split_pieces * max_rows;
    }
    out->tiles = kXcds * pieces;
    // kGroup tiles replace at least two narrow tiles each (the counts above hold), and
    // their sequence table holds two entries per sequence
    out->seqtab = 2 * int64_t(batch);
    out->merges = merges;
    out->partial_rows = partial;
    return OK;
}

void recycle_schedule(Schedule* s) {
    if (s && s->tiles.capacity() > t_sched.tiles.capacity()) std::swap(*s, t_sched);
}

int build_schedule(const PlanParams& p, int32_t batch, const int32_t* qo_indptr,
                   const int32_t* kv_page_indptr, const int32_t* kv_last_page_len, Schedule* out,
                   std::string* err) {
    if (!out || batch < 0) return fail(err, E_ARG, "batch must be >= 0 and out non-NULL");
    if (batch > 0 && (!qo_indptr || !kv_page_indptr || !kv_last_page_len))
        return fail(err, E_ARG, "qo_indptr, kv_page_indptr and kv_last_page_len must be non-NULL");
    if (p.num_qo_heads < 1 || p.num_kv_heads < 1 || p.num_qo_heads % p.num_kv_heads != 0)
        return fail(err, E_SHAPE, "num_qo_heads (%ld) must be a positive multiple of num_kv_heads (%ld)",
                    p.num_qo_heads, p.num_kv_heads);
    if (p.head_dim != 64 && p.head_dim != 128)
        return fail(err, E_SHAPE, "head_dim %ld not supported (64 or 128)", p.head_dim);
    if (p.page_size != kPageSize) return fail(err, E_SHAPE, "page_size %ld not supported (16)", p.page_size);
    const int32_t G = p.num_qo_heads / p.num_kv_heads;
    if (G > kMaxGroup) return fail(err, E_SHAPE, "query group %ld exceeds %ld heads per kv head", G, kMaxGroup);
    if (p.max_kv_splits < 0) return fail(err, E_ARG, "max_kv_splits must be >= 0");

    Schedule& S = t_sched;
    std::vector<QTile>& base = t_base;
    std::vector<Piece>& wide = t_wide;
    std::vector<Piece>& narrow = t_narrow;
    std::vector<Piece>& group = t_group;
    std::vector<std::pair<int32_t, int32_t>>& elig = t_elig;
    S.tiles.clear();
    S.merges.clear();
    S.seqtab.clear();
    S.group_tiles = 0;
    S.partial_rows = 0;
    S.tokens_per_tile = S.block_m = S.block_n = 0;
    S.wide_tiles = S.narrow_tiles = 0;
    S.fused = false;
    S.max_splits = 1;
    S.narrow_max_rows = 0;
    S.narrow_split = false;
    S.total_q = S.visible_pairs = S.kv_tokens = 0;
    base.clear();
    wide.clear();
    narrow.clear();
    group.clear();
    elig.clear();
    if (p.shared_pages < 0) return fail(err, E_ARG, "shared_pages must be >= 0");
    S.block_n = block_n_for(p.head_dim);
    S.block_m = block_m_for(p.head_dim);
    S.tokens_per_tile = S.block_m / G;
    const int32_t BN = S.block_n, TQ = S.tokens_per_tile;

    if (batch > 0 && (qo_indptr[0] != 0 || kv_page_indptr[0] != 0))
        return fail(err, E_INDPTR, "qo_indptr[0] (%ld) and kv_page_indptr[0] (%ld) must be 0", qo_indptr[0],
                    kv_page_indptr[0]);
    base.reserve(size_t(batch) * p.num_kv_heads);
    // query tiles of one sequence: tokens in chunks of TQ, per kv head
    auto add_seq_tiles = [&](int32_t b, int32_t q_len, int32_t kv_len) {
        for (int32_t hk = 0; hk < p.num_kv_heads; ++hk)
            for (int32_t t0 = 0; t0 < q_len; t0 += TQ) {
                QTile t;
                t.seq = b;
                t.kv_head = hk;
                t.q_row0 = qo_indptr[b] + t0;
                t.q_count = std::min(TQ, q_len - t0);
                t.pos0 = kv_len - q_len + t0;
                t.kv_len = kv_len;
                t.page_base = kv_page_indptr[b];
                // keys past the last query's position are masked for every row: skip them
                t.kv_end = p.causal && p.tail_skip ? std::min(kv_len, t.pos0 + t.q_count) : kv_len;
                // The path is chosen per sequence, not per tile: a sequence whose rows
                // all fit one narrow tile (decode rows, a few tokens of few heads) is
                // narrow; every tile of a longer sequence is wide, its partial last tile
                // included.  A row's path (and so its rounding) then depends on its own
                // sequence only: a padded batch and its ragged twin put each real row
                // in tiles of the same kind, at the same offset.
                t.kind = int64_t(q_len) * G <= (p.narrow_valu ? kValuRows : kNarrowRows) ? kNarrow : kWide;
                base.push_back(t);
            }
    };
    // Shared-prefix grouping (kGroup tiles): MFMA narrow path only, at least two rows'
    // worth of sequences per tile.
    const int64_t shared_keys = int64_t(p.shared_pages) * kPageSize;
    const int32_t group_rows = p.shared_pages > 0 && !p.narrow_valu ? kNarrowRows / G : 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (qo_indptr[b + 1] < qo_indptr[b]) return fail(err, E_INDPTR, "qo_indptr decreases at %ld", b);
        if (kv_page_indptr[b + 1] < kv_page_indptr[b])
            return fail(err, E_INDPTR, "kv_page_indptr decreases at %ld", b);
        const int32_t q_len = qo_indptr[b + 1] - qo_indptr[b];
        const int32_t n_pages = kv_page_indptr[b + 1] - kv_page_indptr[b];
        if (n_pages > 0 && (kv_last_page_len[b] < 1 || kv_last_page_len[b] > kPageSize))
            return fail(err, E_LAST_PAGE_LEN, "kv_last_page_len[%ld] = %ld outside [1, 16]", b,
                        kv_last_page_len[b]);
        const int64_t kv_len64 = n_pages == 0 ? 0 : int64_t(n_pages - 1) * kPageSize + kv_last_page_len[b];
        if (kv_len64 > INT32_MAX / 2) return fail(err, E_ARG, "sequence %ld too long", b);
        const int32_t kv_len = int32_t(kv_len64);
        // Causal queries are the last q_len positions (q_len <= kv_len); non-causal ones
        // see all keys and may outnumber them (a cascade's shared-prefix segment), but
        // need at least one key.
        if (p.causal ? q_len > kv_len : (q_len > 0 && kv_len == 0))
            return fail(err, E_QLEN_GT_KVLEN, "sequence %ld: q_len %ld with kv_len %ld", b, q_len, kv_len);
        if (q_len == 0) continue;
        S.total_q += q_len;
        S.kv_tokens += kv_len;
        const int64_t d = kv_len - q_len;
        S.visible_pairs += p.causal ? (int64_t(q_len) * d + int64_t(q_len) * (q_len + 1) / 2) * p.num_qo_heads
                                    : int64_t(q_len) * kv_len * p.num_qo_heads;
        // A decode row that sees the whole declared shared prefix can join a kGroup tile.
        if (group_rows >= 2 && q_len == 1 && kv_len >= shared_keys) {
            elig.push_back({b, kv_len});
            continue;
        }
        add_seq_tiles(b, q_len, kv_len);
    }
    if (batch > 0 && int64_t(qo_indptr[batch]) * p.num_qo_heads * p.head_dim > (int64_t(1) << 40))
        return fail(err, E_ARG, "batch too large");

    // ---- kGroup tiles: consecutive decode rows over a shared prefix -----------------------
    // Up to group_rows (16 / G) consecutive sequences per tile, so that the prefix is read
    // once for all of them.  Members' own keys are walked in 16-key pages, each member's
    // padded to the longest member's count and two pages per 32-key step, so that a step
    // may hold the last page of one member and the first of the next; a group ends early
    // rather than pad more than a quarter of its private pages.  A lone sequence keeps an
    // ordinary narrow tile.
    if (!elig.empty()) {
        const int64_t SP = shared_keys / kPageSize;  // shared pages
        auto priv_pages = [&](int32_t kv_len) { return int32_t(ceil_div(kv_len - shared_keys, kPageSize)); };
        size_t i = 0;
        while (i < elig.size()) {
            size_t j = i + 1;
            int64_t sum = priv_pages(elig[i].second);
            int32_t pmax = int32_t(sum);
            while (j < elig.size() && int64_t(j - i) < group_rows && elig[j].first == elig[j - 1].first + 1) {
                const int32_t pj = priv_pages(elig[j].second);
                const int32_t pm = std::max(pmax, pj);
                if (4 * (sum + pj) < 3 * int64_t(j - i + 1) * pm) break;  // padding would waste > 1/4
                sum += pj;
                pmax = pm;
                ++j;
            }
            const int32_t b0 = elig[i].first, n = int32_t(j - i);
            if (n == 1) {
                add_seq_tiles(b0, 1, elig[i].second);
            } else {
                for (int32_t hk = 0; hk < p.num_kv_heads; ++hk) {
                    Tile t{};
                    t.q_row0 = qo_indptr[b0];
                    t.q_count = n;
                    t.pos0 = pmax;  // private pages per member
                    t.kv_len = int32_t(shared_keys);
                    t.page_base = kv_page_indptr[b0];
                    t.kv_head = hk;
                    t.kv_begin = 0;
                    t.kv_end = int32_t(32 * ceil_div(SP + int64_t(n) * pmax, 2));
                    t.part = -1;
                    t.seq = b0;
                    t.split = 0;
                    t.n_splits = 1;
                    t.kind = kGroup;
                    t.group = -1;
                    group.push_back({t, int64_t(t.kv_end) + 64});
                }
            }
            i = j;
        }
    }
    if (!group.empty()) {
        S.group_tiles = int64_t(group.size());
        S.seqtab.resize(2 * size_t(batch));
        for (int32_t b = 0; b < batch; ++b) {
            const int32_t n_pages = kv_page_indptr[b + 1] - kv_page_indptr[b];
            S.seqtab[2 * b] = kv_page_indptr[b];
            S.seqtab[2 * b + 1] = n_pages == 0 ? 0 : (n_pages - 1) * kPageSize + kv_last_page_len[b];
        }
    }

    if (batch > 0 && int64_t(qo_indptr[batch]) * p.num_qo_heads * p.head_dim > (int64_t(1) << 40))
        return fail(err, E_ARG, "batch too large");

    // ---- split-KV decision -------------------------------------------------------------
    // A split costs a merge at the end of the launch (partials written, counted and read
    // back by the last piece), so it is made only when the tiles are unbalanced: when the
    // longest key range is more than twice a CU's fair share of all keys (the keys of
    // every tile over num_cus).  Then the longest key ranges are cut into pieces of C
    // keys (C a multiple of kChunkKeys; pieces start at absolute key positions that are
    // multiples of C), the largest C that still gives `target` work items: one per CU
    // when every tile is narrow (measured on decode batches of 16 to 256 sequences of
    // 1024 to 8192 keys: one piece per CU beat two, and an unsplit batch of 128 x 1024
    // keys beat every split of it), two per CU with wide tiles.
    const int32_t num_cus = p.num_cus > 0 ? p.num_cus : 256;
    int32_t max_keys = kChunkKeys;
    int64_t total_keys = 0;
    bool any_wide = false;
    for (auto& t : base) {
        max_keys = std::max(max_keys, t.kv_end);
        total_keys += t.kv_end;
        any_wide = any_wide || t.kind == kWide;
    }
    for (auto& g : group) total_keys += g.t.kv_end;
    const int64_t target = (any_wide ? 2LL : 1LL) * num_cus;
    const bool balanced = 2 * total_keys >= int64_t(max_keys) * num_cus;
    const int32_t max_chunks = int32_t(ceil_div(max_keys, kChunkKeys));
    auto units = [&](int64_t chunk_keys) {
        int64_t u = int64_t(group.size());  // kGroup tiles: one work item each, never split
        for (auto& t : base) u += std::max<int64_t>(1, ceil_div(t.kv_end, chunk_keys));
        return u;
    };
    int64_t C = int64_t(max_chunks) * kChunkKeys;
    if (p.max_kv_splits != 1 && !balanced && int64_t(base.size() + group.size()) < target && max_chunks > 1) {
        if (units(kChunkKeys) < target) {
            C = kChunkKeys;
        } else {  // largest c in [1, max_chunks] with units(c * kChunkKeys) >= target
            int32_t lo = 1, hi = max_chunks;
            while (lo < hi) {
                int32_t mid = lo + (hi - lo + 1) / 2;
                if (units(int64_t(mid) * kChunkKeys) >= target) lo = mid; else hi = mid - 1;
            }
            C = int64_t(lo) * kChunkKeys;
        }
    }

    // ---- expand into pieces ------------------------------------------------------------
    int64_t part_next = 0;
    for (size_t i = 0; i < base.size(); ++i) {
        const QTile& q = base[i];
        int32_t ns = 1;
        int64_t per = int64_t(q.kv_end);  // keys per piece
        if (q.kv_end > C) {  // (a key range within one piece needs no division)
            const int64_t nchunks = ceil_div(q.kv_end, kChunkKeys);
            ns = int32_t(ceil_div(q.kv_end, C));
            if (p.max_kv_splits > 0) ns = std::min(ns, p.max_kv_splits);
            per = ceil_div(nchunks, ns) * kChunkKeys;
            ns = int32_t(std::max<int64_t>(1, ceil_div(q.kv_end, per)));
        }
        const int32_t rows = q.q_count * G;
        if (ns > 1) {
            Merge m{};
            m.q_row0 = q.q_row0;
            m.q_count = q.q_count;
            m.kv_head = q.kv_head;
            m.part0 = int32_t(part_next);
            m.n_splits = ns;
            S.merges.push_back(m);
            S.max_splits = std::max(S.max_splits, ns);
        }
        for (int32_t s = 0; s < ns; ++s) {
            Tile t{};
            t.q_row0 = q.q_row0;
            t.q_count = q.q_count;
            t.pos0 = q.pos0;
            t.kv_len = q.kv_len;
            t.page_base = q.page_base;
            t.kv_head = q.kv_head;
            t.kv_begin = int32_t(s * per);
            t.kv_end = int32_t(std::min<int64_t>(q.kv_end, (s + 1) * per));
            t.part = ns > 1 ? int32_t(part_next + int64_t(s) * rows) : -1;
            t.seq = q.seq;
            t.split = s;
            t.n_splits = ns;
            t.kind = q.kind;
            t.group = ns > 1 ? int32_t(S.merges.size()) - 1 : -1;
            if (t.kind == kNarrow) {
                ++S.narrow_tiles;
                S.narrow_max_rows = std::max(S.narrow_max_rows, t.q_count * G);
                if (ns > 1) S.narrow_split = true;
            }
            // cost ~ keys walked (wide tiles: rounded up to whole blocks) plus a fixed overhead
            // (every path steps through keys in blocks of 32)
            static_assert(kValuKeys == 32 && kWaveKeys == 32 && block_n_for(0) == 32, "32-key steps");
            const int64_t keys = ((int64_t(t.kv_end) - t.kv_begin + 31) & ~int64_t(31)) + 64;
            (t.kind == kWide ? wide : narrow).push_back({t, keys});
        }
        if (ns > 1) part_next += int64_t(ns) * rows;
    }
    if (part_next > INT32_MAX) return fail(err, E_ARG, "too many partial rows");
    S.partial_rows = part_next;

    // ---- launch order: wide tiles (one kernel), then narrow tiles (another) ----------------
    // A little narrow work beside wide tiles (the shortest prompts of a ragged prefill
    // batch) would cost a second launch, or narrow workgroups in the mixed launch, for
    // little work: it runs in the wide launch instead, where a tile of up to 16 rows is
    // a valid, partly empty wide tile.  Then every row of such a batch takes the wide
    // path, as it does in the batch padded to equal lengths.
    if (!p.narrow_valu && !narrow.empty() && !wide.empty()) {
        int64_t keys = 0;
        for (const auto& pc : narrow) keys += pc.t.kv_end - pc.t.kv_begin;
        if (keys * int64_t(p.head_dim) * 4 <= kFoldBytes) {
            for (auto& pc : narrow) {
                pc.t.kind = kWide;
                pc.cost = ceil_div(pc.t.kv_end - pc.t.kv_begin, BN) * BN + 64;
                wide.push_back(pc);
            }
            narrow.clear();
            S.narrow_tiles = 0;
            S.narrow_max_rows = 0;
            S.narrow_split = false;
        }
    }
    // kGroup tiles run on the narrow path, never as wide tiles.
    for (const auto& pc : group) {
        narrow.push_back(pc);
        ++S.narrow_tiles;
        S.narrow_max_rows = std::max(S.narrow_max_rows, pc.t.q_count * G);
    }
    // Narrow tiles read their keys once: longest first (LPT), ties in natural order.
    auto longer = [](const Piece& a, const Piece& b) { return a.cost > b.cost; };
    if (!std::is_sorted(narrow.begin(), narrow.end(), longer)) std::stable_sort(narrow.begin(), narrow.end(), longer);
    order_wide_for_xcds(wide);
    S.wide_tiles = int64_t(wide.size());
    S.tiles.reserve(wide.size() + narrow.size());
    if (!p.narrow_valu && !wide.empty() && !narrow.empty()) {
        // Both kinds in one launch (a mixed batch: prompts and decode rows), so that the
        // decode rows' K/V stream overlaps the prompts' matrix work.  Narrow tiles go in
        // blocks of kXcds between blocks of kXcds wide tiles, spread evenly over the
        // launch; a wide tile thus keeps its launch slot modulo kXcds (its XCD), and a
        // partial block of either kind comes last.
        S.fused = true;
        const size_t wb = (wide.size() + kXcds - 1) / kXcds, nb = (narrow.size() + kXcds - 1) / kXcds;
        size_t next_nb = 0;
        for (size_t k = 0; k < wb; ++k) {
            for (size_t i = k * kXcds; i < std::min(wide.size(), (k + 1) * kXcds); ++i) S.tiles.push_back(wide[i].t);
            for (const size_t upto = (k + 1) * nb / wb; next_nb < upto; ++next_nb)
                for (size_t i = next_nb * kXcds; i < std::min(narrow.size(), (next_nb + 1) * kXcds); ++i)
                    S.tiles.push_back(narrow[i].t);
        }
    } else {
        for (auto& pc : wide) S.tiles.push_back(pc.t);
        for (auto& pc : narrow) S.tiles.push_back(pc.t);
    }
    std::swap(*out, S);  // out's previous buffers are reused by the next call
    return OK;
}

}  // namespace rpa
