// rpa_schedule.h -- work items shared by the host planner and the gfx950
// kernels.  Internal to the library (not part of the C ABI).
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

namespace rpa {

constexpr int kPageSize = 16;
constexpr int kMaxGroup = 128;  // largest number of qo heads per kv head
constexpr int kWaves = 4;       // wavefronts per narrow-tile workgroup

// Query rows (token x qo head of one kv group, token-major) per wide tile: each of
// the 4 waves owns one 32-row MFMA column block.
constexpr int kWideWaves = 4;  // wavefronts per wide-tile workgroup, 32 query rows each
constexpr int block_m_for(int head_dim) { return head_dim > 0 ? 32 * kWideWaves : 32 * kWideWaves; }

constexpr int kNarrowRows = 16;  // sequences with at most this many rows (q_len * G) take the narrow path
constexpr int kWaveKeys = 32;     // keys one wave handles per step on the narrow path
constexpr int kValuRows = 8;      // narrow threshold when narrow tiles run on the VALU kernel
constexpr int kValuKeys = 32;     // keys one wave handles per step on the VALU narrow path
constexpr int kXcds = 8;          // MI355X: workgroup i of a launch runs on XCD i % 8
constexpr int kChunkKeys = 256;   // split pieces start at multiples of this many keys
// Narrow tiles join the wide launch when the plan has wide tiles and the narrow
// tiles' K/V come to at most kFoldBytes.
constexpr int64_t kFoldBytes = int64_t(8) << 20;

// Keys per inner block (unit) of the wide path, whatever the head_dim.
constexpr int block_n_for(int) { return 32; }

enum TileKind : int32_t {
    kWide = 0,    // up to 128 rows; 4 waves split the rows, walk keys together
    kNarrow = 1,  // up to 16 rows (decode-like); 4 waves split the keys
    kGroup = 2,   // up to 16 rows of several decode sequences that share a prefix; run
                  // by the narrow path over a virtual key range (see below)
};

// A kGroup tile holds the decode rows (q_len 1) of q_count consecutive sequences
// seq .. seq + q_count - 1 whose first kv_len keys (the shared prefix, a multiple of
// 16) lie in the same physical pages.  Its keys are walked as virtual 16-key page
// slots, two per 32-key step: slots 0 .. kv_len / 16 - 1 are the shared pages (from
// page_base = the first sequence's kv_page_indptr), visible to every row; then pos0
// slots per member sequence i (its own keys kv_len + 16 p, p < pos0, pages from its own
// page table), visible to its rows only, masked past its length; kv_end = 32 ceil(
// (kv_len / 16 + q_count pos0) / 2).  The members' page bases and lengths come from
// the per-sequence table (Schedule::seqtab).  Never split.

// One unit of attention work: the rows (tokens q_row0 .. q_row0+q_count-1, all
// qo heads of kv head `kv_head`) against keys [kv_begin, kv_end) of one sequence.
struct Tile {
    int32_t q_row0;     // token row in Q / O of the first query
    int32_t q_count;    // query tokens (1 .. tokens_per_tile)
    int32_t pos0;       // position of the first query: kv_len - q_len + first token
    int32_t kv_len;     // tokens cached for the sequence
    int32_t page_base;  // kv_page_indptr[seq]
    int32_t kv_head;
    int32_t kv_begin;   // first key (a multiple of block_n)
    int32_t kv_end;     // one past the last key
    int32_t part;       // -1: write O / LSE; else first fp32 partial row of this piece
    int32_t seq;
    int32_t split;      // piece index within its query tile
    int32_t n_splits;   // pieces of its query tile
    int32_t kind;       // TileKind
    int32_t group;      // split group (index of its counter) when n_splits > 1, else -1
    int32_t reserved[2];
};
static_assert(sizeof(Tile) == 64, "Tile is 16 int32");

// Combine the pieces of one split query tile.  Rows r < q_count*G of piece s
// are at partial row part0 + s*(q_count*G) + r.
struct Merge {
    int32_t q_row0;
    int32_t q_count;
    int32_t kv_head;
    int32_t part0;
    int32_t n_splits;
    int32_t reserved[3];
};
static_assert(sizeof(Merge) == 32, "Merge is 8 int32");

struct PlanParams {
    int32_t num_qo_heads, num_kv_heads, head_dim, page_size, causal;
    int32_t max_kv_splits;  // 0 = decide, 1 = never, n = cap
    int32_t num_cus;
    int32_t narrow_valu;    // 1: narrow tiles (<= kValuRows rows) run on the VALU kernel
    int32_t shared_pages;   // > 0: every sequence's first shared_pages page ids are the same
                            // pages; decode rows are grouped into kGroup tiles
    int32_t tail_skip = 1;  // 0: causal query tiles walk every key up to kv_len, masking the
                            // fully masked tail instead of skipping it (cost measurement)
};

struct Schedule {
    std::vector<Tile> tiles;    // launch order
    std::vector<Merge> merges;
    std::vector<int32_t> seqtab;  // with kGroup tiles: {kv_page_indptr[b], kv_len} per sequence
    int64_t group_tiles = 0;      // kGroup tiles among the narrow ones
    int64_t partial_rows = 0;
    int32_t tokens_per_tile = 0;
    int32_t block_m = 0;
    int32_t block_n = 0;
    int64_t wide_tiles = 0;     // tiles[0, wide_tiles) are wide, the rest narrow (unless fused)
    bool fused = false;         // both kinds, interleaved, in one launch of the mixed kernel
    int32_t max_splits = 1;
    int64_t narrow_tiles = 0;
    int32_t narrow_max_rows = 0;  // largest row count among narrow tiles
    bool narrow_split = false;    // some narrow tile's key range is split into pieces
    int64_t total_q = 0;
    int64_t visible_pairs = 0;  // per qo head, summed over heads
    int64_t kv_tokens = 0;
};

// Status codes match rpa_status in rpa.h.
int build_schedule(const PlanParams& p, int32_t batch, const int32_t* qo_indptr,
                   const int32_t* kv_page_indptr, const int32_t* kv_last_page_len, Schedule* out,
                   std::string* err);

// Hand a schedule that is no longer needed back to the calling thread's planner, whose
// next build_schedule reuses its buffers (a decode loop re-plans every step).
void recycle_schedule(Schedule* s);

// Upper bounds on the sizes of every schedule build_schedule can produce for a batch
// of `batch` sequences holding `total_q` query tokens and `total_pages` pages in all,
// whatever their individual lengths.
struct ScheduleBound {
    int64_t tiles;         // launch slots (split pieces and XCD padding included)
    int64_t seqtab;        // sequence-table entries (int32)
    int64_t merges;        // split groups
    int64_t partial_rows;  // fp32 partial rows
};
int schedule_bound(const PlanParams& p, int32_t batch, int64_t total_q, int64_t total_pages, ScheduleBound* out,
                   std::string* err);

// Byte layout of a plan's workspace: [tiles][sequence table][split counters][error word]
// [partial LSE][partial O].  rpa_plan_bind copies [0, off_part_lse) (tiles, sequence
// table, zeroed counters, zeroed error word); rpa_plan_upload copies [0, off_flags)
// only, so the error word keeps what earlier runs raised until rpa_plan_check reads it.
struct WorkspaceLayout {
    size_t off_tiles, off_seqtab, off_counters, off_flags, off_part_lse, off_part_o, bytes;
};
WorkspaceLayout workspace_layout(int64_t tiles, int64_t seqtab_entries, int64_t merges, int64_t partial_rows,
                                 int head_dim);

}  // namespace rpa
