/*
 * rpa.h -- C ABI of a gfx950 (MI355X) library for batched attention over a
 * paged KV cache with a ragged batch of sequences.
 *
 * The operation (flashinfer issue #323, "How are prefill and decode kernels
 * different?": the BatchPrefillWithPagedKVCacheWrapper repro, its tensors and
 * its begin_forward / forward / end_forward lifecycle):
 *
 *   A batch of `batch` sequences.  Sequence b brings q_len[b] new query tokens
 *   (1 for decode, more for prefill or for a suffix after a cached prefix),
 *   packed in Q at rows qo_indptr[b] .. qo_indptr[b+1]-1.  Its kv_len[b]
 *   cached tokens live in pages of `page_size` (16) token slots:
 *     n_pages = kv_page_indptr[b+1] - kv_page_indptr[b]
 *     kv_len  = n_pages == 0 ? 0 : (n_pages - 1) * page_size + kv_last_page_len[b]
 *     token t < kv_len is in page kv_page_indices[kv_page_indptr[b] + t / page_size],
 *     slot t % page_size.
 *   The cache is [num_pages][2][page_size][num_kv_heads][head_dim] (per page:
 *   K then V, each "NHD"), in the same dtype as Q.
 *
 *   The queries are the last q_len tokens of the sequence: query i is at
 *   position kv_len - q_len + i, and with causal != 0 it sees keys 0..that
 *   position (llama.cpp discussion #15958, "Pad for prefill stage?": real
 *   tokens first, fully masked tails skipped); with causal == 0 it sees all
 *   kv_len keys, and q_len may exceed kv_len (one shared prefix attended by
 *   many requests' queries, the first half of a cascade; vLLM issue #227).
 *   qo head h reads kv head h / (num_qo_heads / num_kv_heads).
 *
 *   O[row][h][:] = sum_j softmax_j(sm_scale * <Q[row][h], K_j>) * V_j   (input dtype,
 *                  rounded to nearest-even from fp32)
 *   LSE[row][h]  = ln sum_j exp(sm_scale * <Q[row][h], K_j>)             (fp32, optional)
 *
 * Conventions for every entry point:
 *   - Every call returns an rpa_status; RPA_OK is 0.  rpa_last_error() returns
 *     a thread-local message for the last non-OK status.  No C++ exception
 *     crosses this ABI.
 *   - "host" pointers are CPU memory read during the call only.  "device"
 *     pointers are GPU memory the caller owns; the library borrows them and
 *     never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - Kernel faults are asynchronous and surface at the caller's next
 *     synchronisation, as usual for HIP.
 *
 * Environment (read by rpa_plan_create / rpa_plan_create_shared; for tests and
 * measurement, off by default):
 *   RPA_DISABLE_TAIL_SKIP=1  causal query tiles walk every key up to kv_len and
 *                            mask the fully masked tail instead of skipping it
 *                            (the skip of llama.cpp discussion #15958, switched
 *                            off to time what it saves); results are unchanged.
 *                            rpa_plan_update keeps the plan's setting.
 *   RPA_LOG=1                one summary line per created or updated plan on
 *                            stderr: tiles by kind, split groups, partial rows,
 *                            workspace bytes.
 */
#ifndef RPA_H
#define RPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RPA_OK = 0,
    RPA_E_ARG = 1,             /* NULL pointer, bad enum, negative size          */
    RPA_E_SHAPE = 2,           /* heads / head_dim / page_size not supported      */
    RPA_E_INDPTR = 3,          /* an indptr does not start at 0 or decreases      */
    RPA_E_LAST_PAGE_LEN = 4,   /* kv_last_page_len outside [1, page_size]         */
    RPA_E_QLEN_GT_KVLEN = 5,   /* causal: q_len > kv_len; non-causal: queries but
                                  no cached token                                 */
    RPA_E_WORKSPACE = 6,       /* workspace too small or misaligned               */
    RPA_E_UNSUPPORTED = 7,     /* valid request the library does not implement    */
    RPA_E_HIP = 8,             /* a HIP runtime call failed (message has details) */
    RPA_E_PAGE_OOB = 9,        /* a page index outside [0, num_pages)             */
    RPA_E_V_RANGE = 10         /* bf16 V above 65504 met by the fp16 P V product  */
} rpa_status;

typedef enum { RPA_F16 = 0, RPA_BF16 = 1 } rpa_dtype;

typedef struct {
    int32_t num_qo_heads;   /* H_qo >= 1                                          */
    int32_t num_kv_heads;   /* H_kv >= 1, H_qo % H_kv == 0                        */
    int32_t head_dim;       /* 64 or 128                                          */
    int32_t page_size;      /* 16                                                 */
    int32_t dtype;          /* rpa_dtype of Q, the cache and O                    */
    int32_t causal;         /* 1: queries are the last q_len positions, causal    */
    float sm_scale;         /* <= 0 selects 1/sqrt(head_dim)                      */
    int32_t max_kv_splits;  /* 0: planner decides; 1: never split; n: at most n   */
    int32_t num_cus;        /* compute units the schedule targets; 0 selects 256  */
    int32_t narrow_kernel;  /* decode-like tiles: 0 MFMA kernel (up to 16 rows per
                               tile), 1 VALU kernel without MFMA (up to 8 rows;
                               the design of the pages' CUDA-core decode)        */
    int32_t kv_shared;      /* 0: each cache page is read by one sequence (no
                               shared prefix): decode-like tiles load K/V as
                               non-temporal streams that do not displace the
                               caches; 1: pages may be shared by several
                               sequences (a common prefix, vLLM issue #227):
                               K/V loads stay cacheable so sequences reading the
                               same page together hit in L2.  A caching hint
                               only: results are bitwise the same either way. */
} rpa_params;

typedef struct rpa_plan rpa_plan;

typedef struct {
    int64_t num_tiles;         /* work items: split pieces and empty XCD padding  */
    int64_t num_split_groups;  /* query tiles whose key range is split            */
    int32_t max_splits;        /* largest split count of any query tile           */
    int32_t block_m;           /* query rows (token, head) per tile               */
    int32_t block_n;           /* keys per inner block                            */
    int32_t tokens_per_tile;   /* query tokens per tile                           */
    int64_t partial_rows;      /* fp32 partial rows the workspace holds           */
    size_t workspace_bytes;    /* bytes rpa_plan_bind needs                       */
    int64_t total_q;           /* query tokens of the batch                       */
    int64_t visible_pairs;     /* sum over rows and qo heads of visible keys      */
    int64_t kv_tokens;         /* sum of kv_len over sequences with queries       */
} rpa_plan_info_t;

/*
 * Workspace size bound (flashinfer issue #323, "How are prefill and decode kernels
 * different?": the repro allocates one uint8 workspace buffer before it builds the
 * wrapper and calls begin_forward).  Writes to *bytes_out an upper bound on
 * rpa_plan_info().workspace_bytes over every batch of `batch` sequences holding
 * `total_q` query tokens and `total_pages` pages (the sum of their page counts) in
 * all, whatever the individual lengths, for these params.  A caller can allocate
 * the workspace once from it and bind any such plan into it.  Host-only.
 * The bound is loose by design: it covers splitting a few long sequences into
 * many pieces and the empty tiles that align wide tiles to XCDs.
 * Errors: E_ARG (NULL pointer, negative size), E_SHAPE.
 */
rpa_status rpa_workspace_bytes(const rpa_params* params, int32_t batch, int64_t total_q, int64_t total_pages,
                               size_t* bytes_out);

/*
 * Plan (the host half of begin_forward in flashinfer issue #323's repro, which
 * takes qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len, the head
 * counts, head_dim and page_size): validate the ragged lengths and build the work
 * schedule.  Host-only: no HIP call is made, so it also runs where no GPU is
 * present.  The schedule depends only on the lengths and parameters, never on
 * page ids, so equal lengths give equal schedules.  The path of a query row
 * (wide tiles of up to 128 rows, or narrow decode tiles of up to 16) is chosen
 * per sequence: a sequence whose q_len * G rows fit one narrow tile is narrow,
 * every tile of a longer one is wide; narrow tiles whose K/V total at most 8 MiB
 * run as wide tiles when the batch has wide tiles.  Key ranges are split into
 * pieces (merged inside the launch; flashinfer issue #323's kv-parallel decode)
 * only when the tiles are unbalanced -- the longest range above twice the batch's
 * keys per compute unit (num_cus) -- and then toward one piece per compute unit
 * (two when the batch has wide tiles); max_kv_splits caps the pieces of a tile.
 * A ragged prefill batch and its twin padded to equal lengths (llama.cpp
 * discussion #15958, "Pad for prefill stage?") give bit-identical real rows when
 * the ragged batch has a sequence of more than 16 rows and neither run splits key
 * ranges.
 *   qo_indptr_h        host int32 [batch+1]; [0] == 0, non-decreasing
 *   kv_page_indptr_h   host int32 [batch+1]; [0] == 0, non-decreasing
 *   kv_last_page_len_h host int32 [batch]; in [1, page_size] for a sequence with pages
 *   out                receives a plan the caller frees with rpa_plan_destroy
 * Errors: E_ARG, E_SHAPE, E_INDPTR, E_LAST_PAGE_LEN, E_QLEN_GT_KVLEN.
 */
rpa_status rpa_plan_create(const rpa_params* params, int32_t batch, const int32_t* qo_indptr_h,
                           const int32_t* kv_page_indptr_h, const int32_t* kv_last_page_len_h,
                           rpa_plan** out);

/*
 * Plan a batch whose sequences share a prefix stored once (vLLM issue #227,
 * "Question about efficient memory sharing": many requests over one system prompt,
 * its KV pages shared): as rpa_plan_create, with the caller's declaration that the
 * first `shared_pages` entries of the page list of every sequence that has at least
 * that many pages name the same physical pages.  Decode rows (q_len 1) that see the whole prefix are then
 * grouped, up to 16 / G consecutive sequences per tile, so that the prefix's K and
 * V are read once per group instead of once per sequence; their own keys follow,
 * visible to their own rows only.  Other sequences are planned as by
 * rpa_plan_create.  The declaration is trusted, not checked: if the pages differ,
 * the grouped rows attend to the first sequence's prefix.  The schedule still
 * depends only on the lengths and shared_pages.  Results equal those of
 * rpa_plan_create within the oracle tolerance (the keys are combined in another
 * order); rpa_plan_update keeps the declaration.  With narrow_kernel = 1, or more
 * than 8 query heads per kv head, nothing is grouped.
 * Errors: those of rpa_plan_create; E_ARG for shared_pages < 0.
 */
rpa_status rpa_plan_create_shared(const rpa_params* params, int32_t batch, const int32_t* qo_indptr_h,
                                  const int32_t* kv_page_indptr_h, const int32_t* kv_last_page_len_h,
                                  int32_t shared_pages, rpa_plan** out);

/* Summary of a plan (sizes, tile shape, work counts): the auxiliary data that
 * begin_forward builds in flashinfer issue #323, made inspectable.  Host-only. */
rpa_status rpa_plan_info(const rpa_plan* plan, rpa_plan_info_t* out);

/*
 * Copy of the plan's work items for inspection (tests; host-only; no passage of
 * the pages names this call): up to `cap` records of 16
 * int32 each into `out_h` (host), in launch order: the wide records, then the
 * narrow ones, or, when the plan has both kinds (and narrow_kernel is 0), both
 * in one launch with narrow records in blocks of 8 between blocks of 8 wide ones.
 * Wide records with [1] == 0 are empty padding that aligns tiles to XCDs
 * (workgroup i of a launch runs on XCD i % 8).  Fields per record:
 *   [0] first query row, [1] query tokens, [2] position of the first query,
 *   [3] kv_len, [4] kv_page_indptr[b], [5] kv head, [6] first key, [7] end key,
 *   [8] first partial row (-1: writes O directly), [9] sequence, [10] split
 *   index, [11] split count, [12] kind (0: wide, up to 128 rows; 1: narrow, up to
 *   16 rows; 2: a group of [1] decode rows of sequences [9].. over a shared prefix
 *   of [3] keys, then [2] private 16-key pages per member, two pages per 32-key
 *   step, so [7] = 32 ceil(([3] / 16 + [1] [2]) / 2)), [13] split group (-1 if not
 *   split), [14..15] reserved.
 * *n_out receives the number of records in the plan.
 */
rpa_status rpa_plan_tiles(const rpa_plan* plan, int32_t* out_h, int64_t cap, int64_t* n_out);

/*
 * Bind (the device half of begin_forward in flashinfer issue #323: the wrapper is
 * built over a caller-allocated workspace and begin_forward receives the device
 * kv_page_indices): upload the schedule into the caller's workspace and remember
 * the page-index array.
 *   kv_page_indices_d  device int32 [kv_page_indptr[batch]], borrowed until the
 *                      plan is destroyed or bound again
 *   num_pages          pages in the cache (rows of its leading axis); a page index
 *                      outside [0, num_pages) is never dereferenced: the kernel
 *                      reads zeros instead and raises the plan's error flag
 *   workspace_d        device buffer of at least rpa_plan_info().workspace_bytes,
 *                      256-byte aligned, borrowed until destroy or the next bind
 *   stream             the upload is enqueued here; rpa_run must be ordered after it
 * Errors: E_ARG, E_WORKSPACE (message states the size needed), E_HIP.
 */
rpa_status rpa_plan_bind(rpa_plan* plan, const int32_t* kv_page_indices_d, int64_t num_pages,
                         void* workspace_d, size_t workspace_bytes, void* stream);

/*
 * Run (forward in flashinfer issue #323's repro: q and the paged kv_cache in, the
 * output out, repeatable after one begin_forward): attention for every query row
 * of the plan.
 *   q         device [total_q][num_qo_heads][head_dim], dtype of the plan
 *   kv_cache  device [num_pages][2][page_size][num_kv_heads][head_dim], same dtype
 *   o         device [total_q][num_qo_heads][head_dim], same dtype (written)
 *   lse       device fp32 [total_q][num_qo_heads] (written), or NULL
 * Enqueues on `stream` one kernel over the plan's tiles: wide tiles (up to 128
 * query rows each), narrow tiles (up to 16 rows: decode-like), or both kinds
 * interleaved in one launch.  With params.narrow_kernel = 1 the narrow tiles (up
 * to 8 rows) run on the VALU kernel, launched after the wide tiles' kernel.  When
 * the plan splits key ranges, the piece
 * of each split group that finishes last merges the group inside its kernel.
 * No allocation, no host<->device synchronisation.  One run at a time per
 * (plan, workspace): the partial-result region and the split counters are
 * shared by all runs of a plan.
 * Errors: E_ARG (unbound plan, NULL pointer), E_HIP (launch failure).
 */
rpa_status rpa_run(const rpa_plan* plan, const void* q, const void* kv_cache, void* o, float* lse,
                   void* stream);

/*
 * Run without a workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation and kernels as rpa_run, for a plan that need not be bound: the
 * schedule, the split counters, the error word and the fp32 partials live in a
 * 16 MiB scratch array that the library holds in device memory (one per GPU, from
 * the first call on that GPU until the process ends).  Each call copies the plan's
 * schedule into it from the plan's host memory (hipMemcpyAsync; the plan must not
 * be updated or destroyed before `stream` has passed this call) and clears the
 * counters and error word with a kernel, then launches the attention kernels.
 *   kv_page_indices_d, num_pages  as for rpa_plan_bind
 *   q, kv_cache, o, lse           as for rpa_run
 *   err_flag_d  device int32 the kernels OR error bits into (1: page index out of
 *               range, 2: bf16 V above 65504; see rpa_plan_check), never cleared
 *               by the library; or NULL to drop them
 * Calls that overlap on one GPU (other streams, other threads) share the scratch
 * and race: order them.  No allocation of any kind (device, pinned or library).
 * Errors: E_WORKSPACE (the plan needs more than 16 MiB of scratch, checked before
 * any HIP call; rpa_plan_info().workspace_bytes tells), E_ARG, E_HIP.
 */
rpa_status rpa_run_noalloc(const rpa_plan* plan, const int32_t* kv_page_indices_d, int64_t num_pages,
                           const void* q, const void* kv_cache, void* o, float* lse, int32_t* err_flag_d,
                           void* stream);

/*
 * Re-plan in place for new lengths of the same batch (a decode step: every
 * sequence one token longer), keeping the launch shape: the new schedule must
 * have the same number of tiles, wide tiles and split groups, and no more partial
 * rows; otherwise RPA_E_UNSUPPORTED (create and bind a new plan).  Host-only: the
 * new schedule is written into the plan's pinned staging image (if bound) and
 * reaches the device with the next rpa_plan_upload.  This is what lets a captured
 * HIP graph [rpa_plan_upload, rpa_append_kv, rpa_run] be replayed step after step
 * (flashinfer issue #323: auxiliary data built by begin_forward, reused by
 * forward).  The caller makes sure the previous upload has completed (e.g. by
 * synchronising its stream) before calling this, since it rewrites the staging
 * image that upload reads.
 * Errors: those of rpa_plan_create, E_UNSUPPORTED.
 */
rpa_status rpa_plan_update(rpa_plan* plan, const int32_t* qo_indptr_h, const int32_t* kv_page_indptr_h,
                           const int32_t* kv_last_page_len_h);

/*
 * Enqueue on `stream` the copy of the plan's current schedule into its workspace
 * (the tile records and zeroed split counters, as rpa_plan_bind copies them; the
 * error word is left as it is).  One hipMemcpyAsync from pinned host memory, so it
 * can be captured into a HIP graph (the second half of the auxiliary-data reuse
 * in flashinfer issue #323: begin_forward once, forward per step).
 * Errors: E_ARG (unbound plan), E_HIP.
 */
rpa_status rpa_plan_upload(const rpa_plan* plan, void* stream);

/*
 * Error word of a bound plan.  The pages show no error convention beyond the
 * repro's assertions (flashinfer issue #323); a kernel cannot return a status, so
 * the runs OR bits into a word of the workspace that this call reads and clears.
 * Synchronises `stream`, then writes to *flag_out the bits raised by the runs
 * since the last bind or check (rpa_plan_upload does not clear them):
 *   1  a page index outside [0, num_pages) was met; its keys read as zero K and V
 *      (returns RPA_E_PAGE_OOB);
 *   2  a bf16 V value above 65504, the largest fp16 value, was read by the fp16
 *      P V product and saturated there: the rows that read it are wrong (returns
 *      RPA_E_V_RANGE unless bit 1 is also set).  bf16 V below 2^-14 rounds toward
 *      zero there, an absolute error under 2^-24, and raises nothing.  The VALU
 *      narrow kernel (narrow_kernel = 1) multiplies in fp32 and never raises it.
 * 0 returns RPA_OK.
 * Errors: E_ARG (NULL, unbound plan), E_HIP, E_PAGE_OOB, E_V_RANGE.
 */
rpa_status rpa_plan_check(const rpa_plan* plan, void* stream, int32_t* flag_out);

/* Free a plan's host memory (end_forward in flashinfer issue #323's repro).  The
 * caller first makes sure no run using it is still in flight.  NULL is ignored. */
void rpa_plan_destroy(rpa_plan* plan);

/*
 * Host-side check of a page table (tests and debugging): every index of every
 * sequence inside [0, num_pages), the pool of pages the cache holds
 * (flashinfer issue #323's repro: kv_page_indices index the leading axis of
 * kv_cache).  Host pointers only.
 * Errors: E_ARG, E_INDPTR, E_PAGE_OOB.
 */
rpa_status rpa_validate_page_table(int32_t batch, const int32_t* kv_page_indptr_h,
                                   const int32_t* kv_page_indices_h, int64_t num_pages);

/*
 * Append new tokens' K and V into their page slots (the page-table addressing of
 * flashinfer issue #323's repro: token t of sequence b is in page
 * kv_page_indices[kv_page_indptr[b] + t / 16], slot t % 16).  The page table
 * describes the sequences AFTER the append; the new tokens of sequence b are its
 * last append_indptr[b+1] - append_indptr[b] tokens, like queries and qo_indptr.
 *   append_indptr_d     device int32 [batch+1], [0] == 0, [batch] == n_new
 *   kv_page_indptr_d    device int32 [batch+1]
 *   kv_page_indices_d   device int32 [kv_page_indptr[batch]]
 *   kv_last_page_len_d  device int32 [batch]
 *   new_kv_d            device [n_new][2][num_kv_heads][head_dim] (K then V), the
 *                       cache's dtype, 16-byte aligned
 *   kv_cache_d          device [num_pages][2][16][num_kv_heads][head_dim], written
 *   err_flag_d          device int32, set to 1 if a token has no valid slot (its
 *                       position or page is out of range; it is not written); or NULL
 * The device arrays are read by the kernel, not checked on the host.  Enqueues one
 * kernel on `stream`; no allocation, no synchronisation (graph-capturable).
 * Errors: E_ARG, E_SHAPE, E_HIP.
 */
rpa_status rpa_append_kv(int32_t batch, int64_t n_new, int32_t num_kv_heads, int32_t head_dim,
                         const int32_t* append_indptr_d, const int32_t* kv_page_indptr_d,
                         const int32_t* kv_page_indices_d, const int32_t* kv_last_page_len_d, const void* new_kv_d,
                         void* kv_cache_d, int64_t num_pages, int32_t* err_flag_d, void* stream);

/*
 * Trim sequences to shorter lengths (drop padding KV after a padded prefill;
 * llama.cpp discussion #15958, "Pad for prefill stage?"): a page-table edit, no
 * data moves.  Sequence b keeps its first new_kv_len[b] <= kv_len tokens, i.e. its
 * first ceil(new_kv_len[b] / 16) pages, in order; the dropped pages go back to the
 * caller's allocator and later appends overwrite the kept page's tail slots.
 * Host arrays only:
 *   in:  kv_page_indptr_h [batch+1], kv_page_indices_h, kv_last_page_len_h [batch],
 *        new_kv_len_h [batch]
 *   out: out_kv_page_indptr_h [batch+1], out_kv_page_indices_h (room for
 *        kv_page_indptr_h[batch] entries), out_kv_last_page_len_h [batch] (0 for an
 *        emptied sequence)
 * Errors: E_ARG (NULL array, new length outside [0, kv_len]), E_INDPTR, E_LAST_PAGE_LEN.
 */
rpa_status rpa_trim_page_table(int32_t batch, const int32_t* kv_page_indptr_h, const int32_t* kv_page_indices_h,
                               const int32_t* kv_last_page_len_h, const int32_t* new_kv_len_h,
                               int32_t* out_kv_page_indptr_h, int32_t* out_kv_page_indices_h,
                               int32_t* out_kv_last_page_len_h);

/*
 * Merge two attention states of the same query rows computed over disjoint key
 * sets A and B (the split-KV merge applied to whole outputs; it joins the two
 * halves of a cascade: a prefix shared by many requests, attended once for all of
 * them with causal == 0, plus each request's private suffix; vLLM issue #227,
 * "Question about efficient memory sharing"):
 *   w_x = exp(LSE_x - max(LSE_a, LSE_b)),
 *   O   = (w_a O_a + w_b O_b) / (w_a + w_b)   (rounded to nearest-even to dtype),
 *   LSE = max(LSE_a, LSE_b) + ln(w_a + w_b).
 * A state with LSE = -inf has weight 0 and its O values are ignored (they may be
 * anything, NaN included); when both do, O = 0 and LSE = -inf.
 *   o_a, o_b, o   device [rows][num_heads][head_dim], dtype, 16-byte aligned
 *   lse_a, lse_b  device fp32 [rows][num_heads]
 *   lse           device fp32 [rows][num_heads] (written), or NULL
 * o may alias o_a or o_b, and lse may alias lse_a or lse_b (in-place merge).
 * Enqueues one kernel on `stream`; no allocation, no synchronisation.
 * Errors: E_ARG (NULL pointer, misaligned O, bad dtype), E_SHAPE (head_dim not
 * 64 or 128), E_HIP (launch failure).
 */
rpa_status rpa_merge_states(int64_t rows, int32_t num_heads, int32_t head_dim, int32_t dtype, const void* o_a,
                            const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                            void* stream);

/* Thread-local message describing the last non-OK status ("" if none). */
const char* rpa_last_error(void);

/* Library version, "major.minor.patch". */
const char* rpa_version(void);

/*
 * Kernel timing (benchmarks): while enabled, rpa_run has a HIP event pair
 * stamped by each kernel dispatch it enqueues (start and end of the kernel).
 * rpa_prof_stop synchronises those events and returns, per kernel kind
 * (0 = wide-tile or mixed kernel, 1 = narrow-tile kernel), the number of
 * launches and their summed duration in milliseconds.
 */
rpa_status rpa_prof_start(void);
rpa_status rpa_prof_stop(int64_t counts_out[2], double ms_out[2]);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H */
