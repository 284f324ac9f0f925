// rpa_launch.h -- kernel argument blocks and launchers (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa_schedule.h"

namespace rpa {

// Bits of a plan's error word (OR-ed by the kernels, read by rpa_plan_check).
enum ErrBits : int32_t {
    kErrPage = 1,    // a page index outside [0, num_pages): its keys read as zero K and V
    kErrVRange = 2,  // a bf16 V value above the largest fp16 value (65504) entered P V
};

struct AttnArgs {
    const Tile* tiles;
    const int32_t* page_idx;  // kv_page_indices
    int32_t num_pages;
    const uint16_t* q;        // [total_q][H][D]
    const uint16_t* kv;       // [num_pages][2][16][Hkv][D]
    uint16_t* o;              // [total_q][H][D]
    float* lse;               // [total_q][H] or NULL
    float* part_o;            // [partial_rows][D]
    float* part_lse;          // [partial_rows]
    int32_t H, Hkv, G;
    float c_log2;             // sm_scale * log2(e)
    int32_t causal;
    int32_t* err_flag;        // error word: ErrBits OR-ed atomically
    int32_t* counters;        // one per split group: pieces finished (reset to 0 by the last)
    const int32_t* seqtab;    // kGroup tiles: {kv_page_indptr[b], kv_len} per sequence
};

struct LaunchAttn {
    AttnArgs a;       // a.tiles points at this launch's first tile
    int head_dim;
    bool bf16;
    int64_t n_tiles;
    bool k_rows;      // narrow kernel: K loaded in whole rows through LDS (else straight into
                      // MFMA operand layout)
    bool kv_stream;   // narrow tiles: K/V loads non-temporal (pages not shared by sequences)
    bool group;       // the tiles include kGroup tiles (the kernel instantiation that runs them)
};


// Merge of two attention states (O, LSE) computed over disjoint key sets.
struct MergeArgs {
    const uint16_t* o_a;  // [items / (head_dim / 8)][head_dim]: rows x heads x head_dim
    const float* lse_a;   // one per (row, head)
    const uint16_t* o_b;
    const float* lse_b;
    uint16_t* o;          // may alias o_a or o_b
    float* lse;           // may alias lse_a or lse_b; NULL: not written
    int64_t items;        // (row, head, 8-element chunk) triples
    int32_t head_dim;
};

// Append of new tokens' K and V into their page slots.
struct AppendArgs {
    const int32_t* append_indptr;     // [batch + 1]: new tokens of sequence b are rows [b], [b+1) of new_kv
    const int32_t* kv_page_indptr;    // [batch + 1], lengths after the append
    const int32_t* kv_page_indices;
    const int32_t* kv_last_page_len;  // [batch]
    const uint16_t* new_kv;           // [n_new][2][Hkv][D]
    uint16_t* kv;                     // [num_pages][2][16][Hkv][D]
    int64_t n_new;
    int32_t batch, Hkv, D, num_pages;
    int32_t* err_flag;                // set to 1 for a token with no valid slot; may be NULL
};

// ev0 / ev1: optional events stamped at the start and end of the dispatch (NULL: none).
hipError_t launch_wide(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_narrow(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// Wide and narrow tiles (each record's kind) in one launch.
hipError_t launch_mixed(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// Narrow tiles on the VALU kernel; max_rows (<= kValuRows) picks its row capacity.
hipError_t launch_narrow_valu(const LaunchAttn& L, int max_rows, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_merge(const MergeArgs& M, bool bf16, hipStream_t stream);
hipError_t launch_append(const AppendArgs& A, hipStream_t stream);
// Zero n int32 at p (a kernel: no memset node in a captured graph).
hipError_t launch_clear(int32_t* p, int64_t n, hipStream_t stream);

// Device scratch of rpa_run_noalloc: a file-scope __device__ array of this many bytes,
// one copy per GPU, held until the process ends.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
// Device address of the current device's copy of that array, resolved once per device
// with hipGetSymbolAddress (the array's name in host code is only a host-side stand-in).
hipError_t static_scratch(void** ptr);

}  // namespace rpa
