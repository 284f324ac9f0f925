// rpa_kernels.hip -- gfx950 (CDNA4) kernels for ragged attention over a paged
// KV cache.  One 256-thread workgroup (4 wave64) per Tile; rows of a tile are
// (token, qo head) pairs of one kv head's query group, token-major, so the G
// heads sharing a kv head read each K/V block once (grouped-query attention,
// flashinfer issue #323).
//
//   attn_wide_kernel    tiles of up to 128 rows (prefill): S^T = K Q^T and
//                       O^T += V^T P^T on v_mfma_f32_32x32x16, 32-key units
//                       loaded straight from the cache into an LDS ring, a
//                       software pipeline over the units, Q read and O written
//                       in whole rows through LDS (see wide_tile);
//   attn_narrow_kernel  tiles of up to 16 rows (decode-like): the 4 waves split
//                       the keys, v_mfma_f32_16x16x32, K into MFMA registers
//                       directly or in whole rows through LDS, V read back
//                       transposed (see narrow_tile); K/V loads non-temporal
//                       unless the caller says pages are shared by sequences;
//   attn_mixed_kernel   both kinds in one launch, for plans that have both (a
//                       mixed batch of prompts and decode rows);
//   attn_narrow_valu_kernel  the same tiles (up to 8 rows) without MFMA, on dot2
//                       and fp32 FMAs, for comparison (see valu_tile);
//   merge_states_kernel join of two attention states (cascade halves);
//   append_kv_kernel    new tokens' K/V into their page slots.
//
// Common to the attention kernels: online softmax in the exp2 domain with P
// rounded to fp16 for the P V product (bf16 V converted to fp16); masks only on
// boundary units, and blocks past every row's causal position never loaded
// (llama.cpp discussion #15958: fully masked tails are skipped); epilogue O / l
// rounded to nearest-even into the input dtype and LSE = ln(l) + max.  Split KV:
// a long key range is cut into pieces that run as separate work items; each
// writes fp32 partial rows and the last piece to finish merges them by weights
// exp(LSE_s - max LSE) inside the same launch (flashinfer issue #323 speaks of
// kv-parallelism / split-k).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "rpa_launch.h"
#include "rpa_schedule.h"

namespace rpa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c, bool bf16) {
    if (bf16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16_qk(u32x4 a, u32x4 b, f32x4 c, bool bf16) {
    if (bf16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16_pv(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                   0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 from an LDS address (4 x 16-bit, transposed across 16 lanes).
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// LDS address m0 + 16 l (global_load_lds_dwordx4, SGPR base + 32-bit lane offset).
// Written out as assembly so that the compiler's wait-count pass does not track it:
// that pass cannot tell which later LDS reads may overlap the write and would wait
// for every load in flight before them.  The caller waits with s_waitcnt vmcnt
// before anyone reads the bytes.
// The statement sets M0 itself; the compiler does not honour M0 in a clobber list,
// which is safe only because no compiler-generated code in the kernels that use it
// keeps a value in M0 (their assembly has no other M0 access).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t lane_off, uint32_t lds_m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(sbase), "s"(lds_m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// 32-bit LDS address of a pointer into the workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 bytes of K or V from the cache.  NT: a non-temporal (streaming) load, for
// pages that no other tile of the launch reads -- it does not displace the L2
// lines of the schedule, page indices and Q that every workgroup reads first.
template <bool NT>
__device__ __forceinline__ u32x4 ld_kv(const uint16_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return *reinterpret_cast<const u32x4*>(p);
}

// Two fp32 -> packed 16-bit, round to nearest-even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack_out(float a, float b) {
    if (BF16) {
        __bf16 x = (__bf16)a, y = (__bf16)b;
        return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
    }
    _Float16 x = (_Float16)a, y = (_Float16)b;
    return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Two fp32 probabilities in [0, 1] -> packed fp16, round to nearest-even.
// One 16-bit element (low or high half of a packed word) as fp32, exactly.
template <bool BF16>
__device__ __forceinline__ float elem16(uint32_t w, int hi) {
    const uint16_t h = uint16_t(hi ? (w >> 16) : (w & 0xffffu));
    if (BF16) return __builtin_bit_cast(float, uint32_t(h) << 16);
    return float(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint32_t pack_p(float a, float b) { return pack_out<false>(a, b); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// One packed bf16 pair as a packed fp16 pair: exact for |x| in [2^-14, 65504] and
// for zeros, infinities and NaN; round-toward-zero below 2^-14 (absolute error
// < 2^-24); saturation to 65504 above it, which no correct output allows.  No bf16
// value lies strictly between 65280 and 65536, so an fp16 result of magnitude 65504
// (0x7bff) comes from saturation only.  vmax keeps the largest fp16 magnitude
// pattern produced (per 16-bit half: sign cleared, one packed max); a tile that
// produced 0x7bff or more (saturated, infinite or NaN V) raises kErrVRange.
__device__ __forceinline__ uint32_t v_pair_fp16(uint32_t w, u16x2& vmax) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, w << 16),
                                                                               __builtin_bit_cast(float, w & 0xffff0000u)));
    vmax = __builtin_elementwise_max(vmax, __builtin_bit_cast(u16x2, h & 0x7fff7fffu));
    return h;
}

// fp16 magnitude pattern of 65504, the value bf16 V above the fp16 range saturates to.
constexpr unsigned short kF16Saturated = 0x7bff;

// Error bits of a plan (device int32, OR-ed by any workgroup; see rpa_launch.h).
__device__ __forceinline__ void raise_flag(int32_t* flag, int32_t bits) {
    __hip_atomic_fetch_or(flag, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Whether any lane of the wave converted a bf16 V above 65504 (wave-uniform).
__device__ __forceinline__ bool wave_v_big(u16x2 vmax) {
    return __builtin_amdgcn_ballot_w64(vmax[0] >= kF16Saturated || vmax[1] >= kF16Saturated) != 0;
}
// Once per wave: raise kErrVRange if any lane converted a bf16 V above 65504.
__device__ __forceinline__ void flag_v_range(int32_t* flag, u16x2 vmax) {
    if (wave_v_big(vmax) && (threadIdx.x & 63) == 0) raise_flag(flag, kErrVRange);
}

// Value of lane l ^ 32: v_permlane32_swap exchanges the two 32-lane halves of a
// register pair; given x twice, each lane ends up holding {x[l], x[l ^ 32]}.
__device__ __forceinline__ float xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const float a = __builtin_bit_cast(float, (uint32_t)r[0]), b = __builtin_bit_cast(float, (uint32_t)r[1]);
    // one of a, b is x itself; the other is the partner's value
    return __builtin_bit_cast(uint32_t, a) == __builtin_bit_cast(uint32_t, x) ? b : a;
}

// max(x[l], x[l ^ 32]) in every lane: v_permlane32_swap of x with itself leaves each
// lane the pair {x[l], x[l ^ 32]} (in one order or the other), whose max needs no
// selection.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Lazy-rescale threshold (log2 units): P never exceeds 2^kLazy = 256.
constexpr float kLazy = 8.0f;



// Device-coherent fp32 accesses for the split partials.  Agent-scope relaxed
// atomics are performed by gfx950 as global_store / global_load with sc1 (device
// scope): written through to, and read from, the point of coherence shared by all
// XCDs, so no L2 writeback or invalidate is needed to exchange them.  A 16-byte row
// is stored with that same instruction written out (one dwordx4 store instead of
// four dword stores: a quarter of the write transactions); stores return nothing,
// so the compiler's wait counters need not track them (finish_split waits for all
// of them before publishing).  A store of more than 8 bytes reads its data VGPRs
// after issue, so the asm ends with wait states before anything may overwrite them
// (the compiler adds these only after its own stores).  Loads stay
// compiler-generated, 4 bytes at a time.
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev4(float* p, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-KV merge, fused: every piece of a split query tile has written its fp32
// partial rows (O_s normalised by its own sum, and LSE_s) with device-coherent
// stores; once they are complete (s_waitcnt, then a workgroup barrier) one thread
// counts the piece done with an agent-scope atomic on the tile's split group.  The
// piece that arrives last reads the partials back with device-coherent loads,
// combines them with weights exp(LSE_s - max_s LSE_s), writes O and LSE, and resets
// the counter to 0 for the next run.  The combine order is fixed (s = 0, 1, ...), so
// the result does not depend on which piece arrives last.
template <int D, bool BF16>
__device__ __forceinline__ void finish_split(const AttnArgs& A, const Tile& T) {
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
    __syncthreads();                // ... and every other thread's
    if (threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(A.counters + T.group, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        is_last = done == T.n_splits - 1;
    }
    __syncthreads();
    if (!is_last) return;
    const int G = A.G;
    const int R = T.q_count * G;
    const int part0 = T.part - T.split * R;
    constexpr int D4 = D / 4;
    constexpr int NB = 8;  // pieces whose partials are loaded together (one memory round trip)
    for (int idx = threadIdx.x; idx < R * D4; idx += blockDim.x) {
        const int r = idx / D4, c4 = idx - r * D4;
        float mx = -INFINITY, wsum = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int sp0 = 0; sp0 < T.n_splits; sp0 += NB) {
            float l[NB];
            f32x4 v[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                l[k] = -INFINITY;
                v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (sp0 + k < T.n_splits) {
                    const int pr = part0 + (sp0 + k) * R + r;
                    const float* src = A.part_o + (int64_t)pr * D + 4 * c4;
                    l[k] = ld_dev(A.part_lse + pr);
                    v[k] = f32x4{ld_dev(src), ld_dev(src + 1), ld_dev(src + 2), ld_dev(src + 3)};
                }
            }
            float bm = mx;
#pragma unroll
            for (int k = 0; k < NB; ++k) bm = fmaxf(bm, l[k]);
            if (bm == -INFINITY) continue;
            const float sc = __expf(mx - bm);  // 0 while nothing has been merged yet
            acc *= sc;
            wsum *= sc;
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float w = __expf(l[k] - bm);  // 0 for a piece with no visible key
                acc += w * v[k];
                wsum += w;
            }
            mx = bm;
        }
        const float inv = 1.f / wsum;
        const int tok = r / G, g = r - tok * G;
        const int64_t orow = (int64_t)(T.q_row0 + tok) * A.H + T.kv_head * G + g;
        u32x2 w2;
        w2[0] = pack_out<BF16>(acc[0] * inv, acc[1] * inv);
        w2[1] = pack_out<BF16>(acc[2] * inv, acc[3] * inv);
        *(u32x2*)(A.o + orow * D + 4 * c4) = w2;
        if (A.lse && c4 == 0) A.lse[orow] = mx + __logf(wsum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(A.counters + T.group, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Unit slots in the wide tile's LDS ring: 4 lets a unit's loads overlap two units of
// compute at two workgroups per CU; 3 fits three workgroups per CU (three waves per
// SIMD) with one unit of overlap.
constexpr int kWideSlots = 3;
constexpr int kWideWavesPerEU = kWideSlots == 3 ? 3 : 2;

template <int D>
struct WideCfg {
    static constexpr int UK = 32;                            // keys per unit
    static constexpr int R = 1024 / (2 * D);                 // K (or V) rows per 1 KiB load group
    static constexpr int GS = 1024 + (D == 128 ? 64 : 128);  // LDS bytes per group (padded)
    static constexpr int NG = UK / R;                        // groups per matrix per unit
    static constexpr int IPW = NG / kWideWaves;              // loads per wave per matrix per unit
    static constexpr int MAT = NG * GS;                      // LDS bytes of one unit's K (or V)
    static constexpr int SLOT = 2 * MAT;                     // one unit: K then V
    static constexpr int NS = kWideSlots;                    // ring slots
    static constexpr int bytes = NS * SLOT;
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static_assert(IPW * kWideWaves == NG, "the waves share a unit's groups evenly");
};

template <int D>
struct NarrowLds {
    static constexpr int KW = kWaveKeys;  // keys per wave step
    static constexpr int VS = D + 16;     // V row stride (elements), 32-byte pad
    static constexpr int KS = D + 8;      // K row stride (elements), 16-byte pad (shares V's area)
    static constexpr int stage_bytes = kWaves * KW * VS * 2;
    static constexpr int combine_bytes = kWaves * 16 * (D + 4) * 4 + 2 * kWaves * 16 * 4;
    static constexpr int bytes = stage_bytes > combine_bytes ? stage_bytes : combine_bytes;
};

// Wide tile: up to block_m = 128 rows = 4 waves x 32 rows (token-major (token, qo
// head) pairs of one kv head); keys in units of 32.  A unit's K and V go from the
// cache straight into LDS (global_load_lds_dwordx4: each lane's 16 bytes land at
// base + 16 * lane), through a ring of NS = kWideSlots unit slots: unit u + NS - 1
// is requested while unit u is computed, and each wave waits for its own share of
// unit u + 2 before the barrier that ends unit u.  LDS layout of one matrix of a unit: groups of R = 1024 /
// (2D) rows, one load instruction each, stored chunk-major (16-byte chunk c of row r
// at 16 (R c + r)) with GS - 1024 bytes of padding after each group, so that the
// K^T operand reads (16-byte chunks of 16 rows) and the transposing V reads (8-byte
// pieces of 4 rows) fall on distinct banks.  V is read with ds_read_b64_tr_b16,
// which hands each lane 4 keys of one d: the V^T operand, with no transposing store.
// Each wave software-pipelines with one unit of lag between its two products: it
// issues Q K^T of unit u + 1, then P V of unit u with the softmax of unit u + 1
// interleaved product by product, so that its own exponentials run beside its own
// matrix work.  P V runs on fp16: bf16 V is converted in LDS, one unit ahead, by the
// wave that loaded it, and a barrier makes every wave's share visible before any
// wave's P V reads it.
template <int D, bool BF16>
__device__ __forceinline__ void wide_tile(const AttnArgs& A, const Tile& T, char* smem) {
    using C = WideCfg<D>;
    constexpr int R = C::R, GS = C::GS, MAT = C::MAT, SLOT = C::SLOT, IPW = C::IPW;
    constexpr int DK = D / 16;  // k-steps of Q K^T
    constexpr int DB = D / 32;  // 32-wide d blocks of O
    static_assert(kWideWaves == 4, "4 waves of 32 rows");
    // the page table through the constant address space: wave-uniform indices become
    // scalar loads, which leave the vector-memory counter to the K/V loads alone
    typedef __attribute__((address_space(4))) const int32_t const_i32;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int G = A.G;
    const int rows_valid = T.q_count * G;

    // This lane's query row: wave * 32 + col.
    const int row = wave * 32 + col;
    const int tok = row / G, g = row - tok * G;
    const bool row_ok = row < rows_valid;
    const int pos = T.pos0 + tok;
    const int64_t orow = (int64_t)(T.q_row0 + tok) * A.H + T.kv_head * G + g;
    // Q^T operand, 8 consecutive d per k-step, held for the whole tile.  Read from
    // memory in whole rows (16-byte chunk c of row 4i + l/16 by lane l, instruction i:
    // each instruction reads 4 rows of D * 2 contiguous bytes) and moved into the
    // operand layout through LDS in the prologue (qraw -> qf), since loads in the
    // operand layout would scatter every instruction over 32 rows.
    constexpr int QCH = D / 8;               // 16-byte chunks per row
    constexpr int QRPI = 64 / QCH;           // rows per load instruction
    constexpr int QI = 32 / QRPI;            // load instructions per wave
    // Rows past the tile's last one read its last row instead (unconditional loads, no
    // wait inside a branch); they are zeroed when the operand is formed.
    u32x4 qraw[QI];
    u32x4 qf[DK];
#pragma unroll
    for (int i = 0; i < QI; ++i) {
        const int rw = min(wave * 32 + QRPI * i + lane / QCH, rows_valid - 1);
        const int tk = rw / G, gh = rw - tk * G;
        const int64_t orw = (int64_t)(T.q_row0 + tk) * A.H + T.kv_head * G + gh;
        qraw[i] = *(const u32x4*)(A.q + orw * D + 8 * (lane % QCH));
    }
    const int wpos_min = T.pos0 + (wave * 32) / G;  // smallest position among this wave's rows

    // ---- loads of one unit into one ring slot ----
    // Wave w loads groups m = w + 4j (j < IPW) of K and of V: rows R m .. R m + R - 1
    // of the unit, all in one page.  Lane l: row R m + l % R, chunk l / R.
    const int64_t ss = (int64_t)A.Hkv * D;  // elements between token slots
    // The rows a wave's group takes within its page, (R m) % 16, do not depend on j
    // (4R j is a multiple of 16): they go into the wave's base pointer and the lane
    // offsets, so a load's address is base + page * page_bytes.
    const char* kvw = reinterpret_cast<const char*>(A.kv + (int64_t)T.kv_head * D + ((R * wave) & 15) * ss);
    const uint32_t page_bytes = (uint32_t)(32 * ss * 2);
    const uint32_t k_src_lane = (uint32_t)(((lane % R) * ss + 8 * (lane / R)) * 2);  // bytes
    const uint32_t v_src_lane = k_src_lane + (uint32_t)(16 * ss * 2);
    const int nunits = (T.kv_end - T.kv_begin + C::UK - 1) / C::UK;
    // Page of each of this wave's groups for one unit, read ahead (scalar loads, not
    // waited for here).  A group past kv_len reads page 0: its keys are masked and
    // their V zeroed.
    auto pages_of = [&](int t, int (&pg)[IPW]) {
        const int kv0 = T.kv_begin + C::UK * t;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int key0 = kv0 + R * (wave + 4 * j);
            pg[j] = key0 < T.kv_len ? ((const_i32*)A.page_idx)[T.page_base + (key0 >> 4)] : 0;
        }
    };
    // Request one unit into one slot.  A page index outside [0, num_pages) reads page
    // 0; bad_any then sends every later unit through the slow check in fix_unit, which
    // zeroes that page's keys, and raises the error flag after the key loop (a store
    // among the loads would make the compiler wait for them).
    const uint32_t lds_w = lds_addr(smem) + wave * GS;
    int bad_any = 0;
    auto load_unit = [&](int slot, const int (&pg)[IPW]) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            int p = pg[j];
            if ((unsigned)p >= (unsigned)A.num_pages) {
                p = 0;
                bad_any = 1;
            }
            const char* src = kvw + (uint64_t)(uint32_t)p * page_bytes;
            const uint32_t dst = lds_w + slot * SLOT + 4 * j * GS;
            load_lds16(src, k_src_lane, dst);
            load_lds16(src, v_src_lane, dst + MAT);
        }
    };
    // After this wave's loads of unit t have landed: zero V of keys past kv_len, and K
    // and V of bad pages (each lane the 16 bytes it loaded).
    auto fix_unit = [&](int t, int slot) {
        const int kv0 = T.kv_begin + C::UK * t;
        if (!bad_any && kv0 + C::UK <= T.kv_len) return;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int m = wave + 4 * j;
            const int key0 = kv0 + R * m;
            bool b = false;
            if (bad_any && key0 < T.kv_len) {
                const int p = ((const_i32*)A.page_idx)[T.page_base + (key0 >> 4)];
                b = (unsigned)p >= (unsigned)A.num_pages;
            }
            char* q = smem + slot * SLOT + m * GS + 16 * lane;
            if (b) *(u32x4*)q = u32x4{0, 0, 0, 0};
            if (b || key0 + lane % R >= T.kv_len) *(u32x4*)(q + MAT) = u32x4{0, 0, 0, 0};
        }
    };

    // bf16 V to fp16, in place: each lane the 16 bytes it loaded (P V runs on fp16, as
    // P keeps 11 bits there against bf16's 8).  Read and write are split so that other
    // work covers the read's latency.
    auto v_fp16_read = [&](int slot, u32x4 (&w)[IPW]) {
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < IPW; ++j)
                w[j] = *(const u32x4*)(smem + slot * SLOT + MAT + (wave + 4 * j) * GS + 16 * lane);
        }
    };
    // vmax: largest fp16 |V| pattern converted from bf16, over the units of this tile
    // (a slot converted past the last unit holds stale bytes and does not count)
    u16x2 vmax = {0, 0};
    auto v_fp16_write = [&](int slot, const u32x4 (&w)[IPW], bool live) {
        if constexpr (BF16) {
            u16x2 umax = {0, 0};
#pragma unroll
            for (int j = 0; j < IPW; ++j) {
                u32x4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = v_pair_fp16(w[j][e], umax);
                *(u32x4*)(smem + slot * SLOT + MAT + (wave + 4 * j) * GS + 16 * lane) = h;
            }
            if (live) vmax = __builtin_elementwise_max(vmax, umax);
        }
    };

    // ---- per-lane LDS read offsets (bytes, within a slot) ----
    // K^T operand of k-step kk: row col, chunk 2kk + half.
    const int k_lane = (col / R) * GS + 16 * (R * half + col % R);
    // V^T operand (tr16): key 16h + 8r + e8 (e8 = 4 half + (i >> 2), i = lane % 16),
    // d = 32db + 16 ((lane >> 4) & 1) + 4 (i & 3).
    const int vi = lane & 15, e8 = 4 * half + (vi >> 2);
    const int v_lane = MAT + (e8 / R) * GS + 16 * (R * (2 * ((lane >> 4) & 1) + ((vi & 3) >> 1)) + e8 % R) +
                       8 * (vi & 1);

    // ---- state ----
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // reference max of the scaled scores (log2 units)
    float lsum = 0.f;         // this lane's share of the row sum

    auto qk = [&](int slot, f32x16& S) {
        const char* kp = smem + slot * SLOT + k_lane;
        S = f32x16{};
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) S = mfma_qk(*(const u32x4*)(kp + 32 * R * kk), qf[kk], S, BF16);
    };

    int pg_next[IPW];   // pages of the next unit to request
    auto sync_unit = [&](int t, int slot, int younger) {
        // wait for this wave's loads of unit t; those of the `younger` units requested
        // after it (2 IPW loads each) may stay in flight
        switch (younger * 2 * IPW) {
            case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
            case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
            case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
            case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
            case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
            case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
            case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
            case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
            case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        }
        fix_unit(t, slot);
    };
    // units requested after unit t, up to unit last_req (the newest requested so far)
    auto younger_than = [&](int t, int last_req) {
        const int newest = last_req < nunits - 1 ? last_req : nunits - 1;
        return newest > t ? newest - t : 0;
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    auto ring = [](int x) { return x >= C::NS ? x - C::NS : x; };  // x mod NS, x < 2 NS
    constexpr int NS = C::NS;

    // Mask of unit t's scores S: keys past kv_len or past a row's position (boundary
    // units only).
    auto mask_unit = [&](int t, f32x16& S) {
        const int kv0 = T.kv_begin + C::UK * t;
        if ((kv0 + C::UK > T.kv_len) || (A.causal && kv0 + C::UK - 1 > wpos_min)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (key >= T.kv_len || (A.causal && key > pos)) S[r] = -INFINITY;
            }
        }
    };
    // Softmax of a unit's masked scores S, without a branch: the row max, the new
    // reference max (lazy: a row's moves only when its block max exceeds it by more
    // than kLazy) and the factor alpha that rescales what was accumulated against the
    // old one, the probabilities P = exp2(S c - m) in fp16 into pf, and the row sums
    // lsum = alpha lsum + sum P.  Returns alpha; O is rescaled by the caller once the
    // P V products that still use the old reference have been issued.
    auto softmax_unit = [&](f32x16& S, u32x4 (&pf)[2]) -> float {
        float bmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, S[r]);
        bmax = pair_max(bmax);
        const float bx = bmax * A.c_log2;
        const float m_new = bx > m_run + kLazy ? bx : m_run;
        const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        lsum *= alpha;
        const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * h + 2 * e], A.c_log2, nm));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * h + 2 * e + 1], A.c_log2, nm));
                const fp16x2 ph = __builtin_amdgcn_cvt_pkrtz(p0, p1);
                lsum = __builtin_amdgcn_fdot2(ph, fp16x2{(__fp16)1.0f, (__fp16)1.0f}, lsum, false);
                pf[h][e] = __builtin_bit_cast(uint32_t, ph);
            }
        return alpha;
    };
    constexpr int PF = 2;  // operands in flight ahead of the MFMA that uses them
    static_assert(DK == 2 * DB, "as many Q K^T as P V steps");
    // V^T operand of P V step i (keys 16 (i / DB) .., d block i % DB) of the unit in slot sl
    auto vread = [&](int sl, int i) {
        const char* vp = smem + sl * SLOT + v_lane;
        const int h = i / DB, db = i % DB;
        const u32x2 lo = ds_read_tr16((const uint16_t*)(vp + ((16 * h) / R) * GS + 64 * R * db));
        const u32x2 hi = ds_read_tr16((const uint16_t*)(vp + ((16 * h + 8) / R) * GS + 64 * R * db));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    // P V of the unit in slot sl with probabilities pf, each V operand read from LDS
    // ahead of its MFMA.
    auto pv_unit = [&](int sl, const u32x4 (&pf)[2]) {
        u32x4 vb[DK];
#pragma unroll
        for (int i = 0; i < PF; ++i) vb[i] = vread(sl, i);
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            if (i + PF < DK) vb[i + PF] = vread(sl, i + PF);
            oacc[i % DB] = mfma_pv(vb[i], pf[i / DB], oacc[i % DB]);
        }
    };

    // P V of the unit in slot sl with its probabilities p, interleaved with the softmax
    // of the next unit's masked scores S, whose probabilities replace them in p (the
    // same arithmetic, in the same order, as softmax_unit): after each product the
    // wave issues the product's next V operand reads and one slice of the softmax,
    // which runs while the product does.  The exponentials overwrite S; they are
    // packed into p[0] once the products that read p[0] have been issued, and into
    // p[1] after the last product.  The fences keep the compiler from regrouping the
    // slices.
    auto pv_softmax = [&](int sl, f32x16& S, u32x4 (&p)[2]) -> float {
        u32x4 vb[DK];
#pragma unroll
        for (int i = 0; i < PF; ++i) vb[i] = vread(sl, i);
        float bmax = -INFINITY, alpha = 1.f, nm = 0.f;
        // softmax slice k of DK: the row max over S[0..7], then over S[8..15] and the new
        // reference, then the exponentials of the 8 score pairs, spread over the DK - 2
        // remaining slices (pairs [8 (k - 2) / NE, 8 (k - 1) / NE)); slice K0, the first
        // after the products of p[0] and after the exponentials of pairs 0..3, packs them
        constexpr int NE = DK - 2;
        constexpr int K3 = 1 + (NE + 1) / 2;  // slice whose exponentials end with pair 3
        constexpr int K0 = DB > K3 ? DB : K3;
        static_assert(NE >= 1 && K0 < DK, "a slice of exponentials, and pairs 0..3 packed in the loop");
        auto pack = [&](int h) {  // pairs 4h .. 4h + 3 to fp16 into p[h], row sums in order
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const fp16x2 ph = __builtin_amdgcn_cvt_pkrtz(S[8 * h + 2 * e], S[8 * h + 2 * e + 1]);
                lsum = __builtin_amdgcn_fdot2(ph, fp16x2{(__fp16)1.0f, (__fp16)1.0f}, lsum, false);
                p[h][e] = __builtin_bit_cast(uint32_t, ph);
            }
        };
        auto slice = [&](int k) {
            if (k == 0) {
#pragma unroll
                for (int r = 0; r < 8; ++r) bmax = fmaxf(bmax, S[r]);
            } else if (k == 1) {
#pragma unroll
                for (int r = 8; r < 16; ++r) bmax = fmaxf(bmax, S[r]);
                bmax = pair_max(bmax);
                const float bx = bmax * A.c_log2;
                const float m_new = bx > m_run + kLazy ? bx : m_run;
                alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                lsum *= alpha;
                nm = m_run == -INFINITY ? 0.f : -m_run;
            } else {
#pragma unroll
                for (int q = 8 * (k - 2) / NE; q < 8 * (k - 1) / NE; ++q) {
                    S[2 * q] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * q], A.c_log2, nm));
                    S[2 * q + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * q + 1], A.c_log2, nm));
                }
            }
            if (k == K0) pack(0);
        };
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            if (i + PF < DK) vb[i + PF] = vread(sl, i + PF);
            oacc[i % DB] = mfma_pv(vb[i], p[i / DB], oacc[i % DB]);
            __builtin_amdgcn_sched_barrier(0);
            slice(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        pack(1);
        return alpha;
    };

    // Iteration u (slot SL = u % NS, unit u + 1 exists) enters with unit u's
    // probabilities in p (its row sums already in lsum), K of unit u + 1 and V of unit
    // u (fp16) in LDS, and V of unit u + 1 landed as loaded:
    //   A: request unit u + NS - 1 into the slot unit u - 1 has left; Q K^T of unit
    //      u + 1 into S, beside the fp16 conversion of V of unit u + 1;
    //   B: P V of unit u, beside the softmax of unit u + 1 into p: one basic block, so
    //      a wave's exponentials issue while its own matrix products run;
    //   then O is rescaled where a row's reference moved, and the wave waits for its
    //   loads of unit u + 2 and meets the others at the barrier, which also makes the
    //   converted V of unit u + 1 visible to every wave.
    auto unit = [&](int u, int SL, f32x16& S, u32x4 (&p)[2]) {
        u32x4 vcv[IPW];
        v_fp16_read(ring(SL + 1), vcv);
        if (u + NS - 1 < nunits) load_unit(ring(SL + NS - 1), pg_next);
        {
            const char* kp = smem + ring(SL + 1) * SLOT + k_lane;
            auto kread = [&](int kk) { return *(const u32x4*)(kp + 32 * R * kk); };
            u32x4 kb[DK];
#pragma unroll
            for (int i = 0; i < PF; ++i) kb[i] = kread(i);
            S = f32x16{};
#pragma unroll
            for (int i = 0; i < DK; ++i) {
                if (i + PF < DK) kb[i + PF] = kread(i + PF);
                S = mfma_qk(kb[i], qf[i], S, BF16);
            }
        }
        v_fp16_write(ring(SL + 1), vcv, true);
        mask_unit(u + 1, S);
        const float alpha = pv_softmax(SL, S, p);
        // (keeps the exponentials in this block, beside the P V products, rather than
        // sunk past the rescale branch below)
        asm volatile("" ::"v"(p[0]), "v"(p[1]), "v"(lsum));
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        // pages of unit u + NS (their latency overlaps the wait below)
        if (u + NS < nunits) pages_of(u + NS, pg_next);
        if (u + 2 < nunits) {
            // unit u + 2 must be in LDS (and slot SL free) before unit u + 1's iteration
            sync_unit(u + 2, ring(SL + 2), younger_than(u + 2, u + NS - 1));
            barrier();
        } else if (BF16) {
            barrier();  // the last unit's V, converted above by every wave
        }
    };

    if (nunits > 0) {
        // ---- prologue: units 0 .. NS-2 requested, 0 and 1 landed, scores of unit 0 ----
        {
            int pg[IPW];
#pragma unroll
            for (int t = 0; t < NS - 1; ++t)
                if (t < nunits) {
                    pages_of(t, pg);
                    load_unit(t, pg);
                }
            if (NS - 1 < nunits) pages_of(NS - 1, pg_next);
            sync_unit(0, 0, younger_than(1, NS - 2));
            if (nunits > 1) sync_unit(1, 1, younger_than(1, NS - 2));
            u32x4 vcv[IPW];
            v_fp16_read(0, vcv);
            v_fp16_write(0, vcv, true);
            // Q rows into the operand layout, through ring slot NS - 1 (no unit is
            // requested into it before the barrier below): 16 rows per wave at a time,
            // at a stride of D * 2 + 16 bytes (conflict-free 16-byte reads).
            {
                constexpr int QS = D + 8;  // staged row stride (elements)
                static_assert(kWideWaves * 16 * QS * 2 <= SLOT, "Q staging fits one ring slot");
                uint16_t* qs = reinterpret_cast<uint16_t*>(smem + (NS - 1) * SLOT) + wave * 16 * QS;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int i = 0; i < QI / 2; ++i) {
                        const int r = QRPI * i + lane / QCH;  // row within this half
                        *(u32x4*)(qs + r * QS + 8 * (lane % QCH)) = qraw[h * (QI / 2) + i];
                    }
                    if ((col >> 4) == h)
#pragma unroll
                        for (int kk = 0; kk < DK; ++kk)
                            qf[kk] = *(const u32x4*)(qs + (col & 15) * QS + 16 * kk + 8 * half);
                }
#pragma unroll
                for (int kk = 0; kk < DK; ++kk)
                    if (!row_ok) qf[kk] = u32x4{0, 0, 0, 0};
            }
            barrier();
        }
        // One score buffer (unit u + 1's Q K^T starts once unit u's exponentials have
        // used its scores up) and one probability buffer (each half refilled once the
        // products that read it have been issued).
        f32x16 sc;
        u32x4 pf[2];
        qk(0, sc);
        mask_unit(0, sc);
        softmax_unit(sc, pf);  // nothing accumulated yet: no rescale
        int u = 0, sl = 0;
        for (; u + 1 < nunits; ++u, sl = ring(sl + 1)) unit(u, sl, sc, pf);
        pv_unit(sl, pf);
    }

    if (bad_any && lane == 0) raise_flag(A.err_flag, kErrPage);
    if constexpr (BF16) flag_v_range(A.err_flag, vmax);

    // ---- epilogue ----
    const float ltot = lsum + xor32(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const float lse_val = ltot > 0.f ? (m_run + __log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
    if (T.part < 0) {
        // O through LDS, so that 16 lanes store one row's D * 2 contiguous bytes: in
        // the MFMA layout a lane holds 4-element pieces of one row, and storing them
        // directly scatters every store instruction over 32 rows.  Each wave stages
        // its 32 rows in its own part of the ring, which every wave has finished with
        // at the barrier.
        constexpr int OSTR = D + 8;  // staged row stride (elements): 16-byte pad
        static_assert(kWideWaves * 32 * OSTR * 2 <= C::bytes, "O staging fits the ring");
        __syncthreads();
        uint16_t* ost = reinterpret_cast<uint16_t*>(smem) + wave * 32 * OSTR;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                u32x2 w;
                w[0] = pack_out<BF16>(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
                w[1] = pack_out<BF16>(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
                *(u32x2*)(ost + col * OSTR + 32 * db + 8 * jj + 4 * half) = w;
            }
        constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
        for (int i = 0; i < 32 * CPR / 64; ++i) {
            const int idx = 64 * i + lane, r = idx / CPR, c = idx - r * CPR;
            const int rw = wave * 32 + r;
            if (rw < rows_valid) {
                const int tk = rw / G, gh = rw - tk * G;
                const int64_t orw = (int64_t)(T.q_row0 + tk) * A.H + T.kv_head * G + gh;
                *(u32x4*)(A.o + orw * D + 8 * c) = *(const u32x4*)(ost + r * OSTR + 8 * c);
            }
        }
        if (row_ok && A.lse && half == 0) A.lse[orow] = lse_val;
    } else if (row_ok) {
        float* pp = A.part_o + ((int64_t)T.part + row) * D + 4 * half;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 w = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv, oacc[db][4 * jj + 2] * inv,
                           oacc[db][4 * jj + 3] * inv};
                st_dev4(pp + 32 * db + 8 * jj, w);
            }
        if (half == 0) st_dev(A.part_lse + T.part + row, lse_val);
    }
    if (T.part >= 0) finish_split<D, BF16>(A, T);
}


// Keys of one 32-key step of a narrow tile (wave-uniform).  An ordinary tile: first
// key's position, keys that exist from it (masked at or past this count), offset of
// its first page id in kv_page_indices.  A kGroup tile, per 16-key block b: keys that
// exist in it (bv), the offset of its page id (bp) and the member whose rows alone
// see it (bo; -1: all rows).
struct StepKeys {
    int key0, valid, pidx;
    int bv[2], bp[2], bo[2];
};

// Combine of the 4 waves of a narrow tile (each walked its own keys) and the tile's
// output: c_o holds each wave's unnormalised O rows ([wave * 16 + row][D + 4] fp32),
// c_m / c_l its running max (log2 units) and sum per row.  Writes O (and LSE), or
// the split partials followed by the fused merge.
template <int D, bool BF16>
__device__ __forceinline__ void narrow_combine_store(const AttnArgs& A, const Tile& T, const float* c_o,
                                                     const float* c_m, const float* c_l, int rows_valid) {
    constexpr int OS = D + 4;
    constexpr int D4 = D / 4;
    const int G = A.G;
    for (int idx = threadIdx.x; idx < 16 * D4; idx += blockDim.x) {
        const int r = idx / D4, c4 = idx - r * D4;
        if (r >= rows_valid) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, c_m[w * 16 + r]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = __builtin_amdgcn_exp2f(c_m[w * 16 + r] - Mu);
            L += wt * c_l[w * 16 + r];
            acc += wt * *(const f32x4*)(c_o + (w * 16 + r) * OS + 4 * c4);
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const float lse_val = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
        const int rt = r / G, rg = r - rt * G;
        const int64_t orow_r = (int64_t)(T.q_row0 + rt) * A.H + T.kv_head * G + rg;
        if (T.part < 0) {
            u32x2 w2;
            w2[0] = pack_out<BF16>(acc[0] * inv, acc[1] * inv);
            w2[1] = pack_out<BF16>(acc[2] * inv, acc[3] * inv);
            *(u32x2*)(A.o + orow_r * D + 4 * c4) = w2;
            if (A.lse && c4 == 0) A.lse[orow_r] = lse_val;
        } else {
            st_dev4(A.part_o + ((int64_t)T.part + r) * D + 4 * c4, acc * inv);
            if (c4 == 0) st_dev(A.part_lse + T.part + r, lse_val);
        }
    }
    if (T.part >= 0) finish_split<D, BF16>(A, T);
}

// Narrow tile (decode-like): at most 16 rows (q_count * G <= 16), all in one
// 16-column MFMA block.  The 4 waves split the key range: wave w takes the
// kWaveKeys-key steps w, w+4, w+8, ... of [kv_begin, kv_end), each with its own running max,
// sum and O, and the waves are combined through LDS at the end.
//   * K goes into the A operand of v_mfma_f32_16x16x32 (lane l: key 16b + l%16, 8
//     consecutive d) either in whole rows through the wave's LDS area (KROWS; each
//     load instruction reads KPJ complete rows -- loads that touch 16 half rows
//     each made shared-prefix decode 14% slower) or, when the plan splits narrow
//     tiles and the last step sits on the merge's critical path, straight from
//     memory into the operand registers;
//   * page ids are scalar loads requested a step ahead, K/V loads carry no
//     condition, and Q is staged through LDS before the key loop, so that the
//     compiler's waits in the loop are exact (see the body);
//   * V is staged in its natural [key][d] layout (fp16; bf16 is converted on the
//     way) and read back transposed with ds_read_b64_tr_b16: within each 16-lane
//     group, lane j receives element j%4 of the 8-byte rows addressed by lanes
//     j/4 + 4m (m = 0..3), which turns 4 rows of 4 consecutive d into 4 keys of
//     one d per lane -- the V^T operand layout;
//   * S^T = K Q^T gives each lane one row (column l%16) and 4 consecutive keys per
//     16-key block; the running max needs two cross-lane exchanges per step.
template <int D, bool BF16, bool KROWS, bool NT, bool GROUP>
__device__ __forceinline__ void narrow_tile(const AttnArgs& A, const Tile& T, char* smem) {
    constexpr int KW = NarrowLds<D>::KW;  // keys per wave step
    constexpr int VS = NarrowLds<D>::VS;  // V staging row stride (elements)
    constexpr int KS = NarrowLds<D>::KS;  // K staging row stride (elements)
    constexpr int DK = D / 32;            // 32-d k-steps of Q K^T
    constexpr int DB = D / 16;            // 16-d blocks of O^T
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int KPJ = 64 / CH;          // keys per V load instruction
    constexpr int VJ = KW / KPJ;          // V loads per lane per step
    constexpr int KB = KW / 16;           // 16-key blocks per step
    // the page table through the constant address space: wave-uniform indices become
    // scalar loads, counted apart from the K/V loads
    typedef __attribute__((address_space(4))) const int32_t const_i32;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int G = A.G;
    const int rows_valid = T.q_count * G;
    const int row = col;
    const int tok = row / G;
    const bool row_ok = row < rows_valid;
    const int pos = T.pos0 + tok;
    const int pos_min = T.pos0;
    uint16_t* v_lds = reinterpret_cast<uint16_t*>(smem) + wave * KW * VS;

    // Q^T operand (B of 16x16x32): row `col`, d = 32kk + 8grp .. +8.  Read in whole
    // rows (16-byte chunk c of row QRPI i + l / CH by lane l, instruction i) and moved
    // into the operand layout through the wave's LDS area once the first K/V loads
    // are requested: Q is then in registers before the key loop, so the compiler's
    // waits inside the loop count only the loop's own loads.
    constexpr int QRPI = 64 / CH;  // rows per Q load instruction
    constexpr int QI = 16 / QRPI;  // Q load instructions (16 rows)
    // (rows past the tile's last one read its last row instead -- unconditional loads,
    // no wait inside a branch -- and are zeroed when the operand is formed)
    u32x4 qraw[QI];
#pragma unroll
    for (int i = 0; i < QI; ++i) {
        const int r = min(QRPI * i + lane / CH, rows_valid - 1);
        const int tk = r / G, gh = r - tk * G;
        const int64_t orw = (int64_t)(T.q_row0 + tk) * A.H + T.kv_head * G + gh;
        qraw[i] = *(const u32x4*)(A.q + orw * D + 8 * (lane % CH));
    }
    // keep the Q loads ahead of the first K/V loads (no memory access moves across an
    // asm statement that clobbers memory), so that staging Q waits for Q alone
    asm volatile("" ::: "memory");
    u32x4 qf[DK];

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    int v_big = 0;  // a bf16 V above 65504 was converted (wave-uniform; bf16 only)

    const int64_t ss = (int64_t)A.Hkv * D;  // elements between token slots
    const uint16_t* kvh = A.kv + (int64_t)T.kv_head * D;
    const int vkey = lane / CH, vch = lane % CH;  // K/V gather: key j*KPJ + vkey, chunk vch

    // Gathers for one step: page ids (scalar loads, requested one step ahead), then K
    // and V into registers with unconditional loads, so that the compiler's wait
    // counts stay exact and step n's V can still be in flight while step n's Q K^T
    // waits for its K.  A 16-key block at or past kv_len reads page 0 (valid memory,
    // its keys are masked and their V zeroed once landed); a page index outside
    // [0, num_pages) raises the error flag and its keys read as zero K and V.
    constexpr int STRIDE = kWaves * KW;
    // The keys of the step at (virtual) key v, wave-uniform.  An ordinary tile walks
    // its own keys: v is the key; keys at or past `valid` are masked and their V
    // zeroed.  A kGroup tile walks 16-key page slots, blocks 2 v / 32 and 2 v / 32 + 1:
    // the kv_len / 16 shared pages, then pos0 pages per member over that member's keys
    // past the prefix (page base and length from the sequence table, scalar loads);
    // slots past a member's keys or past the last member are empty.
    static_assert(KB == 2, "two 16-key blocks per step");
    auto step_keys = [&](int v) -> StepKeys {
        if constexpr (!GROUP) {
            return StepKeys{v, T.kv_len - v, T.page_base + (v >> 4), {0, 0}, {0, 0}, {-1, -1}};
        } else {
            StepKeys sk{v, 0, 0, {0, 0}, {0, 0}, {-1, -1}};
            // past the last step (the first step of a wave with no keys): nothing to read
            if (v >= T.kv_end) return sk;
            const int SP = T.kv_len >> 4, NP = T.q_count * T.pos0;  // shared pages, private slots
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const int slot = (v >> 4) + b;
                if (slot < SP) {
                    sk.bv[b] = 16;
                    sk.bp[b] = T.page_base + slot;
                } else if (slot < SP + NP) {  // here pos0 > 0
                    const int i = (slot - SP) / T.pos0, pp = slot - SP - i * T.pos0;
                    const int pb = ((const_i32*)A.seqtab)[2 * (T.seq + i)];
                    const int kvl = ((const_i32*)A.seqtab)[2 * (T.seq + i) + 1];
                    const int key = T.kv_len + 16 * pp;
                    sk.bv[b] = min(16, kvl - key);
                    sk.bp[b] = pb + (key >> 4);
                    sk.bo[b] = i;
                }
            }
            return sk;
        }
    };
    auto pages_of = [&](const StepKeys& sk, int (&pg)[KB]) {
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if constexpr (GROUP)
                pg[b] = sk.bv[b] > 0 ? ((const_i32*)A.page_idx)[sk.bp[b]] : 0;
            else
                pg[b] = sk.key0 + 16 * b < T.kv_len ? ((const_i32*)A.page_idx)[T.page_base + (sk.key0 >> 4) + b] : 0;
        }
    };
    // Bad pages of a step: bit b set for block b (wave-uniform); such blocks read page 0.
    // The error flag is written once after the key loop: a store between the loads
    // would make the compiler wait for all of them (stores share their counter).
    int bad_seen = 0;
    auto check_pages = [&](int (&pg)[KB]) {
        int bad = 0;
#pragma unroll
        for (int b = 0; b < KB; ++b)
            if ((unsigned)pg[b] >= (unsigned)A.num_pages) {
                bad |= 1 << b;
                pg[b] = 0;
            }
        bad_seen |= bad;
        return bad;
    };
    u32x4 kr[VJ];      // K rows (KROWS)
    u32x4 kf[KB][DK];  // K in MFMA operand layout
    u32x4 vf[VJ];
    auto load_k = [&](const int (&pg)[KB]) {
        if constexpr (KROWS) {
#pragma unroll
            for (int j = 0; j < VJ; ++j) {
                const int key = j * KPJ + vkey;
                kr[j] = ld_kv<NT>(kvh + ((int64_t)pg[(j * KPJ) >> 4] * 32 + (key & 15)) * ss + 8 * vch);
            }
        } else {
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const uint16_t* src = kvh + ((int64_t)pg[b] * 32 + col) * ss + 8 * grp;
#pragma unroll
                for (int kk = 0; kk < DK; ++kk) kf[b][kk] = ld_kv<NT>(src + 32 * kk);
            }
        }
    };
    auto load_v = [&](const int (&pg)[KB]) {
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            const int key = j * KPJ + vkey;  // key within the step; its page is pg[key / 16]
            vf[j] = ld_kv<NT>(kvh + ((int64_t)pg[(j * KPJ) >> 4] * 32 + 16 + (key & 15)) * ss + 8 * vch);
        }
    };
    // Landed V of a step: zero keys at or past kv_len and keys of bad pages (a mask,
    // not a branch, so that each load is waited for on its own).
    auto fix_v = [&](const StepKeys& sk, int bad) {
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            const bool past = GROUP ? ((j * KPJ + vkey) & 15) >= sk.bv[(j * KPJ) >> 4]
                                    : sk.key0 + j * KPJ + vkey >= T.kv_len;
            const bool z = (bad & (1 << ((j * KPJ) >> 4))) || past;
            const uint32_t keep = z ? 0u : ~0u;
            vf[j] &= u32x4{keep, keep, keep, keep};
        }
    };

    // Software pipeline: while step n is computed, step n+1's K (issued right after
    // step n's Q K^T) and V (issued right after step n's V is staged) are in flight,
    // and step n+2's page ids are requested.
    int kbase = T.kv_begin + wave * KW;
    int pg_cur[KB], pg_nxt[KB];
    StepKeys sk_cur = step_keys(kbase), sk_nxt = sk_cur;
    int bad_cur = 0, bad_nxt = 0;
    // First step's loads, unconditional: a wave with no keys (a tile of fewer than
    // kWaves * KW keys) reads page 0 and never uses it.  A branch here would leave the
    // compiler, where its two paths join, waiting for every load in flight.
    pages_of(sk_cur, pg_cur);
    bad_cur = check_pages(pg_cur);
    load_k(pg_cur);
    load_v(pg_cur);
    if (kbase + STRIDE < T.kv_end) {
        sk_nxt = step_keys(kbase + STRIDE);
        pages_of(sk_nxt, pg_nxt);
    }
    // (kGroup tiles carry the descriptors of the current and next steps, which cost
    // scalar loads; an ordinary tile recomputes its own from the key position.)
    // Q into the MFMA operand layout through the wave's LDS area (free until its first
    // step), while those loads are in flight.
    static_assert(16 * KS <= KW * VS, "Q staging fits the wave's area");
#pragma unroll
    for (int i = 0; i < QI; ++i) *(u32x4*)(v_lds + (QRPI * i + lane / CH) * KS + 8 * (lane % CH)) = qraw[i];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qf[kk] = row_ok ? *(const u32x4*)(v_lds + col * KS + 32 * kk + 8 * grp) : u32x4{0, 0, 0, 0};
    // One step at key kbase; MORE: a next step exists and its loads are issued here.  The
    // last step is a separate copy, so that in the others every load is unconditional and
    // the compiler waits for exactly the loads each use needs.
    auto step = [&](int kbase, auto more_tag) {
        constexpr bool more = decltype(more_tag)::value;
        const int knext = kbase + STRIDE;
        const StepKeys cur = GROUP ? sk_cur : step_keys(kbase);

        // ---- (KROWS) K through the wave's LDS area: rows in, MFMA operands out (lane:
        // key 16b + col, d = 32kk + 8grp .. +8); V reuses the area after Q K^T ----
        if constexpr (KROWS) {
#pragma unroll
            for (int j = 0; j < VJ; ++j) *(u32x4*)(v_lds + (j * KPJ + vkey) * KS + 8 * vch) = kr[j];
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int kk = 0; kk < DK; ++kk)
                    kf[b][kk] = *(const u32x4*)(v_lds + (16 * b + col) * KS + 8 * grp + 32 * kk);
        }

        // ---- S^T = K Q^T ----
        f32x4 s[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            s[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) s[b] = mfma16_qk(kf[b][kk], qf[kk], s[b], BF16);
        }
        // keys of a bad page count as zero K: score 0 (K registers are not zeroed, which
        // would have to wait for their loads)
        if (bad_cur)
#pragma unroll
            for (int b = 0; b < KB; ++b)
                if (bad_cur & (1 << b)) s[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (more) {
            bad_nxt = check_pages(pg_nxt);
            load_k(pg_nxt);
        }

        // ---- stage V (fp16, natural layout) ----
        if (bad_cur || (GROUP ? cur.bv[0] < 16 || cur.bv[1] < 16 : kbase + KW > T.kv_len)) fix_v(cur, bad_cur);
        u16x2 vmax = {0, 0};  // largest fp16 |V| pattern of this step (bf16 only)
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            u32x4 w = vf[j];
            if (BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = v_pair_fp16(vf[j][e], vmax);
            }
            *(u32x4*)(v_lds + (j * KPJ + vkey) * VS + 8 * vch) = w;
        }
        if (BF16) v_big |= wave_v_big(vmax);
        if constexpr (more) {
            load_v(pg_nxt);
            bad_cur = bad_nxt;
            if constexpr (GROUP) sk_cur = sk_nxt;
            if (knext + STRIDE < T.kv_end) {
                if constexpr (GROUP) {
                    sk_nxt = step_keys(knext + STRIDE);
                    pages_of(sk_nxt, pg_nxt);
                } else {
                    pages_of(step_keys(knext + STRIDE), pg_nxt);
                }
            }
        }

        // ---- online softmax (lane: row `col`, keys 16b + 4grp + i) ----
        // (kGroup rows are decode rows: every key of their steps is at or before their
        // position, so only members and the valid count mask them)
        const bool need_mask = GROUP ? cur.bv[0] < 16 || cur.bv[1] < 16 || cur.bo[0] >= 0 || cur.bo[1] >= 0
                                     : (kbase + KW > T.kv_len) || (A.causal && kbase + KW - 1 > pos_min);
        float bmax = -INFINITY;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[b][i] * A.c_log2;
                if (need_mask) {
                    if constexpr (GROUP) {
                        const int koff = 4 * grp + i;  // within block b
                        if (koff >= cur.bv[b] || (cur.bo[b] >= 0 && tok != cur.bo[b])) x = -INFINITY;
                    } else {
                        const int key = kbase + 16 * b + 4 * grp + i;
                        if (key >= T.kv_len || (A.causal && key > pos)) x = -INFINITY;
                    }
                }
                s[b][i] = x;
                bmax = fmaxf(bmax, x);
            }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        const float m_new = fmaxf(m, bmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(s[b][i] - m_use);
                lsum += p;
                s[b][i] = p;
            }
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

        // ---- O^T += V^T P^T, 32 keys per MFMA ----
#pragma unroll
        for (int h = 0; h < KW / 32; ++h) {
            // P^T operand: logical k = 8grp + e <-> key 32h + 16(e/4) + 4grp + e%4
            u32x4 pf;
            pf[0] = pack_p(s[2 * h][0], s[2 * h][1]);
            pf[1] = pack_p(s[2 * h][2], s[2 * h][3]);
            pf[2] = pack_p(s[2 * h + 1][0], s[2 * h + 1][1]);
            pf[3] = pack_p(s[2 * h + 1][2], s[2 * h + 1][3]);
            const uint16_t* vrow0 = v_lds + (32 * h + 4 * grp + (col >> 2)) * VS + 4 * (col & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                u32x4 va;
                const u32x2 lo = ds_read_tr16(vrow0 + 16 * db);
                const u32x2 hi = ds_read_tr16(vrow0 + 16 * VS + 16 * db);
                va[0] = lo[0];
                va[1] = lo[1];
                va[2] = hi[0];
                va[3] = hi[1];
                oacc[db] = mfma16_pv(va, pf, oacc[db]);
            }
        }
    };
    for (; kbase + STRIDE < T.kv_end; kbase += STRIDE) step(kbase, std::true_type{});
    if (kbase < T.kv_end) step(kbase, std::false_type{});

    if (bad_seen && lane == 0) raise_flag(A.err_flag, kErrPage);
    if (v_big && lane == 0) raise_flag(A.err_flag, kErrVRange);

    // ---- combine the 4 waves ----
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    __syncthreads();  // every wave is done with its V staging area
    constexpr int OS = D + 4;  // fp32 row stride of the combine area
    float* c_o = reinterpret_cast<float*>(smem);
    float* c_m = c_o + kWaves * 16 * OS;
    float* c_l = c_m + kWaves * 16;
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)(c_o + (wave * 16 + col) * OS + 16 * db + 4 * grp) = oacc[db];
    if (grp == 0) {
        c_m[wave * 16 + col] = m;
        c_l[wave * 16 + col] = lsum;
    }
    __syncthreads();
    narrow_combine_store<D, BF16>(A, T, c_o, c_m, c_l, rows_valid);
}

// Narrow tile on the VALU, without MFMA: the decode design of the pages' GPUs,
// where decode runs on the CUDA cores and prefill on the tensor cores (flashinfer
// issue #323, "How are prefill and decode kernels different?"), kept for
// comparison with the MFMA narrow kernel.  At most RM <= 8 rows; the 4 waves split
// the key range in 32-key steps (wave w takes steps w, w+4, ...).  Lane layout:
// lane = LPR * g + j, LPR = D / 8 lanes per K/V row (j: d = 8j .. 8j+7) and
// KPI = 64 / LPR keys per load instruction (g: which key).
//   * Q is pinned in VGPRs: each lane holds its 8 d of every row;
//   * scores: per key, 4 dot2 per row, then a reduce-scatter over the key's LPR
//     lanes (halving exchanges), after which each lane holds one row's score;
//   * P and the per-row rescale factors go through LDS ([key][row]) and are read
//     back as broadcasts;
//   * O: each lane accumulates its 8 d of every row over its keys, fp32 FMAs; the
//     KPI key groups are summed once at the end;
//   * page ids are read a step ahead by scalar loads; a step's K and V are
//     requested at its start (carrying the next step's K/V in registers across the
//     step, as the MFMA narrow kernel does, costs this kernel a wave per SIMD).
template <int D, bool BF16, int RM>
__device__ __forceinline__ void valu_tile(const AttnArgs& A, const Tile& T, char* smem) {
    constexpr int LPR = D / 8;
    constexpr int KPI = 64 / LPR;
    constexpr int KW = kValuKeys;
    constexpr int NI = KW / KPI;
    constexpr int KB = KW / 16;  // pages per step
    static_assert(RM <= LPR && KW % KPI == 0, "lane layout");
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane / LPR, j = lane % LPR;
    const int G = A.G;
    const int rows_valid = T.q_count * G;
    int my_row = 0;  // the row whose score this lane holds after the reduce-scatter
#pragma unroll
    for (int dl = LPR / 2, half = RM / 2; dl >= 1 && half >= 1; dl /= 2, half /= 2)
        if (j & dl) my_row += half;
    const int my_pos = T.pos0 + my_row / G;
    const int pos_min = T.pos0;

    u32x4 qv[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        const int tok = r / G, gh = r - tok * G;
        const int64_t orow = (int64_t)(T.q_row0 + tok) * A.H + T.kv_head * G + gh;
        qv[r] = r < rows_valid ? *(const u32x4*)(A.q + orow * D + 8 * j) : u32x4{0, 0, 0, 0};
    }
    float oacc[RM][8];
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[r][e] = 0.f;
    float m = -INFINITY, lsum = 0.f;
    float* p_lds = reinterpret_cast<float*>(smem) + wave * (KW * RM + RM);  // [KW][RM], then alpha[RM]
    float* a_lds = p_lds + KW * RM;
    const int64_t ss = (int64_t)A.Hkv * D;
    const uint16_t* kvh = A.kv + (int64_t)T.kv_head * D + 8 * j;

    // Page ids by scalar loads one step ahead; a step's K and V are requested at its
    // start with unconditional loads (a 16-key block at or past kv_len reads page 0,
    // its keys are masked and their V zeroed; a bad page id zeroes its keys' scores
    // and V and raises the error flag after the loop).
    constexpr int STRIDE = kWaves * KW;
    int bad_seen = 0;
    auto pages_of = [&](int kb0, int (&pg)[KB]) {
#pragma unroll
        for (int b = 0; b < KB; ++b)
            pg[b] = kb0 + 16 * b < T.kv_len ? ((const_i32*)A.page_idx)[T.page_base + (kb0 >> 4) + b] : 0;
    };
    auto check_pages = [&](int (&pg)[KB]) {
        int bad = 0;
#pragma unroll
        for (int b = 0; b < KB; ++b)
            if ((unsigned)pg[b] >= (unsigned)A.num_pages) {
                bad |= 1 << b;
                pg[b] = 0;
            }
        bad_seen |= bad;
        return bad;
    };
    u32x4 kr[NI], vr[NI];
    auto load_k = [&](const int (&pg)[KB]) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int kl = KPI * i + g;  // key within the step
            kr[i] = *(const u32x4*)(kvh + ((int64_t)pg[(KPI * i) >> 4] * 32 + (kl & 15)) * ss);
        }
    };
    auto load_v = [&](const int (&pg)[KB]) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int kl = KPI * i + g;
            vr[i] = *(const u32x4*)(kvh + ((int64_t)pg[(KPI * i) >> 4] * 32 + 16 + (kl & 15)) * ss);
        }
    };
    int kbase = T.kv_begin + wave * KW;
    int pg_nxt[KB];
    if (kbase < T.kv_end) pages_of(kbase, pg_nxt);
    for (; kbase < T.kv_end; kbase += STRIDE) {
        const int knext = kbase + STRIDE;
        const int bad_cur = check_pages(pg_nxt);
        load_k(pg_nxt);
        load_v(pg_nxt);
        if (knext < T.kv_end) pages_of(knext, pg_nxt);
        // ---- scores ----
        float sv[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float part[RM];
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // element copies first: __builtin_bit_cast of a vector-element
                    // expression is compiled as a read of element 0
                    const uint32_t qe = qv[r][e], ke = kr[i][e];
                    if (BF16)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qe),
                                                              __builtin_bit_cast(bf16x2, ke), acc, false);
                    else
                        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, qe), __builtin_bit_cast(fp16x2, ke),
                                                     acc, false);
                }
                part[r] = acc;
            }
            int len = RM;
#pragma unroll
            for (int dl = LPR / 2; dl >= 1; dl /= 2) {
                if (len > 1) {
                    const int half = len / 2;
                    const bool bit = (j & dl) != 0;
#pragma unroll
                    for (int t = 0; t < half; ++t) {
                        const float send = bit ? part[t] : part[half + t];
                        const float keep = bit ? part[half + t] : part[t];
                        part[t] = keep + __shfl_xor(send, dl);
                    }
                    len = half;
                } else {
                    part[0] += __shfl_xor(part[0], dl);
                }
            }
            sv[i] = part[0];
        }
        // keys of a bad page count as zero K: score 0
        if (bad_cur)
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (bad_cur & (1 << ((KPI * i) >> 4))) sv[i] = 0.f;
        // ---- online softmax of this lane's row over the step's keys ----
        const bool need_mask = (kbase + KW > T.kv_len) || (A.causal && kbase + KW - 1 > pos_min);
        float bmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float x = sv[i] * A.c_log2;
            if (need_mask) {
                const int key = kbase + KPI * i + g;
                if (key >= T.kv_len || (A.causal && key > my_pos)) x = -INFINITY;
            }
            sv[i] = x;
            bmax = fmaxf(bmax, x);
        }
#pragma unroll
        for (int dl = LPR; dl < 64; dl *= 2) bmax = fmaxf(bmax, __shfl_xor(bmax, dl));
        const float m_new = fmaxf(m, bmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float pv = __builtin_amdgcn_exp2f(sv[i] - m_use);
            lsum += pv;
            p_lds[(KPI * i + g) * RM + my_row] = pv;
        }
        if (g == 0) a_lds[my_row] = alpha;
        // A wave's LDS accesses complete in issue order, so the reads below see the
        // writes above; the previous step's reads were issued before these writes.
        float ar[RM];
#pragma unroll
        for (int r = 0; r < RM; ++r) ar[r] = a_lds[r];
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[r][e] *= ar[r];
        // ---- O += P V (V of keys at or past kv_len and of bad pages zeroed first) ----
        if (bad_cur || kbase + KW > T.kv_len)
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const bool z = (bad_cur & (1 << ((KPI * i) >> 4))) || kbase + KPI * i + g >= T.kv_len;
                const uint32_t keep = z ? 0u : ~0u;
                vr[i] &= u32x4{keep, keep, keep, keep};
            }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float* pk = p_lds + (KPI * i + g) * RM;
            float pr[RM];
#pragma unroll
            for (int r = 0; r < RM; ++r) pr[r] = pk[r];
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = elem16<BF16>(vr[i][e], 0);
                v[2 * e + 1] = elem16<BF16>(vr[i][e], 1);
            }
#pragma unroll
            for (int r = 0; r < RM; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[r][e] = __builtin_fmaf(pr[r], v[e], oacc[r][e]);
        }
    }
    if (bad_seen && lane == 0) raise_flag(A.err_flag, kErrPage);

    // ---- sum the key groups, then combine the 4 waves ----
#pragma unroll
    for (int dl = LPR; dl < 64; dl *= 2) {
        lsum += __shfl_xor(lsum, dl);
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[r][e] += __shfl_xor(oacc[r][e], dl);
    }
    __syncthreads();  // every wave is done with its P staging area
    constexpr int OS = D + 4;
    float* c_o = reinterpret_cast<float*>(smem);
    float* c_m = c_o + kWaves * 16 * OS;
    float* c_l = c_m + kWaves * 16;
    if (g == 0) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            *(f32x4*)(c_o + (wave * 16 + r) * OS + 8 * j) = f32x4{oacc[r][0], oacc[r][1], oacc[r][2], oacc[r][3]};
            *(f32x4*)(c_o + (wave * 16 + r) * OS + 8 * j + 4) = f32x4{oacc[r][4], oacc[r][5], oacc[r][6], oacc[r][7]};
        }
        c_m[wave * 16 + my_row] = m;
        c_l[wave * 16 + my_row] = lsum;
    }
    __syncthreads();
    narrow_combine_store<D, BF16>(A, T, c_o, c_m, c_l, rows_valid);
}

template <int D>
struct ValuLds {
    static constexpr int stage_bytes = kWaves * (kValuKeys * kValuRows + kValuRows) * 4;
    static constexpr int combine_bytes = kWaves * 16 * (D + 4) * 4 + 2 * kWaves * 16 * 4;
    static constexpr int bytes = stage_bytes > combine_bytes ? stage_bytes : combine_bytes;
};

// Narrow tiles on the VALU: at most RM rows each.
template <int D, bool BF16, int RM>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_narrow_valu_kernel(AttnArgs A) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Tile T = A.tiles[blockIdx.x];
    if (T.q_count <= 0) return;
    valu_tile<D, BF16, RM>(A, T, smem);
}

// Wide tiles: three workgroups per CU (three waves per SIMD; see kWideSlots).
template <int D, bool BF16>
__global__ __launch_bounds__(kWideWaves * 64) __attribute__((amdgpu_waves_per_eu(kWideWavesPerEU)))
void attn_wide_kernel(AttnArgs A) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Tile T = A.tiles[blockIdx.x];
    if (T.q_count <= 0) return;
    wide_tile<D, BF16>(A, T, smem);
}

// Narrow tiles: three workgroups per CU (32-key wave steps keep the kernel within
// the 168 registers and 53 KiB of LDS that allows), so more tiles' loads are in
// flight per CU.
// GRP: the plan has kGroup tiles (a separate instantiation, so that plans without them
// keep the register allocation of the plain narrow path).
template <int D, bool BF16, bool KROWS, bool NT, bool GRP>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void attn_narrow_kernel(AttnArgs A) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Tile T = A.tiles[blockIdx.x];
    if (T.q_count <= 0) return;
    if (GRP && T.kind == kGroup)
        narrow_tile<D, BF16, KROWS, NT, true>(A, T, smem);
    else
        narrow_tile<D, BF16, KROWS, NT, false>(A, T, smem);
}

// Both kinds in one launch (mixed batches): each workgroup takes its tile's path.  Both
// paths use 4 waves and fit three workgroups per CU; the LDS is the larger of the two.
template <int D, bool BF16, bool KROWS, bool NT, bool GRP>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void attn_mixed_kernel(AttnArgs A) {
    static_assert(kWaves == kWideWaves, "one workgroup size for both paths");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Tile T = A.tiles[blockIdx.x];
    if (T.q_count <= 0) return;
    if (T.kind == kWide)
        wide_tile<D, BF16>(A, T, smem);
    else if (GRP && T.kind == kGroup)
        narrow_tile<D, BF16, KROWS, NT, true>(A, T, smem);
    else
        narrow_tile<D, BF16, KROWS, NT, false>(A, T, smem);
}

// ---- host-side launchers -----------------------------------------------------------------

// Merge of two attention states over disjoint key sets A and B of the same query
// rows: with weights w = exp(LSE - max(LSE_a, LSE_b)),
//   O = (w_a O_a + w_b O_b) / (w_a + w_b),  LSE = max + ln(w_a + w_b).
// It is the split-KV merge applied to whole outputs (kv-parallelism, flashinfer
// issue #323) and joins the two halves of a cascade: a prefix shared by many
// requests attended once for all of them, plus each request's private suffix
// (vLLM issue #227, "Question about efficient memory sharing").  A state with
// LSE = -inf (no visible key) has weight 0 and its O is not read into the sum
// (it may hold anything); if both have none, O = 0 and LSE = -inf.  One thread per 8 elements of a (row, head); the head_dim / 8
// threads of a (row, head) are adjacent lanes of one wave, so every one of them
// has read LSE_a and LSE_b before the wave's LSE store: O and LSE may be merged
// in place.

template <bool BF16>
__global__ __launch_bounds__(256) void merge_states_kernel(MergeArgs M) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= M.items) return;
    const int C = M.head_dim / 8;
    const int64_t rh = i / C;
    const int c = int(i - rh * C);
    const float la = M.lse_a[rh], lb = M.lse_b[rh];
    const float mx = fmaxf(la, lb);
    const float mu = mx == -INFINITY ? 0.f : mx;
    const float wa = __expf(la - mu), wb = __expf(lb - mu);
    const float sum = wa + wb;
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    const int64_t off = rh * M.head_dim + 8 * c;
    const u32x4 a = *(const u32x4*)(M.o_a + off);
    const u32x4 b = *(const u32x4*)(M.o_b + off);
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = pack_out<BF16>(((wa > 0.f ? wa * elem16<BF16>(a[e], 0) : 0.f) +
                               (wb > 0.f ? wb * elem16<BF16>(b[e], 0) : 0.f)) * inv,
                              ((wa > 0.f ? wa * elem16<BF16>(a[e], 1) : 0.f) +
                               (wb > 0.f ? wb * elem16<BF16>(b[e], 1) : 0.f)) * inv);
    *(u32x4*)(M.o + off) = r;
    if (M.lse && c == 0) M.lse[rh] = sum > 0.f ? mu + __logf(sum) : -INFINITY;
}

// Append: write new tokens' K and V into the cache slots the page table gives them
// (the page-table addressing of flashinfer issue #323's repro: token t of a
// sequence is in page kv_page_indices[kv_page_indptr[b] + t / 16], slot t % 16).
// The new tokens of sequence b are its last append_indptr[b+1] - append_indptr[b]
// tokens under the given (already grown) lengths, the same convention as queries
// and qo_indptr.  One workgroup per new token; its sequence is found by binary
// search over append_indptr.  A token whose position or page is out of range is
// not written and raises err_flag.
__global__ __launch_bounds__(256) void append_kv_kernel(AppendArgs A) {
    const int64_t tok = blockIdx.x;
    if (tok >= A.n_new) return;
    int lo = 0, hi = A.batch - 1;  // last b with append_indptr[b] <= tok
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (A.append_indptr[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int64_t a0 = A.append_indptr[b], a1 = A.append_indptr[b + 1];
    const int np = A.kv_page_indptr[b + 1] - A.kv_page_indptr[b];
    const int last = A.kv_last_page_len[b];
    const bool len_ok = np > 0 && last >= 1 && last <= kPageSize && tok >= a0 && tok < a1;
    const int64_t kv_len = int64_t(np - 1) * kPageSize + last;
    const int64_t pos = kv_len - (a1 - a0) + (tok - a0);
    int page = -1;
    if (len_ok && pos >= 0 && pos < kv_len) page = A.kv_page_indices[A.kv_page_indptr[b] + pos / kPageSize];
    if ((unsigned)page >= (unsigned)A.num_pages) {
        if (threadIdx.x == 0 && A.err_flag) *A.err_flag = 1;
        return;
    }
    const int slot = int(pos % kPageSize);
    const int64_t row = int64_t(A.Hkv) * A.D;  // elements of one K (or V) row
    const int chunks = int(row / 8);           // 16-byte chunks per row
    const uint16_t* src = A.new_kv + tok * 2 * row;
    for (int c = threadIdx.x; c < 2 * chunks; c += 256) {
        const int kvsel = c / chunks, cc = c - kvsel * chunks;
        uint16_t* dst = A.kv + ((int64_t(page) * 2 + kvsel) * kPageSize + slot) * row + 8 * cc;
        *(u32x4*)dst = *(const u32x4*)(src + kvsel * row + 8 * cc);
    }
}

// Launch one workgroup of `threads` per tile with `lds` bytes of dynamic LDS.  Dynamic
// LDS above 64 KiB must be allowed per kernel: done once per kernel (the template
// argument), before its first launch.
template <void (*Kernel)(AttnArgs)>
hipError_t launch_with_lds(const LaunchAttn& L, int lds, int threads, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipExtLaunchKernelGGL(Kernel, dim3((unsigned)L.n_tiles), dim3(threads), (uint32_t)lds, stream, ev0, ev1, 0,
                          L.a);
    return hipGetLastError();
}

hipError_t launch_wide(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (L.n_tiles <= 0) return hipSuccess;
    if (L.head_dim == 128)
        return L.bf16 ? launch_with_lds<&attn_wide_kernel<128, true>>(L, WideCfg<128>::bytes, kWideWaves * 64, stream, ev0, ev1)
                      : launch_with_lds<&attn_wide_kernel<128, false>>(L, WideCfg<128>::bytes, kWideWaves * 64, stream, ev0, ev1);
    return L.bf16 ? launch_with_lds<&attn_wide_kernel<64, true>>(L, WideCfg<64>::bytes, kWideWaves * 64, stream, ev0, ev1)
                  : launch_with_lds<&attn_wide_kernel<64, false>>(L, WideCfg<64>::bytes, kWideWaves * 64, stream, ev0, ev1);
}

template <int D, bool BF16, bool NT, bool GRP>
hipError_t launch_narrow_g(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    return L.k_rows ? launch_with_lds<&attn_narrow_kernel<D, BF16, true, NT, GRP>>(L, NarrowLds<D>::bytes, kWaves * 64, stream, ev0, ev1)
                    : launch_with_lds<&attn_narrow_kernel<D, BF16, false, NT, GRP>>(L, NarrowLds<D>::bytes, kWaves * 64, stream, ev0, ev1);
}

template <int D, bool BF16, bool NT>
hipError_t launch_narrow_nt(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    return L.group ? launch_narrow_g<D, BF16, NT, true>(L, stream, ev0, ev1)
                   : launch_narrow_g<D, BF16, NT, false>(L, stream, ev0, ev1);
}

template <int D, bool BF16>
hipError_t launch_narrow_d(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    return L.kv_stream ? launch_narrow_nt<D, BF16, true>(L, stream, ev0, ev1)
                       : launch_narrow_nt<D, BF16, false>(L, stream, ev0, ev1);
}

template <int D, bool BF16, bool KROWS, bool NT>
hipError_t launch_mixed_k(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int lds = WideCfg<D>::bytes > NarrowLds<D>::bytes ? WideCfg<D>::bytes : NarrowLds<D>::bytes;
    return L.group ? launch_with_lds<&attn_mixed_kernel<D, BF16, KROWS, NT, true>>(L, lds, kWaves * 64, stream, ev0, ev1)
                   : launch_with_lds<&attn_mixed_kernel<D, BF16, KROWS, NT, false>>(L, lds, kWaves * 64, stream, ev0, ev1);
}

template <int D, bool BF16>
hipError_t launch_mixed_d(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (L.k_rows)
        return L.kv_stream ? launch_mixed_k<D, BF16, true, true>(L, stream, ev0, ev1)
                           : launch_mixed_k<D, BF16, true, false>(L, stream, ev0, ev1);
    return L.kv_stream ? launch_mixed_k<D, BF16, false, true>(L, stream, ev0, ev1)
                       : launch_mixed_k<D, BF16, false, false>(L, stream, ev0, ev1);
}

hipError_t launch_mixed(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (L.n_tiles <= 0) return hipSuccess;
    if (L.head_dim == 128)
        return L.bf16 ? launch_mixed_d<128, true>(L, stream, ev0, ev1) : launch_mixed_d<128, false>(L, stream, ev0, ev1);
    return L.bf16 ? launch_mixed_d<64, true>(L, stream, ev0, ev1) : launch_mixed_d<64, false>(L, stream, ev0, ev1);
}

hipError_t launch_narrow(const LaunchAttn& L, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (L.n_tiles <= 0) return hipSuccess;
    if (L.head_dim == 128)
        return L.bf16 ? launch_narrow_d<128, true>(L, stream, ev0, ev1) : launch_narrow_d<128, false>(L, stream, ev0, ev1);
    return L.bf16 ? launch_narrow_d<64, true>(L, stream, ev0, ev1) : launch_narrow_d<64, false>(L, stream, ev0, ev1);
}

template <int D, bool BF16>
hipError_t launch_valu_d(const LaunchAttn& L, int rows, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (rows <= 2)
        return launch_with_lds<&attn_narrow_valu_kernel<D, BF16, 2>>(L, ValuLds<D>::bytes, kWaves * 64, stream, ev0, ev1);
    if (rows <= 4)
        return launch_with_lds<&attn_narrow_valu_kernel<D, BF16, 4>>(L, ValuLds<D>::bytes, kWaves * 64, stream, ev0, ev1);
    return launch_with_lds<&attn_narrow_valu_kernel<D, BF16, 8>>(L, ValuLds<D>::bytes, kWaves * 64, stream, ev0, ev1);
}

hipError_t launch_narrow_valu(const LaunchAttn& L, int max_rows, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (L.n_tiles <= 0) return hipSuccess;
    if (max_rows > kValuRows) return hipErrorInvalidValue;
    if (L.head_dim == 128)
        return L.bf16 ? launch_valu_d<128, true>(L, max_rows, stream, ev0, ev1)
                      : launch_valu_d<128, false>(L, max_rows, stream, ev0, ev1);
    return L.bf16 ? launch_valu_d<64, true>(L, max_rows, stream, ev0, ev1)
                  : launch_valu_d<64, false>(L, max_rows, stream, ev0, ev1);
}

hipError_t launch_append(const AppendArgs& A, hipStream_t stream) {
    if (A.n_new <= 0) return hipSuccess;
    hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)A.n_new), dim3(256), 0, stream, A);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void clear_i32_kernel(int32_t* p, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

hipError_t launch_clear(int32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(clear_i32_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

// The scratch of rpa_run_noalloc (tile records, split counters, error word, partials),
// for callers that cannot allocate device memory.  Each GPU the library runs on holds
// its own copy at its own address; calls that overlap on one GPU share it and race.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {  // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_merge(const MergeArgs& M, bool bf16, hipStream_t stream) {
    if (M.items <= 0) return hipSuccess;
    const int64_t blocks = (M.items + 255) / 256;
    if (bf16)
        hipLaunchKernelGGL(merge_states_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, M);
    else
        hipLaunchKernelGGL(merge_states_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, M);
    return hipGetLastError();
}

}  // namespace rpa
