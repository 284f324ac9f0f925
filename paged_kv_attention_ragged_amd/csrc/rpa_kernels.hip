// rpa_kernels.hip -- gfx950 (CDNA4) kernels for ragged attention over a paged
// KV cache: the attention tile kernel and the split-KV merge kernel.
//
// Attention tile kernel, one 256-thread workgroup (4 wave64) per Tile:
//   * rows of the tile are (token, qo head) pairs of one kv head's query group,
//     token-major; wave w owns rows 32w .. 32w+31, so the G heads sharing a kv
//     head are stacked into the MFMA dimension and read each K/V block once
//     (grouped-query attention, flashinfer issue #323);
//   * keys are walked in blocks of BN = 8192/D: each thread gathers 4 keys x 16
//     bytes of K and of V through the page table (one page per wave for D=128),
//     K goes to LDS as is, V is transposed (and, for bf16 inputs, converted to
//     fp16) on its way to LDS; the next block's gather is in flight while the
//     current block is computed;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: each lane then holds one
//     query row and 16 of its scores, so the running max needs one cross-half
//     exchange and the running sum none until the end;
//   * mask only on boundary blocks (past kv_len, or crossing the causal diagonal
//     of the wave's rows); blocks past every row's position are never loaded
//     (llama.cpp discussion #15958: fully masked tails are skipped);
//   * online softmax in the exp2 domain, O^T += V^T P^T on
//     v_mfma_f32_32x32x16_f16 with P rounded to fp16 (10 fraction bits);
//   * epilogue: O / l rounded to nearest-even into the input dtype and
//     LSE = ln(l) + max, or fp32 partial rows when the key range is split.
// Merge kernel: one workgroup per split query tile combines the pieces'
// (O_s, LSE_s) by weights exp(LSE_s - max LSE) (flashinfer issue #323 speaks of
// kv-parallelism / split-k in the prefill kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

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
__device__ __forceinline__ uint32_t pack_p(float a, float b) { return pack_out<false>(a, b); }

// 16-bit element e (0..7) of a 16-byte vector, widened to an fp32 bit pattern
// for bf16 (exact) -- used only for the bf16 -> fp16 conversion of V.
__device__ __forceinline__ float bf16_elem(u32x4 v, int e) {
    const uint32_t w = v[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Element e of keys i and j as one packed fp16 pair (low = key i).
template <bool BF16>
__device__ __forceinline__ uint32_t v_pair(u32x4 vi, u32x4 vj, int e) {
    if (BF16) {
        // bf16 -> fp16: exact for |x| in [2^-14, 65504]; round-toward-zero below
        // (error < 2^-24) and saturation to 65504 above.
        fp16x2 h = __builtin_amdgcn_cvt_pkrtz(bf16_elem(vi, e), bf16_elem(vj, e));
        return __builtin_bit_cast(uint32_t, h);
    }
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    return __builtin_amdgcn_perm(vj[e >> 1], vi[e >> 1], sel);
}

// XOR swizzle of the 16-byte groups of a transposed-V row, so that both the
// 8-byte transposing writes and the 16-byte MFMA operand reads spread over banks.
__device__ __forceinline__ int vt_swz(int d) { return (d + (d >> 3)) & 7; }


template <int D, bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_tile_kernel(AttnArgs A) {
    constexpr int BN = 8192 / D;  // keys per block
    constexpr int CH = D / 8;     // 16-byte chunks per K/V row
    constexpr int KS = D + 8;     // K row stride in LDS (elements), 16-byte pad
    constexpr int SB = BN / 32;   // 32-key score blocks
    constexpr int DK = D / 16;    // k-steps of Q K^T
    constexpr int DB = D / 32;    // 32-wide d blocks of O
    constexpr int KC = BN / 16;   // 16-key steps of P V
    static_assert(CH * (BN / 4) == 256, "each thread gathers 4 keys x 16 bytes");
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * BN];

    const Tile T = A.tiles[blockIdx.x];
    if (T.q_count <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int G = A.G;
    const int rows_valid = T.q_count * G;
    const int row = wave * 32 + col;
    const int tok = row / G, g = row - tok * G;
    const bool row_ok = row < rows_valid;
    const int pos = T.pos0 + tok;
    const int64_t orow = (int64_t)(T.q_row0 + tok) * A.H + T.kv_head * G + g;

    // Q^T operand: 8 consecutive d per k-step, kept in VGPRs for the whole tile.
    u32x4 qf[DK];
    {
        const uint16_t* qp = A.q + orow * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            qf[kk] = row_ok ? *(const u32x4*)(qp + 16 * kk) : u32x4{0, 0, 0, 0};
    }
    const int wrow0 = wave * 32;
    const int wrows = min(32, rows_valid - wrow0);
    const bool wave_active = wrows > 0;
    const int wpos_min = T.pos0 + wrow0 / G;
    const int wpos_max = T.pos0 + (wrow0 + max(wrows, 1) - 1) / G;

    // Gather mapping: thread -> keys 4kg..4kg+3 of the block, d = 8ch..8ch+7.
    const int ch = tid % CH, kg = tid / CH;
    const int64_t slot_stride = (int64_t)A.Hkv * D;
    const uint16_t* kv_base = A.kv + (int64_t)T.kv_head * D + 8 * ch;
    u32x4 kreg[4], vreg[4];

    auto gather = [&](int kv0) {
        const int key0 = kv0 + 4 * kg;  // 4-aligned: the 4 keys share a page
        int page = -1;
        if (key0 < T.kv_len) {
            page = A.page_idx[T.page_base + (key0 >> 4)];
            if ((unsigned)page >= (unsigned)A.num_pages) {
                *A.err_flag = 1;
                page = -1;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (page >= 0 && key0 + i < T.kv_len) {
                const uint16_t* src = kv_base + ((int64_t)page * 32 + ((key0 + i) & 15)) * slot_stride;
                kreg[i] = *(const u32x4*)src;
                vreg[i] = *(const u32x4*)(src + 16 * slot_stride);
            } else {
                kreg[i] = u32x4{0, 0, 0, 0};
                vreg[i] = u32x4{0, 0, 0, 0};
            }
        }
    };

    // Key slot order inside each 16-key chunk of V^T: bits 2 and 3 of the key
    // swapped, so the 8 keys one lane feeds to a P V step are contiguous.
    const int kb = 4 * kg;
    const int vslot = (kb & ~15) | (((kb >> 2) & 1) << 3) | (((kb >> 3) & 1) << 2);
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)(k_lds + (kb + i) * KS + 8 * ch) = kreg[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * ch + e;
            u32x2 w;
            w[0] = v_pair<BF16>(vreg[0], vreg[1], e);
            w[1] = v_pair<BF16>(vreg[2], vreg[3], e);
            *(u32x2*)(vt_lds + d * BN + 8 * ((vslot >> 3) ^ vt_swz(d)) + (vslot & 7)) = w;
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m = -INFINITY;  // running max of the scaled scores (log2 units)
    float lsum = 0.f;     // this lane's share of the running sum

    const int nblk = (T.kv_end - T.kv_begin + BN - 1) / BN;
    gather(T.kv_begin);
    for (int blk = 0; blk < nblk; ++blk) {
        const int kv0 = T.kv_begin + blk * BN;
        __syncthreads();
        stage();
        if (blk + 1 < nblk) gather(kv0 + BN);
        __syncthreads();
        if (!wave_active) continue;
        if (A.causal && kv0 > wpos_max) continue;  // every row of this wave is masked

        f32x16 s[SB];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            s[sb] = f32x16{};
            const uint16_t* kp = k_lds + (32 * sb + col) * KS + 8 * half;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) s[sb] = mfma_qk(*(const u32x4*)(kp + 16 * kk), qf[kk], s[sb], BF16);
        }

        const bool need_mask = (kv0 + BN > T.kv_len) || (A.causal && kv0 + BN - 1 > wpos_min);
        float bmax = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[sb][r] * A.c_log2;
                if (need_mask) {
                    const int key = kv0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= T.kv_len || (A.causal && key > pos)) x = -INFINITY;
                }
                s[sb][r] = x;
                bmax = fmaxf(bmax, x);
            }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        const float m_new = fmaxf(m, bmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[sb][r] - m_use);
                lsum += p;
                s[sb][r] = p;
            }
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int sb = kc >> 1, r0 = (kc & 1) * 8;
            u32x4 pf;
            pf[0] = pack_p(s[sb][r0 + 0], s[sb][r0 + 1]);
            pf[1] = pack_p(s[sb][r0 + 2], s[sb][r0 + 3]);
            pf[2] = pack_p(s[sb][r0 + 4], s[sb][r0 + 5]);
            pf[3] = pack_p(s[sb][r0 + 6], s[sb][r0 + 7]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = 32 * db + col;
                const u32x4 vf = *(const u32x4*)(vt_lds + d * BN + 8 * ((2 * kc + half) ^ vt_swz(d)));
                oacc[db] = mfma_pv(vf, pf, oacc[db]);
            }
        }
    }

    if (!wave_active) return;
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!row_ok) return;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const float lse_val = ltot > 0.f ? (m + __log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
    if (T.part < 0) {
        uint16_t* op = A.o + orow * D + 4 * half;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x2 w;
                w[0] = pack_out<BF16>(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
                w[1] = pack_out<BF16>(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
                *(u32x2*)(op + 32 * db + 8 * j) = w;
            }
        if (A.lse && half == 0) A.lse[orow] = lse_val;
    } else {
        float* pp = A.part_o + ((int64_t)T.part + row) * D + 4 * half;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 w = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv, oacc[db][4 * j + 2] * inv,
                           oacc[db][4 * j + 3] * inv};
                *(f32x4*)(pp + 32 * db + 8 * j) = w;
            }
        if (half == 0) A.part_lse[T.part + row] = lse_val;
    }
}


template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs A) {
    constexpr int D4 = D / 4;
    const Merge M = A.merges[blockIdx.x];
    const int R = M.q_count * A.G;
    for (int idx = threadIdx.x; idx < R * D4; idx += 256) {
        const int r = idx / D4, d4 = idx - r * D4;
        float mx = -INFINITY;
        for (int s = 0; s < M.n_splits; ++s) mx = fmaxf(mx, A.part_lse[M.part0 + s * R + r]);
        float wsum = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < M.n_splits; ++s) {
            const int pr = M.part0 + s * R + r;
            const float l = A.part_lse[pr];
            const float w = l == -INFINITY ? 0.f : __expf(l - mx);
            const f32x4 v = *(const f32x4*)(A.part_o + (int64_t)pr * D + 4 * d4);
            acc += w * v;
            wsum += w;
        }
        const float inv = 1.f / wsum;
        const int tok = r / A.G, g = r - tok * A.G;
        const int64_t orow = (int64_t)(M.q_row0 + tok) * A.H + M.kv_head * A.G + g;
        u32x2 w2;
        w2[0] = pack_out<BF16>(acc[0] * inv, acc[1] * inv);
        w2[1] = pack_out<BF16>(acc[2] * inv, acc[3] * inv);
        *(u32x2*)(A.o + orow * D + 4 * d4) = w2;
        if (A.lse && d4 == 0) A.lse[orow] = mx + __logf(wsum);
    }
}

// ---- host-side launchers -----------------------------------------------------------------


hipError_t launch_attention(const LaunchAttn& L, hipStream_t stream) {
    if (L.n_tiles <= 0) return hipSuccess;
    dim3 grid((unsigned)L.n_tiles), block(256);
    if (L.head_dim == 128) {
        if (L.bf16) hipLaunchKernelGGL((attn_tile_kernel<128, true>), grid, block, 0, stream, L.a);
        else hipLaunchKernelGGL((attn_tile_kernel<128, false>), grid, block, 0, stream, L.a);
    } else {
        if (L.bf16) hipLaunchKernelGGL((attn_tile_kernel<64, true>), grid, block, 0, stream, L.a);
        else hipLaunchKernelGGL((attn_tile_kernel<64, false>), grid, block, 0, stream, L.a);
    }
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, bool bf16, int64_t n_merges, hipStream_t stream) {
    if (n_merges <= 0) return hipSuccess;
    dim3 grid((unsigned)n_merges), block(256);
    if (head_dim == 128) {
        if (bf16) hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, stream, a);
    } else {
        if (bf16) hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace rpa
