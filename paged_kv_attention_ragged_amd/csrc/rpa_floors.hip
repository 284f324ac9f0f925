// rpa_floors.hip -- microbenchmarks that measure the floors the attention kernels
// are judged against on this chip: the cost of an empty launch, the HBM read rate
// of a plain stream and of the decode kernel's own paged gather, and the dense
// MFMA rate.  Built into librpa_floors.so, which only the benchmark loads; the
// attention library does not link it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void empty_kernel() {}

// Plain HBM read: workgroup w reads its own contiguous share of the buffer, 4 KiB
// per workgroup-wide load, four loads in flight per lane, non-temporal (the fastest
// of the read shapes measured on MI355X), and folds the data into one word per lane,
// stored once so that the loads are not dropped.  per16: 16-byte chunks per
// workgroup, a multiple of 1024.
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ src, int64_t per16, uint32_t* out) {
    const u32x4* p = src + int64_t(blockIdx.x) * per16 + threadIdx.x;
    uint32_t acc = 0;
    for (int64_t i = 0; i < per16; i += 1024) {
        const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + 256);
        const u32x4 c = __builtin_nontemporal_load(p + i + 512), d = __builtin_nontemporal_load(p + i + 768);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^
               d[2] ^ d[3];
    }
    out[int64_t(blockIdx.x) * 256 + threadIdx.x] = acc;
}

// The decode kernel's memory traffic without its arithmetic: workgroup w reads the K
// and V rows of kv head 0 for `chunks` consecutive runs of 256 keys of sequence seq,
// starting at key 256 chunks piece (w = seq * pieces + piece), through the page table,
// with non-temporal 16-byte loads; cache layout [page][2][16][kv_heads][128] of 16-bit
// values.  A run's 16 page ids are wave-uniform (scalar loads); lane t then reads slot
// t / 16, chunk t % 16 of every page, all 32 loads of a run in flight at once.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
                                                     int32_t pages_per_seq, int32_t pieces, int32_t chunks,
                                                     int32_t kv_heads, uint32_t* out) {
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    const int w = blockIdx.x, seq = w / pieces, piece = w - seq * pieces;
    const int slot = threadIdx.x >> 4, ch = threadIdx.x & 15;
    const int64_t ss = int64_t(kv_heads) * 128;  // elements between token slots
    uint32_t acc = 0;
    for (int c = 0; c < chunks; ++c) {
        const int64_t pbase = int64_t(seq) * pages_per_seq + (int64_t(piece) * chunks + c) * 16;
        int pg[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pg[i] = ((const_i32*)idx)[pbase + i];
        u32x4 v[32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint16_t* b = kv + (int64_t(pg[i]) * 32 + slot) * ss + 8 * ch;
            v[2 * i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b));
            v[2 * i + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + 16 * ss));
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    }
    out[int64_t(w) * 256 + threadIdx.x] = acc;
}

// Dense MFMA rate: each wave keeps four independent 32x32x16 bf16 accumulations in
// flight, iters times, from operands held in registers.
__global__ __launch_bounds__(256) void mfma_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * float(lane + e));
        b[e] = (__bf16)(0.002f * float(lane - e));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    out[int64_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Each returns a hipError_t (0 on success) and enqueues one kernel on `stream`.

// `grid` workgroups of 256 threads that return at once.
int rpa_floor_empty(int32_t grid, void* stream) {
    if (grid < 1) return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream));
    return int(hipGetLastError());
}

// Read `bytes` from src, `grid` workgroups each reading a contiguous share;
// bytes must be a multiple of grid * 16 KiB.  out holds grid * 256 words.
int rpa_floor_stream(const void* src, int64_t bytes, uint32_t* out, int32_t grid, void* stream) {
    if (!src || !out || grid < 1 || bytes <= 0 || bytes % (int64_t(grid) * 16384)) return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16 / grid, out);
    return int(hipGetLastError());
}

// The decode gather: batch * pieces workgroups, each reading chunks x 256 keys (K and
// V, kv head 0, head_dim 128) of its sequence; page table idx [batch][pages_per_seq],
// every index a valid page of kv; 16 * pieces * chunks <= pages_per_seq.  out holds
// batch * pieces * 256 words.
int rpa_floor_gather(const void* kv, const int32_t* idx, int32_t batch, int32_t pages_per_seq, int32_t pieces,
                     int32_t chunks, int32_t kv_heads, uint32_t* out, void* stream) {
    if (!kv || !idx || !out || batch < 1 || pieces < 1 || chunks < 1 || kv_heads < 1 ||
        int64_t(16) * pieces * chunks > pages_per_seq)
        return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(gather_kernel, dim3(batch * pieces), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(kv), idx, pages_per_seq, pieces, chunks, kv_heads, out);
    return int(hipGetLastError());
}

// grid workgroups of 4 waves, each wave 4 * iters v_mfma_f32_32x32x16_bf16
// (32768 flops each); out holds grid * 256 floats.
int rpa_floor_mfma(float* out, int32_t grid, int32_t iters, void* stream) {
    if (!out || grid < 1 || iters < 1) return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    return int(hipGetLastError());
}

}  // extern "C"
