// fa_roofs.hip -- microbenchmarks measuring the roofs of this GPU that the
// attention kernels are judged against (C ABI in include/fa_roofs.h): dense
// bf16 MFMA rate, v_exp_f32 and fp32 FMA rates, MFMA/VALU overlap on one SIMD,
// and device-memory copy bandwidth. Each kernel's work is fixed by its
// arguments; the caller times the launches.
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_roofs.h"

namespace {

// Results are positive by construction; a store guarded by an impossible
// value keeps the arithmetic live without any memory traffic.
constexpr float kNever = -1234.5f;

__device__ __forceinline__ void keep(float x, float *sink) {
    if (x == kNever) sink[blockIdx.x] = x;
}

// Four independent accumulator chains of 32x32x16 bf16 MFMAs per wave.
__device__ __forceinline__ float mfma_loop(int n_iter) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (1 + ((lane + e) & 7)));
        b[e] = (__bf16)(0.002f * (1 + ((lane * 3 + e) & 7)));
    }
    f32x16_t c0{}, c1{}, c2{}, c3{};
    for (int i = 0; i < n_iter; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    return c0[0] + c1[1] + c2[2] + c3[3];
}

// Sixteen independent chains of one VALU instruction kind per wave:
// x <- exp2(-x) (stays in (0, 1)) or x <- x * a + b (stays positive).
template <int OP>
__device__ __forceinline__ float valu_loop(int n_iter) {
    const int lane = threadIdx.x & 63;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.25f + 0.01f * ((lane + r) & 15);
    const float a = 0.5f + 1e-3f * (lane & 7), b = 0.125f + 1e-3f * (lane >> 3);
    for (int i = 0; i < n_iter; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[r] = OP == FA_ROOF_EXP ? __builtin_amdgcn_exp2f(-x[r]) : fmaf(x[r], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += x[r];
    return s;
}

__global__ __launch_bounds__(256) void roof_mfma_kernel(int n_iter, float *sink) {
    keep(mfma_loop(n_iter), sink);
}

template <int OP>
__global__ __launch_bounds__(256) void roof_valu_kernel(int n_iter, float *sink) {
    keep(valu_loop<OP>(n_iter), sink);
}

// Waves w and w + 4 of an 8-wave work-group share a SIMD: waves 0-3 issue
// MFMAs, waves 4-7 VALU instructions of kind OP.
template <int OP>
__global__ __launch_bounds__(512) void roof_overlap_kernel(int n_mfma, int n_valu, int mask,
                                                           float *sink) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < 4) {
        if (mask & 1) keep(mfma_loop(n_mfma), sink);
    } else {
        if (mask & 2) keep(valu_loop<OP>(n_valu), sink);
    }
}

// Work-group g of G streams its own contiguous share [n16 g / G, n16 (g+1) / G)
// of the buffer, 256 threads reading consecutive 16-byte vectors. On this
// chip per-work-group streams reach a higher rate than one grid-wide stride
// over the whole buffer (reads about 7.0 against 5.4 TB/s).
__device__ __forceinline__ void my_chunk(long long n16, long long &lo, long long &hi) {
    lo = n16 * blockIdx.x / gridDim.x;
    hi = n16 * (blockIdx.x + 1) / gridDim.x;
}

// Four 16-byte vectors in flight per thread: all loads of a step are issued
// before its stores. n16: 16-byte vectors in the buffer.
__global__ __launch_bounds__(256) void roof_copy_kernel(const u32x4_t *src, u32x4_t *dst,
                                                        long long n16) {
    long long lo, hi;
    my_chunk(n16, lo, hi);
    long long i = lo + threadIdx.x;
    for (; i + 3 * 256 < hi; i += 4 * 256) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + 256);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * 256);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * 256);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + 256);
        __builtin_nontemporal_store(c, dst + i + 2 * 256);
        __builtin_nontemporal_store(d, dst + i + 3 * 256);
    }
    for (; i < hi; i += 256) dst[i] = src[i];
}

// Reads n16 16-byte vectors, eight in flight per thread, and folds them into
// one word per thread (stored only if it matches an impossible pattern).
__global__ __launch_bounds__(256) void roof_read_kernel(const u32x4_t *src, long long n16,
                                                        float *sink) {
    long long lo, hi;
    my_chunk(n16, lo, hi);
    u32x4_t acc = {0u, 0u, 0u, 0u};
    long long i = lo + threadIdx.x;
    for (; i + 7 * 256 < hi; i += 8 * 256) {
        u32x4_t x[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) x[r] = __builtin_nontemporal_load(src + i + r * 256);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc ^= x[r];
    }
    for (; i < hi; i += 256) acc ^= src[i];
    const unsigned w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (w == 0x9e3779b9u && threadIdx.x == 0) sink[blockIdx.x] = 1.f;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : 9; }

constexpr unsigned kStreamBlocks = 256 * 32;   // work-groups of the copy and read roofs

}  // namespace

extern "C" int fa_roof_mfma(int grid_blocks, int n_iter, float *sink, void *stream) {
    if (grid_blocks < 1 || n_iter < 1) return 2;
    if (!sink) return 1;
    return status(launch_kernel(roof_mfma_kernel, dim3(grid_blocks), dim3(256),
                                (hipStream_t)stream, n_iter, sink));
}

extern "C" int fa_roof_valu(int grid_blocks, int n_iter, int op, float *sink, void *stream) {
    if (grid_blocks < 1 || n_iter < 1 || (op != FA_ROOF_FMA && op != FA_ROOF_EXP)) return 2;
    if (!sink) return 1;
    const hipStream_t s = (hipStream_t)stream;
    return status(op == FA_ROOF_EXP
                      ? launch_kernel(roof_valu_kernel<FA_ROOF_EXP>, dim3(grid_blocks),
                                      dim3(256), s, n_iter, sink)
                      : launch_kernel(roof_valu_kernel<FA_ROOF_FMA>, dim3(grid_blocks),
                                      dim3(256), s, n_iter, sink));
}

extern "C" int fa_roof_overlap(int grid_blocks, int n_mfma, int n_valu, int op, int mask,
                               float *sink, void *stream) {
    if (grid_blocks < 1 || n_mfma < 1 || n_valu < 1 || mask < 1 || mask > 3 ||
        (op != FA_ROOF_FMA && op != FA_ROOF_EXP))
        return 2;
    if (!sink) return 1;
    const hipStream_t s = (hipStream_t)stream;
    return status(op == FA_ROOF_EXP
                      ? launch_kernel(roof_overlap_kernel<FA_ROOF_EXP>, dim3(grid_blocks),
                                      dim3(512), s, n_mfma, n_valu, mask, sink)
                      : launch_kernel(roof_overlap_kernel<FA_ROOF_FMA>, dim3(grid_blocks),
                                      dim3(512), s, n_mfma, n_valu, mask, sink));
}

extern "C" int fa_roof_read(const void *src, long long bytes, float *sink, void *stream) {
    if (bytes < 16) return 2;
    if (!src || !sink) return 1;
    if (bytes % 16 != 0 || (uintptr_t)src % 16 != 0) return 7;
    // 32 work-groups of 256 threads per compute unit, each streaming its own chunk
    return status(launch_kernel(roof_read_kernel, dim3(kStreamBlocks), dim3(256),
                                (hipStream_t)stream, (const u32x4_t *)src, bytes / 16, sink));
}

extern "C" int fa_roof_copy(const void *src, void *dst, long long bytes, void *stream) {
    if (bytes < 16) return 2;
    if (!src || !dst) return 1;
    if (bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0) return 7;
    // 32 work-groups of 256 threads per compute unit, each copying its own chunk
    return status(launch_kernel(roof_copy_kernel, dim3(kStreamBlocks), dim3(256),
                                (hipStream_t)stream, (const u32x4_t *)src, (u32x4_t *)dst,
                                bytes / 16));
}
