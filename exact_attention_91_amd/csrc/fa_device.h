// fa_device.h -- device-side building blocks shared by the attention forward
// (fa_fwd.hip) and backward (fa_bwd.hip) kernels for gfx950: vector types,
// the 16-bit MFMA and transposing LDS read, cross-half lane reductions, and the
// LDS tile layout of 64-row tiles of 16-bit elements.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves of 64
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Cross-half (lane <-> lane^32) reductions of a per-lane value.
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// First index in [t, lim) whose 64-bit word of a global-token bitmap is
// nonzero (lim if none): each lane tests one word, 64 words a step, and a
// ballot picks the first. Call from wave-uniform control flow, with every
// word below lim in bounds.
__device__ __forceinline__ int first_nonzero_word(const unsigned long long *bits, int t,
                                                  int lim) {
    const int lane = threadIdx.x & 63;
    for (; t < lim; t += 64) {
        const int w = t + lane;
        const unsigned long long m = __ballot(w < lim && bits[w] != 0ull);
        if (m != 0ull) return t + __builtin_ctzll(m);
    }
    return lim;
}

// ---------------------------------------------------------------------------
// LDS tile of 64 (or ROWS) rows x D 16-bit elements, rows of 2D bytes, unpadded. The
// 16-byte chunks of each row are XOR-permuted so that the MFMA operand reads
// are bank-conflict free (64 banks of 4 bytes; a 16-byte read serves 16 lanes
// per cycle, an 8-byte read 32):
//   row reads (lane = row, 16 bytes of one chunk):  chunk c -> c ^ kswz(row)
//     kswz = (row / R) % C,   C = D/8 chunks per row, R = 16/C rows per 256 B
//   transposed reads (ds_read_b64_tr_b16 of 4-row x 16-column blocks):
//     chunk c -> c ^ vswz(row)   (D=64: 4*((row>>1)&1); D=128: 4*(row&3))
//   both patterns on one tile: chunk c -> c ^ dswz(row), a permutation of
//     the rows' chunk offsets that is conflict-free for both
// Tiles are written by buffer_load_dwordx4 ... lds straight from global
// memory: each 64-lane load fills 1 KB of LDS in lane order, so every lane
// fetches the global chunk that belongs at its LDS slot. Rows past the end of
// the tensor are outside the buffer's range and arrive as zeros.
// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element 16e+i
// (e = 0..3) of the 64 halfwords the group reads, so a group reading a
// 4-row x 16-column block row by row hands lane i the 4 rows of column i.
// ---------------------------------------------------------------------------
template <int D, int ROWS = 64>
struct Bf16Layout {
    static constexpr int BK = ROWS;               // rows (keys) per tile
    static constexpr int C = D / 8;               // 16-byte chunks per row
    static constexpr int R = 16 / C;              // rows per 256 bytes
    static constexpr int ROWB = 2 * D;            // bytes per row
    static constexpr int TILEB = BK * ROWB;       // bytes per K (or V) tile
    static constexpr int NLOAD = TILEB / 1024;    // 1 KB wave loads per tile
    static constexpr int ROWS_PER_LOAD = 1024 / ROWB;
    __device__ static int kswz(int row) { return (row / R) % C; }
    __device__ static int vswz(int row) {
        return D == 64 ? 4 * ((row >> 1) & 1) : (D == 128 ? 4 * (row & 3) : 0);
    }
    // Serves both read patterns at once (tiles read as rows and transposed).
    __device__ static int dswz(int row) {
        if (D == 16) return (row >> 3) & 1;
        if (D == 32) return (row >> 2) & 3;
        if (D == 64) {
            const int e = (row >> 1) & 7;
            return ((e & 1) << 2) | (e >> 1);
        }
        return ((row & 3) << 2) | ((row >> 2) & 3);
    }
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __fp16 fp16x4_t __attribute__((ext_vector_type(4)));   // the builtin's type
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4_t;

// The 16-bit kernel for bfloat16 and for IEEE half: operand vectors, the
// 32x32x16 MFMA with fp32 accumulation, and the transposing LDS read.
template <typename E>
struct Half16;
template <>
struct Half16<__bf16> {
    typedef bf16x8_t v8;
    typedef bf16x4_t v4;
    __device__ static f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static v4 read_tr(const unsigned char *p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)p);
    }
};
template <>
struct Half16<_Float16> {
    typedef f16x8_t v8;
    typedef f16x4_t v4;
    __device__ static f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static v4 read_tr(const unsigned char *p) {
        return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t *)p));
    }
};
constexpr unsigned kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit dwords (gfx9 family)
constexpr int kCachePolicyNT = 2;              // buffer instruction cache policy: nt (gfx950)


// Issue this wave's share (of NW waves) of the global->LDS copies of two
// ROWS-row tiles (64 unless stated), e.g. a K tile and a V tile (buffer loads straight into LDS;
// rows past T read as zeros): loads wave, wave + NW, ... koff/voff: per-lane
// byte offsets of the global chunk each lane fetches for its LDS slot. AUX:
// the loads' cache policy (0, or kCachePolicyNT for tiles read only once).
template <int D, int NW = 4, int ROWS = 64, int AUX = 0>
__device__ __forceinline__ void stage_tile(const unsigned short *kbase, const unsigned short *vbase,
                                           long long ks1, long long vs1, int T, int key0,
                                           int wave, const int *koff, const int *voff,
                                           unsigned char *kdst, unsigned char *vdst) {
    using L = Bf16Layout<D, ROWS>;
    constexpr int NI = (L::NLOAD + NW - 1) / NW;
    // Valid bytes from this tile's first row; (63 * stride + D) * 2 < 2^31 is
    // checked on the host.
    const int rows = min(T - key0, L::BK);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short *>(kbase + (long long)key0 * ks1), (short)0,
        ((rows - 1) * (int)ks1 + D) * 2, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short *>(vbase + (long long)key0 * vs1), (short)0,
        ((rows - 1) * (int)vs1 + D) * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = wave + NW * i;
        if (L::NLOAD % NW == 0 || idx < L::NLOAD) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(kdst + idx * 1024), 16,
                                                     koff[i], 0, 0, AUX);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(vdst + idx * 1024), 16,
                                                     voff[i], 0, 0, AUX);
        }
    }
}

// Issue this wave's share (of NW waves) of the global->LDS copy of `rows`
// (1..64) rows of D 16-bit elements, `stride` elements apart, into one tile in
// the K layout (chunk c of row r at c ^ kswz(r)); rows past `rows` read as zeros.
// The rows are read once, so the loads are non-temporal (cache policy nt):
// they do not displace the K/V tiles other work-groups re-read from L2.
template <int D, int NW = 4>
__device__ __forceinline__ void stage_rows(const unsigned short *base, long long stride, int rows,
                                           int wave, unsigned char *dst) {
    using L = Bf16Layout<D>;
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short *>(base), (short)0, ((rows - 1) * (int)stride + D) * 2,
        kRsrcWord3);
#pragma unroll
    for (int i = 0; i < (L::NLOAD + NW - 1) / NW; ++i) {
        const int idx = wave + NW * i;
        if (L::NLOAD % NW == 0 || idx < L::NLOAD) {
            const int row = idx * L::ROWS_PER_LOAD + lane / L::C;
            const int off = row * (int)stride * 2 + 16 * ((lane % L::C) ^ L::kswz(row));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + idx * 1024), 16, off,
                                                     0, 0, kCachePolicyNT);
        }
    }
}

// base ^ k for a per-lane base and a constant k, issued where it is used: an
// asm statement the compiler neither hoists out of a loop nor keeps live, so a
// kernel can derive many LDS offsets from one register at the cost of one VALU
// instruction per use.
__device__ __forceinline__ int lane_xor(int base, int k) {
    if (k == 0) return base;
    int r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(k), "v"(base));
    return r;
}

// Debug builds compiled with FA_LDS_POISON (libfa_poison.so): between the
// barrier that ends the last reads of an LDS buffer and its refill, the buffer
// is set to all-ones bits (a NaN in every element type) and a second barrier
// orders that fill before the refill, so a read that races the refill, or an
// access the tile's barriers do not cover, returns NaN instead of stale data.
// Every wave of the work-group calls it the same number of times (it holds a
// barrier); `fill` says whether the caller's buffer is refilled at this step;
// threads t, t + nt, ... of the caller's group share the writes. Release
// builds compile it to nothing.
__device__ __forceinline__ void lds_poison(bool fill, void *buf, int bytes, int t, int nt) {
#ifdef FA_LDS_POISON
    if (fill) {
        const u32x4_t ones = {~0u, ~0u, ~0u, ~0u};
        for (int i = t; i < bytes / 16; i += nt)
            *(lds_u32x4_t *)((__attribute__((address_space(3))) unsigned char *)buf + 16 * i) = ones;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#else
    (void)fill; (void)buf; (void)bytes; (void)t; (void)nt;
#endif
}
__device__ __forceinline__ void lds_poison2(bool fill, void *a, void *b, int bytes, int t, int nt) {
#ifdef FA_LDS_POISON
    if (fill) {
        const u32x4_t ones = {~0u, ~0u, ~0u, ~0u};
        for (int i = t; i < bytes / 16; i += nt) {
            *(lds_u32x4_t *)((__attribute__((address_space(3))) unsigned char *)a + 16 * i) = ones;
            *(lds_u32x4_t *)((__attribute__((address_space(3))) unsigned char *)b + 16 * i) = ones;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#else
    (void)fill; (void)a; (void)b; (void)bytes; (void)t; (void)nt;
#endif
}

// Host: a * b for non-negative sizes, saturating at LLONG_MAX instead of
// overflowing (size heuristics compare the result with small thresholds).
inline long long mul_sat(long long a, long long b) {
    long long r;
    return __builtin_mul_overflow(a, b, &r) ? __LONG_LONG_MAX__ : r;
}

// Host: launch `kern` on stream `s` and return the status of this launch alone.
// The thread's last-error state is neither read nor cleared, so an error left
// by an unrelated earlier HIP call is not reported as this launch's failure.
template <typename T>
struct Same {
    typedef T type;
};
template <typename... P>
hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t s,
                         typename Same<P>::type... args) {
    void *argv[] = {(void *)&args...};
    return hipLaunchKernel((const void *)kern, grid, block, argv, 0, s);
}

}  // namespace
