// Small building blocks of the backward and diagnostics kernels: the
// 32x32x16 bf16 MFMA and its operand reads from row-major LDS tiles, and a
// 32-row tile moved global -> registers -> LDS in two steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBwdThreads = 256;  // threads of every workgroup using these
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes of row `row` at column k0 + 8 lh (row-major tile, `stride` elements)
__device__ __forceinline__ bf16x8 rd_row(const uint16_t* t, int stride, int row, int k0, int lh) {
    return *(const bf16x8*)(t + row * stride + k0 + 8 * lh);
}

// Column cb + l32 of rows k0 + 8 lh .. k0 + 8 lh + 7: two transposing reads.
// Within a 16-lane group, lane 4e + r addresses row e at column base + 4r and
// receives column base + (lane % 16) of the 4 rows.
__device__ __forceinline__ bf16x8 rd_col(const uint16_t* t, int stride, int k0, int cb, int lane) {
    const int g = lane >> 4, e = (lane & 15) >> 2, r = lane & 3;
    const uint16_t* p = t + (k0 + 8 * (g >> 1) + e) * stride + cb + 16 * (g & 1) + 4 * r;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(p + 4 * stride));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// registers 8c .. 8c+7 of an accumulator, rounded to bf16 (one B or A operand)
__device__ __forceinline__ void pack(const float (&x)[16], bf16x8 (&o)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[c][j] = (__bf16)x[8 * c + j];
}

// Raw buffer resource over `bytes` bytes from `base` (clamped to [0, 2^31 - 1]);
// loads at offsets past the end return zeros and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const int n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// A tile of 32 rows of a [n][W] bf16 tensor, moved in two steps so that the
// global loads of the next tile are in flight while the current one is used:
// load() into registers (rows at or past n read as zero, by the buffer
// bounds: no select on the loaded value, so nothing waits for the load before
// store()), store() into a padded LDS tile.
template <int W>
struct RowTile {
    static constexpr int kCpr = W / 8;  // 16-byte chunks per row
    static constexpr int kChunks = 32 * kCpr;
    static constexpr int kPer = (kChunks + kBwdThreads - 1) / kBwdThreads;
    uint4 r[kPer];
    __device__ __forceinline__ void load(const uint16_t* g, int64_t row0, int64_t n) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g + row0 * W, (n - row0) * W * 2);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + kBwdThreads * i;
            const int row = c / kCpr, ch = c % kCpr;
            // (chunks past the tile, c >= kChunks, are loaded and not stored)
            r[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (row * W + 8 * ch) * 2, 0, 0));
        }
    }
    __device__ __forceinline__ void store(uint16_t* t) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + kBwdThreads * i;
            if (c < kChunks) *(uint4*)(t + (c / kCpr) * (W + 8) + 8 * (c % kCpr)) = r[i];
        }
    }
};

}  // namespace tile
}  // namespace diffattn
