// Roofline microbenchmarks for gfx950: the rates the operator's kernels are
// measured against, next to the published figures.
//
//   peaks_mfma_bf16   dense bf16 matrix rate: every wave issues independent
//                     v_mfma_f32_32x32x16_bf16 chains (32768 flops each);
//   peaks_read_bw     streaming HBM reads: each block reads one contiguous
//                     chunk of a buffer much larger than the caches with
//                     16-byte non-temporal loads, each byte once (on MI355X
//                     this pattern reads ~7.1 TB/s where a grid-stride walk
//                     over the same buffer, or plain loads, stay near 6.3);
//   peaks_lds_read    LDS read rate: 16 waves per workgroup stream
//                     conflict-free 16-byte reads over 64 KB of LDS (the
//                     attention kernels' operand path);
//   peaks_exp_rate    v_exp_f32 throughput (the softmax's transcendental),
//                     independent chains in every lane; and the same for
//                     v_fma_f32, so the two can be compared.
//
// Each entry point launches on the given stream and returns a hipError_t
// code; the caller times the launch with events and divides the work it
// reports.  The kernels write one value per thread only when an impossible
// condition holds, so the work cannot be optimised away and nothing is
// written in practice.  Built into a library of its own: these are
// measurement tools, not part of the operator's interface.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_bf16_kernel(float* sink, int iters) {
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((t + i) & 7));
        b[i] = (__bf16)(0.002f * (float)((t * 3 + i) & 7));
    }
    f32x16 c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][15];
    if (s == -1.2345f) sink[blockIdx.x * blockDim.x + t] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* sink) {
    // block b reads [b chunk, (b + 1) chunk); the last block also the remainder
    const int64_t chunk = n16 / gridDim.x;
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = blockIdx.x + 1 == gridDim.x ? n16 : beg + chunk;
    const int64_t bs = blockDim.x;
    int64_t i = beg + threadIdx.x;
    uint32_t acc = 0;
    // four loads in flight per lane
    for (; i + 3 * bs < end; i += 4 * bs) {
        const u32x4 x0 = __builtin_nontemporal_load(src + i);
        const u32x4 x1 = __builtin_nontemporal_load(src + i + bs);
        const u32x4 x2 = __builtin_nontemporal_load(src + i + 2 * bs);
        const u32x4 x3 = __builtin_nontemporal_load(src + i + 3 * bs);
        acc ^= (x0[0] ^ x0[1] ^ x0[2] ^ x0[3]) + (x1[0] ^ x1[1] ^ x1[2] ^ x1[3]) +
               (x2[0] ^ x2[1] ^ x2[2] ^ x2[3]) + (x3[0] ^ x3[1] ^ x3[2] ^ x3[3]);
    }
    for (; i < end; i += bs) {
        const u32x4 x = __builtin_nontemporal_load(src + i);
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// every lane: 8 independent 16-byte reads per step; 16 consecutive lanes read
// 256 contiguous bytes (all 64 banks once).  Each address passes through an
// empty asm, so the compiler cannot reuse a load of an earlier step (7 of a
// step's 8 addresses recur in the next), and all four words are used, so
// each read stays 16 bytes wide.
__global__ __launch_bounds__(1024) void lds_read_kernel(uint32_t* sink, int iters) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
    for (int i = threadIdx.x; i < 65536 / 16; i += blockDim.x)
        ((u32x4*)buf)[i] = u32x4{(uint32_t)i, (uint32_t)i + 1, (uint32_t)i + 2, (uint32_t)i + 3};
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            int off = ((wave * 8 + u + it) * 1024 + lane * 16) & 65535;
            asm volatile("" : "+v"(off));
            const u32x4 v = *(const u32x4*)(buf + off);
            acc += (v[0] ^ v[1]) + (v[2] ^ v[3]);
        }
    }
    if (acc == 0x12345u) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

constexpr int kExpChains = 8;

// x <- 2^-x keeps every chain in [0.5, 1]: the negation is a source modifier
// of the one instruction per step
__global__ __launch_bounds__(256) void exp_kernel(float* sink, int iters) {
    float x[kExpChains];
#pragma unroll
    for (int k = 0; k < kExpChains; ++k) x[k] = 0.1f * (float)k + 1e-3f * (float)(threadIdx.x & 63);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kExpChains; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kExpChains; ++k) s += x[k];
    if (s == -1.2345f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// x <- x * c + d with |c| < 1: one v_fma_f32 per step and chain
__global__ __launch_bounds__(256) void fma_kernel(float* sink, int iters, float c, float d) {
    float x[kExpChains];
#pragma unroll
    for (int k = 0; k < kExpChains; ++k) x[k] = 0.1f * (float)k + 1e-3f * (float)(threadIdx.x & 63);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kExpChains; ++k) x[k] = fmaf(x[k], c, d);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kExpChains; ++k) s += x[k];
    if (s == -1.2345f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Flops of one peaks_mfma_bf16 launch: blocks * 4 waves * iters * kChains * 32768.
// sink: blocks * 256 floats of device memory (never written in practice).
int peaks_mfma_bf16(void* sink, int blocks, int iters, void* stream) {
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (float*)sink, iters);
    return (int)hipGetLastError();
}

// Reads n16 16-byte chunks of src once, in `blocks` contiguous pieces.
// sink: blocks * 256 uint32 of device memory.
int peaks_read_bw(const void* src, int64_t n16, void* sink, int blocks, void* stream) {
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)src, n16, (uint32_t*)sink);
    return (int)hipGetLastError();
}

// LDS bytes read by one launch: blocks * 1024 * iters * 8 * 16.
// sink: blocks * 1024 uint32 of device memory.
int peaks_lds_read(void* sink, int blocks, int iters, void* stream) {
    hipLaunchKernelGGL(lds_read_kernel, dim3(blocks), dim3(1024), 0, (hipStream_t)stream,
                       (uint32_t*)sink, iters);
    return (int)hipGetLastError();
}

// exp2 (fma when use_fma) instructions of one launch: blocks * 256 * iters * 8.
// sink: blocks * 256 floats of device memory.
int peaks_vector_rate(void* sink, int blocks, int iters, int use_fma, void* stream) {
    if (use_fma)
        hipLaunchKernelGGL(fma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                           (float*)sink, iters, 0.5f, 0.25f);
    else
        hipLaunchKernelGGL(exp_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                           (float*)sink, iters);
    return (int)hipGetLastError();
}

int peaks_mfma_chains(void) { return kChains; }
int peaks_vector_chains(void) { return kExpChains; }

}  // extern "C"
