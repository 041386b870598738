// Differential Attention prefill for fp32 inputs (gfx950).
//
// Operator: the DiffAttn formula (iloveeagents.com, "Mathematical Formula")
// followed by the per-head GroupNorm and (1 - lambda_init) scale of step 4 on
// llmbytes.dev ("How Differential Attention Cancels Common-Mode Noise").
//
// gfx950 has no reduced-precision fp32 matrix path that would keep fp32
// accuracy, so this variant runs on the vector ALUs in full fp32 with the same
// one-sweep structure as the bf16 kernel: one workgroup owns 32 query rows of
// one (batch, head), K1/K2/V tiles of 32 keys pass through LDS, each map keeps
// its own online-softmax state (max, sum, O), and the subtraction, GroupNorm and
// scale happen in the epilogue.  It serves small fp32 problems; the bf16 MFMA
// kernel is the throughput path.

#include "internal.h"

#include <math.h>

namespace diffattn {
namespace {

constexpr int kThreads = 256;
constexpr int kBr = 32;
constexpr int kBc = 32;

__device__ __forceinline__ float xor_lanes(float x, int m) { return __shfl_xor(x, m); }

// a*b - c*d with both products rounded before the subtraction (no fused
// multiply-add), so equal operands cancel to exactly zero
__device__ __forceinline__ float diff_of_products(float a, float b, float c, float d) {
#pragma clang fp contract(off)
    return a * b - c * d;
}

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillArgs a) {
    __shared__ float q1s[kBr][D], q2s[kBr][D];
    __shared__ float k1s[kBc][D + 1], k2s[kBc][D + 1];
    __shared__ float vs[kBc][DV];
    __shared__ float p1s[kBr][kBc + 1], p2s[kBr][kBc + 1];
    __shared__ float al1s[kBr], al2s[kBr], m1s[kBr], m2s[kBr], l1s[kBr], l2s[kBr];

    const int tid = threadIdx.x;
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + kBr - 1) / kBr;
    const int t = blockIdx.x / BH;
    const int bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? (nqt - 1 - t) : t;
    const int h = bh % a.H;

    const float* gq1 = (const float*)a.q1 + (size_t)bh * a.Nq * D;
    const float* gq2 = (const float*)a.q2 + (size_t)bh * a.Nq * D;
    const float* gk1 = (const float*)a.k1 + (size_t)bh * a.Nk * D;
    const float* gk2 = (const float*)a.k2 + (size_t)bh * a.Nk * D;
    const float* gv = (const float*)a.v + (size_t)bh * a.Nk * DV;
    float* gout = (float*)a.out + (size_t)bh * a.Nq * DV;

    const int q0 = qt * kBr;
    for (int idx = tid; idx < kBr * D; idx += kThreads) {
        const int r = idx / D, c = idx % D;
        const bool ok = q0 + r < a.Nq;
        q1s[r][c] = ok ? gq1[(size_t)(q0 + r) * D + c] : 0.f;
        q2s[r][c] = ok ? gq2[(size_t)(q0 + r) * D + c] : 0.f;
    }
    if (tid < kBr) {
        m1s[tid] = -INFINITY;
        m2s[tid] = -INFINITY;
        l1s[tid] = 0.f;
        l2s[tid] = 0.f;
    }

    const float inv_sqrt_d = 1.f / sqrtf((float)D);
    const int row = tid >> 3;  // query row this thread accumulates
    const int cg = tid & 7;    // its channel / key group
    float o1[DV / 8], o2[DV / 8];
#pragma unroll
    for (int u = 0; u < DV / 8; ++u) {
        o1[u] = 0.f;
        o2[u] = 0.f;
    }

    const int nkt_all = (a.Nk + kBc - 1) / kBc;
    const int nkt = CAUSAL ? min(nkt_all, (q0 + kBr + kBc - 1) / kBc) : nkt_all;
    for (int kt = 0; kt < nkt; ++kt) {
        const int key0 = kt * kBc;
        __syncthreads();  // previous tile fully consumed
        for (int idx = tid; idx < kBc * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const bool ok = key0 + r < a.Nk;
            k1s[r][c] = ok ? gk1[(size_t)(key0 + r) * D + c] : 0.f;
            k2s[r][c] = ok ? gk2[(size_t)(key0 + r) * D + c] : 0.f;
        }
        for (int idx = tid; idx < kBc * DV; idx += kThreads) {
            const int r = idx / DV, c = idx % DV;
            vs[r][c] = key0 + r < a.Nk ? gv[(size_t)(key0 + r) * DV + c] : 0.f;
        }
        __syncthreads();

        // scaled scores of both maps, masked entries at -inf
#pragma unroll
        for (int u = 0; u < kBc / 8; ++u) {
            const int j = cg + 8 * u;
            float s1 = 0.f, s2 = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; ++c) {
                s1 = fmaf(q1s[row][c], k1s[j][c], s1);
                s2 = fmaf(q2s[row][c], k2s[j][c], s2);
            }
            const int key = key0 + j;
            const bool ok = key < a.Nk && (!CAUSAL || key <= q0 + row);
            p1s[row][j] = ok ? s1 * inv_sqrt_d : -INFINITY;
            p2s[row][j] = ok ? s2 * inv_sqrt_d : -INFINITY;
        }
        __syncthreads();

        // online softmax update, one thread per (map, row)
        if (tid < 2 * kBr) {
            const int r = tid % kBr;
            float(*p)[kBc + 1] = tid < kBr ? p1s : p2s;
            float* ms = tid < kBr ? m1s : m2s;
            float* ls = tid < kBr ? l1s : l2s;
            float* as = tid < kBr ? al1s : al2s;
            float mx = -INFINITY;
            for (int j = 0; j < kBc; ++j) mx = fmaxf(mx, p[r][j]);
            const float mold = ms[r];
            const float mnew = fmaxf(mold, mx);
            const float base = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = expf(mold - base);
            float sum = 0.f;
            for (int j = 0; j < kBc; ++j) {
                const float e = expf(p[r][j] - base);
                p[r][j] = e;
                sum += e;
            }
            ms[r] = mnew;
            ls[r] = ls[r] * alpha + sum;
            as[r] = alpha;
        }
        __syncthreads();

        const float a1 = al1s[row], a2 = al2s[row];
#pragma unroll
        for (int u = 0; u < DV / 8; ++u) {
            const int c = cg + 8 * u;
            float acc1 = o1[u] * a1, acc2 = o2[u] * a2;
#pragma unroll 8
            for (int j = 0; j < kBc; ++j) {
                acc1 = fmaf(p1s[row][j], vs[j][c], acc1);
                acc2 = fmaf(p2s[row][j], vs[j][c], acc2);
            }
            o1[u] = acc1;
            o2[u] = acc2;
        }
    }
    __syncthreads();

    // epilogue: the 8 threads of a row are 8 consecutive lanes of one wave
    const float lam = a.lam[h];
    const float c1 = 1.f / l1s[row];
    const float c2 = lam / l2s[row];
    float dsum = 0.f;
#pragma unroll
    for (int u = 0; u < DV / 8; ++u) {
        o1[u] = diff_of_products(o1[u], c1, o2[u], c2);
        dsum += o1[u];
    }
    if (!(a.flags & 1u)) {
        dsum += xor_lanes(dsum, 1);
        dsum += xor_lanes(dsum, 2);
        dsum += xor_lanes(dsum, 4);
        const float mean = dsum / DV;
        float vsum = 0.f;
#pragma unroll
        for (int u = 0; u < DV / 8; ++u) {
            const float c = o1[u] - mean;
            vsum = fmaf(c, c, vsum);
        }
        vsum += xor_lanes(vsum, 1);
        vsum += xor_lanes(vsum, 2);
        vsum += xor_lanes(vsum, 4);
        const float scale = (1.f - a.lambda_init) / sqrtf(vsum / DV + a.eps);
#pragma unroll
        for (int u = 0; u < DV / 8; ++u) o1[u] = (o1[u] - mean) * scale;
    }
    const int q = q0 + row;
    if (q < a.Nq) {
#pragma unroll
        for (int u = 0; u < DV / 8; ++u) gout[(size_t)q * DV + cg + 8 * u] = o1[u];
    }
}

template <int D, int DV>
hipError_t launch_dims(const PrefillArgs& a, bool causal, hipStream_t stream) {
    const int nqt = (a.Nq + kBr - 1) / kBr;
    const dim3 grid((unsigned)((int64_t)nqt * a.B * a.H));
    PrefillArgs copy = a;
    void* args[] = {&copy};
    const void* fn = causal ? (const void*)prefill_f32_kernel<D, DV, true>
                            : (const void*)prefill_f32_kernel<D, DV, false>;
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, int dv, bool causal,
                              hipStream_t stream) {
    if (d == 32 && dv == 64) return launch_dims<32, 64>(a, causal, stream);
    if (d == 64 && dv == 128) return launch_dims<64, 128>(a, causal, stream);
    if (d == 128 && dv == 256) return launch_dims<128, 256>(a, causal, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
