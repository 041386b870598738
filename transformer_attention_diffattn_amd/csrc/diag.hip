// Diagnostics of the two softmax maps, for bf16 inputs on gfx950: the
// quantities the pages report for trained models, computed here on the
// synthetic needle workload.
//
//   row max  each query row's largest scaled score q_i . k_j / sqrt(d) over
//            the keys it sees, per map -- the top attention logit whose size
//            the pages compare between models (llmbytes.dev, "Solving the
//            Quantization Crisis").  A QK^T-only sweep on MFMA; the forward's
//            running maximum is lazy, so it is not this exact value.
//   needles  for planted (query, key) pairs: the weight each map puts on the
//            pair, and the query row's total weight on all of the head's
//            needle keys -- the attention share on needles the pages report
//            for multi-needle retrieval (same page, "Benchmark Performance").
//            The weights come from the training forward's log-sum-exp:
//            A_k(i, j) = exp(S_k(i, j) - lse_k(i)).

#include "internal.h"
#include "tile_ops.h"

#include <math.h>

namespace diffattn {
namespace {

using namespace tile;

// Row maxima: workgroup = 64 query rows of one (b, h); wave w owns rows
// 32 (w % 2) .. of map w / 2.  Key tiles of 32 go through two LDS buffers.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void diag_rowmax_kernel(DiagArgs a) {
    constexpr int NKB = D / 16, KS = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sk[2][2][32 * KS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int qb = wave & 1, map = wave >> 1;
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + 63) / 64;
    const int t = blockIdx.x / BH;  // longest causal tiles first
    const int bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int qrow = qt * 64 + qb * 32 + l32;
    const bool qok = qrow < a.Nq;

    const uint16_t* gq = (const uint16_t*)(map ? a.q2 : a.q1) + (size_t)bh * a.Nq * D;
    const uint16_t* gk1 = (const uint16_t*)a.k1 + (size_t)bh * a.Nk * D;
    const uint16_t* gk2 = (const uint16_t*)a.k2 + (size_t)bh * a.Nk * D;
    bf16x8 qf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
        qf[kb] = qok ? *(const bf16x8*)(gq + (size_t)qrow * D + 16 * kb + 8 * lh) : bf16x8{};

    const int nkt_all = (a.Nk + 31) / 32;
    const int nkt = CAUSAL ? min(nkt_all, (qt * 64 + 64 + 31) / 32) : nkt_all;
    RowTile<D> t1, t2;
    t1.load(gk1, 0, a.Nk);
    t2.load(gk2, 0, a.Nk);
    t1.store(sk[0][0]);
    t2.store(sk[0][1]);
    __syncthreads();
    float m = -INFINITY;
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) {
            t1.load(gk1, (int64_t)(kt + 1) * 32, a.Nk);
            t2.load(gk2, (int64_t)(kt + 1) * 32, a.Nk);
        }
        // S^T = K Q^T with key rows in swap23 order: register r is key
        // 16 (r/8) + 8 lh + r%8 of the tile, column l32 this lane's query
        f32x16 s = f32x16{};
        const uint16_t* kt_ = sk[buf][map];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s = mfma(rd_row(kt_, KS, swap23(l32), 16 * kb, lh), qf[kb], s);
        // the mask is needed only where the tile meets the diagonal or the
        // ragged end (a wave-uniform test; elsewhere every key is visible)
        const int qw0 = __builtin_amdgcn_readfirstlane(qt * 64 + qb * 32);
        if (kt * 32 + 31 < a.Nk && (!CAUSAL || kt * 32 + 31 <= qw0)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, s[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt * 32 + 16 * (r >> 3) + 8 * lh + (r & 7);
                const bool ok = key < a.Nk && (!CAUSAL || key <= qrow);
                m = fmaxf(m, ok ? s[r] : -INFINITY);
            }
        }
        if (more) {
            t1.store(sk[buf ^ 1][0]);
            t2.store(sk[buf ^ 1][1]);
        }
        __syncthreads();
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    if (qok && lh == 0)
        a.row_max[((size_t)map * BH + bh) * a.Nq + qrow] = m * (1.f / sqrtf((float)D));
}

// Needles: workgroup = one (b, h); thread r handles needle r (query
// needle_q[r], key needle_k[r]).  Scores in fp32 from the bf16 inputs, in a
// fixed order.  A needle whose query or key is out of range gets NaNs.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void diag_needles_kernel(DiagArgs a) {
    const int bh = blockIdx.x;
    const int BH = a.B * a.H;
    const int n = a.n_needles;
    const int32_t* nq = a.needle_q + (size_t)bh * n;
    const int32_t* nk = a.needle_k + (size_t)bh * n;
    const float tau = 1.f / sqrtf((float)D);
    for (int r = threadIdx.x; r < n; r += kBwdThreads) {
        const int i = nq[r];
        float* o = a.needles + ((size_t)bh * n + r) * 4;
        if (i < 0 || i >= a.Nq || nk[r] < 0 || nk[r] >= a.Nk) {
            o[0] = o[1] = o[2] = o[3] = NAN;
            continue;
        }
        const __bf16* q1 = (const __bf16*)a.q1 + ((size_t)bh * a.Nq + i) * D;
        const __bf16* q2 = (const __bf16*)a.q2 + ((size_t)bh * a.Nq + i) * D;
        const float lse1 = a.lse[(size_t)bh * a.Nq + i];
        const float lse2 = a.lse[((size_t)BH + bh) * a.Nq + i];
        float own1 = 0.f, own2 = 0.f, sum1 = 0.f, sum2 = 0.f;
        for (int mm = 0; mm < n; ++mm) {
            const int j = nk[mm];
            if (j < 0 || j >= a.Nk || (CAUSAL && j > i)) continue;
            const __bf16* k1 = (const __bf16*)a.k1 + ((size_t)bh * a.Nk + j) * D;
            const __bf16* k2 = (const __bf16*)a.k2 + ((size_t)bh * a.Nk + j) * D;
            float s1 = 0.f, s2 = 0.f;
            for (int c = 0; c < D; ++c) {
                s1 = fmaf((float)q1[c], (float)k1[c], s1);
                s2 = fmaf((float)q2[c], (float)k2[c], s2);
            }
            const float a1 = expf(s1 * tau - lse1), a2 = expf(s2 * tau - lse2);
            sum1 += a1;
            sum2 += a2;
            if (mm == r) {
                own1 = a1;
                own2 = a2;
            }
        }
        o[0] = own1;
        o[1] = own2;
        o[2] = sum1;
        o[3] = sum2;
    }
}

template <int D>
hipError_t launch_d(const DiagArgs& a, bool causal, hipStream_t stream) {
    DiagArgs copy = a;
    void* args[] = {&copy};
    const int64_t BH = (int64_t)a.B * a.H;
    if (a.row_max) {
        const int64_t g = (int64_t)((a.Nq + 63) / 64) * BH;
        if (g > 0x7fffffff) return hipErrorInvalidValue;
        const hipError_t e = hipLaunchKernel(causal ? (const void*)diag_rowmax_kernel<D, true>
                                                    : (const void*)diag_rowmax_kernel<D, false>,
                                             dim3((unsigned)g), dim3(kBwdThreads), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (a.needles && a.n_needles > 0) {
        if (BH > 0x7fffffff) return hipErrorInvalidValue;
        return hipLaunchKernel(causal ? (const void*)diag_needles_kernel<D, true>
                                      : (const void*)diag_needles_kernel<D, false>,
                               dim3((unsigned)BH), dim3(kBwdThreads), args, 0, stream);
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_diag_bf16(const DiagArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 32) return launch_d<32>(a, causal, stream);
    if (d == 64) return launch_d<64>(a, causal, stream);
    if (d == 128) return launch_d<128>(a, causal, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
