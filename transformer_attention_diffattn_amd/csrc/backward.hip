// Backward of the fused Differential Attention operator for bf16 inputs on
// gfx950, head_dim 32 or 64 (v_dim 64 or 128); head_dim 128 (v_dim 256) runs
// the prep and dlambda kernels here and the dQ and dK/dV kernels of
// backward_ring.hip.
//
// The pages treat the operator as trained: lambda is learnable
// (iloveeagents.com, "Mathematical Formula") and the per-head GroupNorm with
// the (1 - lambda_init) scale of step 4 on llmbytes.dev ("How Differential
// Attention Cancels Common-Mode Noise") keeps gradients stable.  This is the
// chain rule through that forward, in the forward's notation (tau = 1/sqrt(d)):
//
//   dD   = GroupNorm backward of dy (or dy itself for a pre-norm output);
//   dP   = dD V^T                       (shared by both maps: dA1 = dP,
//                                        dA2 = -lambda dP);
//   delta_k = rowsum(A_k * dP);
//   dS_1 = A_1 (dP - delta_1),  dS_2 = -lambda A_2 (dP - delta_2);
//   dQ_k = tau dS_k K_k,  dK_k = tau dS_k^T Q_k,  dV = (A_1 - lambda A_2)^T dD;
//   dlambda = -sum(O_2 . dD) = -sum_rows delta_2.
//
// A_k is recomputed from the scores and the per-row log-sum-exp that the
// training forward saved, so no N x N map is ever stored.  Four kernels, in
// stream order:
//   prep   one wave per row: dD from the saved D and dy, in bf16 for the MFMAs;
//   dq     a workgroup per 64 query rows (wave = 32 rows of one map), looping
//          over key tiles; dQ_k = tau (X_k - delta_k Y_k) with X_k = (A_k * dP)
//          K_k and Y_k = A_k K_k, so delta_k comes out of the same sweep;
//          writes dQ and delta_k;
//   dkdv   a workgroup per 128 keys, looping over query tiles; head_dim 32:
//          wave = 32 keys and both maps, accumulating dV^T and dK_k^T on
//          32x32x16 products; head_dim 64 (dkdv16): wave = 16 keys and both
//          maps on 16x16x32 products, two waves per SIMD;
//   dlam   one workgroup per head: dlambda = -sum delta_2 (fixed order).
//
// MFMA v_mfma_f32_32x32x16_bf16 throughout (lane l, lh = l / 32, l32 = l % 32:
// A row l32 / B column l32 hold k-slots 8 lh .. 8 lh + 7; accumulator register
// r is row 8 (r/4) + 4 lh + r%4, column l32).  A product whose output rows feed
// the next product's k dimension loads its A rows in swap23 order, which makes
// accumulator registers 8c .. 8c+7 exactly the k-slots of 16-row step c; the
// other operands are either rows read 16 bytes at a time or columns read with
// the transposing ds_read_b64_tr_b16.  Tiles sit in LDS row-major with rows
// padded by 16 bytes.

#include "internal.h"
#include "tile_ops.h"

#include <math.h>

namespace diffattn {
namespace {

using namespace tile;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// ---------------------------------------------------------------------------
// prep: dD for every row.  A wave takes kPrepRows rows, lane l elements
// kPer l .. kPer l + kPer - 1 of each (vector loads), and issues all the
// rows' loads before the first reduction: with one row per wave the kernel
// waited out one load latency per row.
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 4;

template <int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(BackwardArgs a) {
    constexpr int kPer = DV / 64;
    typedef float fv __attribute__((ext_vector_type(kPer)));
    typedef __bf16 bv __attribute__((ext_vector_type(kPer)));
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6)) * kPrepRows;
    const int64_t rows = (int64_t)a.B * a.H * a.Nq;
    if (row0 >= rows) return;
    fv y[kPrepRows], x[kPrepRows];
#pragma unroll
    for (int j = 0; j < kPrepRows; ++j) {
        const int64_t row = min(row0 + j, rows - 1);  // (a repeated last row is not stored)
        const bv yb = *(const bv*)((const __bf16*)a.dout + row * DV + kPer * lane);
#pragma unroll
        for (int i = 0; i < kPer; ++i) y[j][i] = (float)yb[i];
        if (!(a.flags & 1u)) x[j] = *(const fv*)(a.d_save + row * DV + kPer * lane);
    }
#pragma unroll
    for (int j = 0; j < kPrepRows; ++j) {
        fv dd;
        if (a.flags & 1u) {
            dd = y[j];
        } else {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < kPer; ++i) s += x[j][i];
            const float mu = wave_sum(s) * (1.f / DV);
            float q = 0.f;
#pragma unroll
            for (int i = 0; i < kPer; ++i) q = fmaf(x[j][i] - mu, x[j][i] - mu, q);
            const float inv = 1.f / sqrtf(wave_sum(q) * (1.f / DV) + a.eps);
            const float c = 1.f - a.lambda_init;
            float sg = 0.f, sgx = 0.f;
            fv xh, g;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                xh[i] = (x[j][i] - mu) * inv;
                g[i] = y[j][i] * c;
                sg += g[i];
                sgx = fmaf(g[i], xh[i], sgx);
            }
            const float mg = wave_sum(sg) * (1.f / DV);
            const float mgx = wave_sum(sgx) * (1.f / DV);
#pragma unroll
            for (int i = 0; i < kPer; ++i) dd[i] = (g[i] - mg - xh[i] * mgx) * inv;
        }
        if (row0 + j < rows) {
            bv ob;
#pragma unroll
            for (int i = 0; i < kPer; ++i) ob[i] = (__bf16)dd[i];
            *(bv*)((__bf16*)a.dd + (row0 + j) * DV + kPer * lane) = ob;
        }
    }
}

// ---------------------------------------------------------------------------
// dq: dQ_k and delta_k.  Workgroup = 64 query rows of one (b, h); wave w owns
// rows 32 (w % 2) .. of map w / 2.
// ---------------------------------------------------------------------------
template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BackwardArgs a) {
    constexpr int NKB = D / 16, NVB = DV / 16, NCB = D / 32;
    constexpr int KS = D + 8, VS = DV + 8;
    // two buffers, each K1 | K2 | V of one 32-key tile
    __shared__ __attribute__((aligned(16))) uint16_t sk[2][2][32 * KS];
    __shared__ __attribute__((aligned(16))) uint16_t sv[2][32 * VS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int qb = wave & 1, map = wave >> 1;
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + 63) / 64;
    const int t = blockIdx.x / BH;  // longest causal tiles first
    const int bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int h = bh % a.H;
    const int qrow = qt * 64 + qb * 32 + l32;
    const bool qok = qrow < a.Nq;

    const uint16_t* gq = (const uint16_t*)(map ? a.q2 : a.q1) + (size_t)bh * a.Nq * D;
    const uint16_t* gk1 = (const uint16_t*)a.k1 + (size_t)bh * a.Nk * D;
    const uint16_t* gk2 = (const uint16_t*)a.k2 + (size_t)bh * a.Nk * D;
    const uint16_t* gv = (const uint16_t*)a.v + (size_t)bh * a.Nk * DV;
    const uint16_t* gdd = (const uint16_t*)a.dd + (size_t)bh * a.Nq * DV;

    // B operands of this lane's query (column l32): Q_k^T over d, dD^T over dv
    bf16x8 qf[NKB], df[NVB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
        qf[kb] = qok ? *(const bf16x8*)(gq + (size_t)qrow * D + 16 * kb + 8 * lh) : bf16x8{};
#pragma unroll
    for (int c = 0; c < NVB; ++c)
        df[c] = qok ? *(const bf16x8*)(gdd + (size_t)qrow * DV + 16 * c + 8 * lh) : bf16x8{};
    const float lse2 =
        qok ? a.lse[((size_t)map * BH + bh) * a.Nq + qrow] * kLog2e : 0.f;
    const float sl2 = a.scale_log2;

    f32x16 xt[NCB], yt[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) xt[cb] = yt[cb] = f32x16{};
    float dsum = 0.f;

    const int nkt_all = (a.Nk + 31) / 32;
    const int nkt = CAUSAL ? min(nkt_all, (qt * 64 + 64 + 31) / 32) : nkt_all;
    RowTile<D> t1, t2;
    RowTile<DV> tv;
    t1.load(gk1, 0, a.Nk);
    t2.load(gk2, 0, a.Nk);
    tv.load(gv, 0, a.Nk);
    t1.store(sk[0][0]);
    t2.store(sk[0][1]);
    tv.store(sv[0]);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) {  // next tile's loads fly while this one is used
            t1.load(gk1, (int64_t)(kt + 1) * 32, a.Nk);
            t2.load(gk2, (int64_t)(kt + 1) * 32, a.Nk);
            tv.load(gv, (int64_t)(kt + 1) * 32, a.Nk);
        }
        const uint16_t* kt_ = sk[buf][map];
        const uint16_t* sv_ = sv[buf];
        // S^T = K Q^T and dP^T = V dD^T, key rows in swap23 order
        f32x16 s = f32x16{}, dp = f32x16{};
        const int kr = swap23(l32);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s = mfma(rd_row(kt_, KS, kr, 16 * kb, lh), qf[kb], s);
#pragma unroll
        for (int c = 0; c < NVB; ++c) dp = mfma(rd_row(sv_, VS, kr, 16 * c, lh), df[c], dp);
        float p[16], w[16];
        // the mask is needed only where the tile meets the diagonal or a
        // ragged end (a wave-uniform test; elsewhere every pair is visible)
        const int qw0 = __builtin_amdgcn_readfirstlane(qt * 64 + qb * 32);
        const bool full = qw0 + 31 < a.Nq && kt * 32 + 31 < a.Nk && (!CAUSAL || kt * 32 + 31 <= qw0);
        auto probs = [&](auto masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = fmaf(s[r], sl2, -lse2);
                if constexpr (decltype(masked)::value) {
                    const int key = kt * 32 + 16 * (r >> 3) + 8 * lh + (r & 7);
                    const bool ok = qok && key < a.Nk && (!CAUSAL || key <= qrow);
                    asm volatile("" : "+v"(x));  // formed for every lane (no branch)
                    x = ok ? x : -INFINITY;
                }
                p[r] = __builtin_amdgcn_exp2f(x);
                w[r] = p[r] * dp[r];
                dsum += w[r];
            }
        };
        if (full)
            probs(std::false_type{});
        else
            probs(std::true_type{});
        bf16x8 pp[2], pw[2];
        pack(p, pp);
        pack(w, pw);
        // X^T += K^T (A*dP)^T,  Y^T += K^T A^T
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 kc = rd_col(kt_, KS, 16 * kk, 32 * cb, lane);
                xt[cb] = mfma(kc, pw[kk], xt[cb]);
                yt[cb] = mfma(kc, pp[kk], yt[cb]);
            }
        }
        // the other buffer was last read before the previous barrier
        if (more) {
            t1.store(sk[buf ^ 1][0]);
            t2.store(sk[buf ^ 1][1]);
            tv.store(sv[buf ^ 1]);
        }
        __syncthreads();
    }

    const float delta = dsum + __shfl_xor(dsum, 32);
    if (!qok) return;
    const float tau = 1.f / sqrtf((float)D);
    const float sc = map ? -a.lam[h] * tau : tau;
    __bf16* gout = (__bf16*)(map ? a.dq2 : a.dq1) + ((size_t)bh * a.Nq + qrow) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = (__bf16)(sc * (xt[cb][4 * g + e] - delta * yt[cb][4 * g + e]));
            *(bf16x4*)(gout + 32 * cb + 8 * g + 4 * lh) = o;
        }
    }
    if (lh == 0) a.delta[((size_t)map * BH + bh) * a.Nq + qrow] = delta;
}

// ---------------------------------------------------------------------------
// dkdv: dK_1, dK_2 and dV.  Workgroup = 128 keys of one (b, h); wave w owns
// keys 32 w .. 32 w + 31 and both maps.
// ---------------------------------------------------------------------------
template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BackwardArgs a) {
    constexpr int NKB = D / 16, NVB = DV / 16, NCB = D / 32, NDB = DV / 32;
    constexpr int KS = D + 8, VS = DV + 8;
    // two buffers, each Q1 | Q2 | dD and the row terms of one 32-query tile
    __shared__ __attribute__((aligned(16))) uint16_t sq[2][2][32 * KS];
    __shared__ __attribute__((aligned(16))) uint16_t sd[2][32 * VS];
    // per query: lse1, lse2 (log2 units), delta1, delta2 -- one 16-byte read
    __shared__ __attribute__((aligned(16))) float4 srow[2][32];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int BH = a.B * a.H;
    // key tile kt = blockIdx / BH: under the causal mask the first key tiles
    // see the most queries, so the longest workgroups start first
    const int kt = blockIdx.x / BH;
    const int bh = blockIdx.x - kt * BH;
    const int h = bh % a.H;
    const int key = kt * 128 + wave * 32 + l32;
    const bool kok = key < a.Nk;

    const uint16_t* gk1 = (const uint16_t*)a.k1 + (size_t)bh * a.Nk * D;
    const uint16_t* gk2 = (const uint16_t*)a.k2 + (size_t)bh * a.Nk * D;
    const uint16_t* gv = (const uint16_t*)a.v + (size_t)bh * a.Nk * DV;
    const uint16_t* gq1 = (const uint16_t*)a.q1 + (size_t)bh * a.Nq * D;
    const uint16_t* gq2 = (const uint16_t*)a.q2 + (size_t)bh * a.Nq * D;
    const uint16_t* gdd = (const uint16_t*)a.dd + (size_t)bh * a.Nq * DV;

    // B operands of this lane's key (column l32): K_k^T over d, V^T over dv
    bf16x8 k1f[NKB], k2f[NKB], vf[NVB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        k1f[kb] = kok ? *(const bf16x8*)(gk1 + (size_t)key * D + 16 * kb + 8 * lh) : bf16x8{};
        k2f[kb] = kok ? *(const bf16x8*)(gk2 + (size_t)key * D + 16 * kb + 8 * lh) : bf16x8{};
    }
#pragma unroll
    for (int c = 0; c < NVB; ++c)
        vf[c] = kok ? *(const bf16x8*)(gv + (size_t)key * DV + 16 * c + 8 * lh) : bf16x8{};
    const float sl2 = a.scale_log2;
    const float lam = a.lam[h];

    f32x16 dvt[NDB], dk1t[NCB], dk2t[NCB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dvt[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < NCB; ++i) dk1t[i] = dk2t[i] = f32x16{};

    const int nqt = (a.Nq + 31) / 32;
    const int qt0 = CAUSAL ? (kt * 128) / 32 : 0;
    const float* lse1 = a.lse + (size_t)bh * a.Nq;
    const float* lse2 = a.lse + ((size_t)BH + bh) * a.Nq;
    const float* del1 = a.delta + (size_t)bh * a.Nq;
    const float* del2 = a.delta + ((size_t)BH + bh) * a.Nq;
    // row terms: thread t < 128 carries term t / 32 of query t % 32
    const int which = threadIdx.x >> 5;
    const float row_scale = which < 2 ? kLog2e : 1.f;  // log-sum-exps to log2 units
    auto put_row = [&](int b, float v) {
        if (threadIdx.x < 128) ((float*)&srow[b][threadIdx.x & 31])[which] = v * row_scale;
    };
    const float* rsrc = which == 0 ? lse1 : which == 1 ? lse2 : which == 2 ? del1 : del2;
    // rows past Nq load the last row's terms (an index clamp, not a select
    // on the loaded value, so nothing waits for the load before put_row);
    // their pairs are masked
    auto load_row = [&](int qt) {
        return rsrc[min(qt * 32 + (int)(threadIdx.x & 31), a.Nq - 1)];
    };
    RowTile<D> t1, t2;
    RowTile<DV> td;
    float rv = 0.f;
    if (qt0 < nqt) {
        t1.load(gq1, (int64_t)qt0 * 32, a.Nq);
        t2.load(gq2, (int64_t)qt0 * 32, a.Nq);
        td.load(gdd, (int64_t)qt0 * 32, a.Nq);
        rv = load_row(qt0);
        t1.store(sq[0][0]);
        t2.store(sq[0][1]);
        td.store(sd[0]);
        put_row(0, rv);
    }
    __syncthreads();
    for (int qt = qt0; qt < nqt; ++qt) {
        const int buf = (qt - qt0) & 1;
        const bool more = qt + 1 < nqt;
        if (more) {  // next tile's loads fly while this one is used
            t1.load(gq1, (int64_t)(qt + 1) * 32, a.Nq);
            t2.load(gq2, (int64_t)(qt + 1) * 32, a.Nq);
            td.load(gdd, (int64_t)(qt + 1) * 32, a.Nq);
            rv = load_row(qt + 1);
        }
        const uint16_t* sq1 = sq[buf][0];
        const uint16_t* sq2 = sq[buf][1];
        const uint16_t* sd_ = sd[buf];
        const float4* sr = srow[buf];
        // S_k = Q_k K_k^T and dP = dD V^T, query rows in swap23 order.  All
        // operand reads are issued before the first product (one wave per
        // SIMD: nothing else hides the LDS latency of a read issued right
        // before its product)
        const int qr = swap23(l32);
        bf16x8 aq1[NKB], aq2[NKB], ad[NVB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            aq1[kb] = rd_row(sq1, KS, qr, 16 * kb, lh);
            aq2[kb] = rd_row(sq2, KS, qr, 16 * kb, lh);
        }
#pragma unroll
        for (int c = 0; c < NVB; ++c) ad[c] = rd_row(sd_, VS, qr, 16 * c, lh);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s1 = f32x16{}, s2 = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s1 = mfma(aq1[kb], k1f[kb], s1);
            s2 = mfma(aq2[kb], k2f[kb], s2);
        }
#pragma unroll
        for (int c = 0; c < NVB; ++c) dp = mfma(ad[c], vf[c], dp);
        // the transposed operands of the dV and dK products (independent of
        // the vector work below), in flight meanwhile.  The row terms are
        // read where they are used: held for all 16 rows they took 64
        // registers, whose copies to and from the accumulation registers
        // cost more than the reads' latency (2K workload backward 0.536 ->
        // 0.500 ms, back to back on one GPU).
        bf16x8 ov[2][NDB], o1c[2][NCB], o2c[2][NCB];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb) ov[kk][cb] = rd_col(sd_, VS, 16 * kk, 32 * cb, lane);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                o1c[kk][cb] = rd_col(sq1, KS, 16 * kk, 32 * cb, lane);
                o2c[kk][cb] = rd_col(sq2, KS, 16 * kk, 32 * cb, lane);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        float wd[16], d1[16], d2[16];
        // the mask is needed only where the tile meets the diagonal or a
        // ragged end (a wave-uniform test; elsewhere every pair is visible)
        const int kw0 = __builtin_amdgcn_readfirstlane(kt * 128 + wave * 32);
        const bool full = kw0 + 31 < a.Nk && qt * 32 + 31 < a.Nq && (!CAUSAL || kw0 + 31 <= qt * 32);
        auto probs = [&](auto masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float4 t = sr[16 * (r >> 3) + 8 * lh + (r & 7)];
                float x1 = fmaf(s1[r], sl2, -t.x), x2 = fmaf(s2[r], sl2, -t.y);
                if constexpr (decltype(masked)::value) {
                    const int qi = 16 * (r >> 3) + 8 * lh + (r & 7);
                    const int q = qt * 32 + qi;
                    const bool ok = kok && q < a.Nq && (!CAUSAL || key <= q);
                    // masked pairs take exp2(-inf) = 0; the arguments are formed
                    // for every lane (the empty asm keeps the compiler from
                    // moving them, and the row-term read, into a branch per
                    // element)
                    asm volatile("" : "+v"(x1), "+v"(x2));
                    x1 = ok ? x1 : -INFINITY;
                    x2 = ok ? x2 : -INFINITY;
                }
                const float p1 = __builtin_amdgcn_exp2f(x1);
                const float p2 = __builtin_amdgcn_exp2f(x2);
                wd[r] = p1 - lam * p2;
                d1[r] = p1 * (dp[r] - t.z);
                d2[r] = -lam * p2 * (dp[r] - t.w);
            }
        };
        if (full)
            probs(std::false_type{});
        else
            probs(std::true_type{});
        bf16x8 pwd[2], pd1[2], pd2[2];
        pack(wd, pwd);
        pack(d1, pd1);
        pack(d2, pd2);
        // dV^T += dD^T W,  dK_k^T += Q_k^T dS_k  (k = queries)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb) dvt[cb] = mfma(ov[kk][cb], pwd[kk], dvt[cb]);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                dk1t[cb] = mfma(o1c[kk][cb], pd1[kk], dk1t[cb]);
                dk2t[cb] = mfma(o2c[kk][cb], pd2[kk], dk2t[cb]);
            }
        }
        // the other buffer was last read before the previous barrier
        if (more) {
            t1.store(sq[buf ^ 1][0]);
            t2.store(sq[buf ^ 1][1]);
            td.store(sd[buf ^ 1]);
            put_row(buf ^ 1, rv);
        }
        __syncthreads();
    }

    if (!kok) return;
    const float tau = 1.f / sqrtf((float)D);
    __bf16* o1 = (__bf16*)a.dk1 + ((size_t)bh * a.Nk + key) * D;
    __bf16* o2 = (__bf16*)a.dk2 + ((size_t)bh * a.Nk + key) * D;
    __bf16* ov = (__bf16*)a.dv + ((size_t)bh * a.Nk + key) * DV;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            bf16x4 w1, w2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w1[e] = (__bf16)(tau * dk1t[cb][4 * g + e]);
                w2[e] = (__bf16)(tau * dk2t[cb][4 * g + e]);
            }
            *(bf16x4*)(o1 + 32 * cb + 8 * g + 4 * lh) = w1;
            *(bf16x4*)(o2 + 32 * cb + 8 * g + 4 * lh) = w2;
        }
#pragma unroll
        for (int cb = 0; cb < NDB; ++cb) {
            bf16x4 wv;
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[e] = (__bf16)dvt[cb][4 * g + e];
            *(bf16x4*)(ov + 32 * cb + 8 * g + 4 * lh) = wv;
        }
    }
}

// ---------------------------------------------------------------------------
// dkdv16: the dkdv products for head_dim 64 on v_mfma_f32_16x16x32_bf16, 16
// keys per wave, so that a wave holds half the key-side state of bwd_dkdv and
// two waves share each SIMD.  Workgroup = 128 keys of one (b, h), 8 waves;
// wave w owns keys 16 w .. 16 w + 15 and both maps.
//
// 16x16x32 operands (lane l, g = l / 16, i = l % 16): A row i and B column i
// hold k-slots 8 g .. 8 g + 7; accumulator register r is row 4 g + r, column i.
// Per 32-query tile, in two blocks b of 16 queries:
//   S_k^T[b] = Q_k[b] K_k^T,   dP^T[b] = dD[b] V^T          (queries x keys)
// so lane l holds key i of the wave and queries 16 b + 4 g + r: the eight
// queries 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, which serve as lane
// group g's k-slots in
//   dV += W dD,   dK_k += dS_k Q_k                          (keys x channels)
// whose A operands are the weights already in registers and whose B operands
// (columns of dD and Q_k over those queries) come from two transposing reads
// of four rows each.
// The LDS tiles are unpadded; chunk c (16 bytes) of row r sits at c ^ swz16(r),
// which puts both the row reads (16 rows at one chunk) and the transposing
// reads (8 rows by two chunks per half-wave) on 64 distinct banks.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ int swz16(int r) {
    static_assert(W == 64 || W == 128, "rows of 128 or 256 bytes");
    if constexpr (W == 128)
        return 2 * (r & 7) + ((r >> 3) & 1);
    else
        return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// chunk c of row r of a swizzled tile of W-element rows
template <int W>
__device__ __forceinline__ bf16x8 rd_chunk(const uint16_t* t, int r, int c) {
    return *(const bf16x8*)(t + r * W + 8 * (c ^ swz16<W>(r)));
}

// B operand over queries 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, column
// c0 + i: lane i of a 16-lane group addresses row (i / 4) of its four rows at
// columns c0 + 4 (i % 4) ..  and receives column c0 + i of the four rows
template <int W>
__device__ __forceinline__ bf16x8 rd_qcol(const uint16_t* t, int c0, int lane) {
    const int g = lane >> 4, e = (lane & 15) >> 2, col = c0 + 4 * (lane & 3);
    const int r0 = 4 * g + e, r1 = 16 + 4 * g + e;
    const uint16_t* p0 = t + r0 * W + 8 * ((col >> 3) ^ swz16<W>(r0)) + (col & 7);
    const uint16_t* p1 = t + r1 * W + 8 * ((col >> 3) ^ swz16<W>(r1)) + (col & 7);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr int kKv16Threads = 512;

template <bool CAUSAL>
__global__ __launch_bounds__(kKv16Threads) void bwd_dkdv16_kernel(BackwardArgs a) {
    constexpr int D = 64, DV = 128;
    constexpr int NS = D / 32, NSV = DV / 32;   // k-steps over d and over dv
    constexpr int NC = D / 16, NCV = DV / 16;   // 16-channel output blocks
    // two buffers, each Q1 | Q2 | dD of one 32-query tile and its row terms
    __shared__ __attribute__((aligned(16))) uint16_t sq[2][2][32 * D];
    __shared__ __attribute__((aligned(16))) uint16_t sd[2][32 * DV];
    // per query: lse1, lse2 (log2 units), delta1, delta2
    __shared__ __attribute__((aligned(16))) float4 srow[2][32];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int BH = a.B * a.H;
    // key tile kt = blockIdx / BH: under the causal mask the first key tiles
    // see the most queries, so the longest workgroups start first
    const int kt = blockIdx.x / BH;
    const int bh = blockIdx.x - kt * BH;
    const int h = bh % a.H;
    const int kw0 = kt * 128 + 16 * wave;  // first key of this wave
    const int key = kw0 + i16;             // this lane's key (column i)
    const bool kok = key < a.Nk;

    const uint16_t* gk1 = (const uint16_t*)a.k1 + (size_t)bh * a.Nk * D;
    const uint16_t* gk2 = (const uint16_t*)a.k2 + (size_t)bh * a.Nk * D;
    const uint16_t* gv = (const uint16_t*)a.v + (size_t)bh * a.Nk * DV;
    const uint16_t* gq1 = (const uint16_t*)a.q1 + (size_t)bh * a.Nq * D;
    const uint16_t* gq2 = (const uint16_t*)a.q2 + (size_t)bh * a.Nq * D;
    const uint16_t* gdd = (const uint16_t*)a.dd + (size_t)bh * a.Nq * DV;

    // B operands of this lane's key: K_k^T and V^T, k-step s = channels 32 s + 8 g ..
    bf16x8 k1f[NS], k2f[NS], vf[NSV];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        k1f[s] = kok ? *(const bf16x8*)(gk1 + (size_t)key * D + 32 * s + 8 * g) : bf16x8{};
        k2f[s] = kok ? *(const bf16x8*)(gk2 + (size_t)key * D + 32 * s + 8 * g) : bf16x8{};
    }
#pragma unroll
    for (int s = 0; s < NSV; ++s)
        vf[s] = kok ? *(const bf16x8*)(gv + (size_t)key * DV + 32 * s + 8 * g) : bf16x8{};
    const float sl2 = a.scale_log2;
    const float lam = a.lam[h];

    f32x4 dvv[NCV], dk1[NC], dk2[NC];
#pragma unroll
    for (int c = 0; c < NCV; ++c) dvv[c] = f32x4{};
#pragma unroll
    for (int c = 0; c < NC; ++c) dk1[c] = dk2[c] = f32x4{};

    const int nqt = (a.Nq + 31) / 32;
    const int qt0 = CAUSAL ? (kt * 128) / 32 : 0;
    const float* lse1 = a.lse + (size_t)bh * a.Nq;
    const float* lse2 = a.lse + ((size_t)BH + bh) * a.Nq;
    const float* del1 = a.delta + (size_t)bh * a.Nq;
    const float* del2 = a.delta + ((size_t)BH + bh) * a.Nq;
    // row terms: thread t < 128 carries term t / 32 of query t % 32
    const int which = tid >> 5;
    const float row_scale = which < 2 ? kLog2e : 1.f;  // log-sum-exps to log2 units
    const float* rsrc = which == 0 ? lse1 : which == 1 ? lse2 : which == 2 ? del1 : del2;
    // tile chunks: thread t moves chunk t of Q1 | Q2 (t < 256: Q1) and chunk t of dD
    const int qsel = __builtin_amdgcn_readfirstlane(tid >> 8), qc = tid & 255;  // uniform per wave
    const int q_row = qc >> 3, q_ch = qc & 7;
    const int d_row = tid >> 4, d_ch = tid & 15;
    uint4 rq, rd;
    float rv = 0.f;
    // rows past Nq read as zeros (buffer bounds) and, for the row terms, as the
    // last row's (an index clamp); their pairs are masked
    auto load_tile = [&](int qt) {
        const int64_t row0 = (int64_t)qt * 32;
        const __amdgpu_buffer_rsrc_t rs_q =
            buffer_rsrc((qsel ? gq2 : gq1) + row0 * D, ((int64_t)a.Nq - row0) * D * 2);
        const __amdgpu_buffer_rsrc_t rs_d = buffer_rsrc(gdd + row0 * DV, ((int64_t)a.Nq - row0) * DV * 2);
        rq = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs_q, (q_row * D + 8 * q_ch) * 2, 0, 0));
        rd = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs_d, (d_row * DV + 8 * d_ch) * 2, 0, 0));
        if (tid < 128) rv = rsrc[min(qt * 32 + (tid & 31), a.Nq - 1)];
    };
    auto store_tile = [&](int b) {
        *(uint4*)(&sq[b][qsel][q_row * D + 8 * (q_ch ^ swz16<D>(q_row))]) = rq;
        *(uint4*)(&sd[b][d_row * DV + 8 * (d_ch ^ swz16<DV>(d_row))]) = rd;
        if (tid < 128) ((float*)&srow[b][tid & 31])[which] = rv * row_scale;
    };
    if (qt0 < nqt) {
        load_tile(qt0);
        store_tile(0);
    }
    __syncthreads();
    for (int qt = qt0; qt < nqt; ++qt) {
        const int buf = (qt - qt0) & 1;
        const bool more = qt + 1 < nqt;
        if (more) load_tile(qt + 1);  // in flight while this tile is used
        const uint16_t* sq1 = sq[buf][0];
        const uint16_t* sq2 = sq[buf][1];
        const uint16_t* sd_ = sd[buf];
        const float4* sr = srow[buf];

        // S_k^T and dP^T, query block b: A rows 16 b + i, chunk 4 s + g
        f32x4 s1[2], s2[2], dp[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            s1[b] = s2[b] = dp[b] = f32x4{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                s1[b] = mfma16(rd_chunk<D>(sq1, 16 * b + i16, 4 * s + g), k1f[s], s1[b]);
                s2[b] = mfma16(rd_chunk<D>(sq2, 16 * b + i16, 4 * s + g), k2f[s], s2[b]);
            }
#pragma unroll
            for (int s = 0; s < NSV; ++s)
                dp[b] = mfma16(rd_chunk<DV>(sd_, 16 * b + i16, 4 * s + g), vf[s], dp[b]);
        }
        // the B operands of the dV and dK products (independent of the vector
        // work below), in flight meanwhile
        bf16x8 bd[NCV], bq1[NC], bq2[NC];
#pragma unroll
        for (int c = 0; c < NCV; ++c) bd[c] = rd_qcol<DV>(sd_, 16 * c, lane);
        // weights; the mask only where the tile meets the diagonal or an end
        const bool full = __builtin_amdgcn_readfirstlane(kw0) + 15 < a.Nk && qt * 32 + 31 < a.Nq &&
                          (!CAUSAL || __builtin_amdgcn_readfirstlane(kw0) + 15 <= qt * 32);
        bf16x8 wa, da1, da2;
        auto probs = [&](auto masked) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = 16 * b + 4 * g + r;
                    const float4 t = sr[qi];
                    float x1 = fmaf(s1[b][r], sl2, -t.x), x2 = fmaf(s2[b][r], sl2, -t.y);
                    if constexpr (decltype(masked)::value) {
                        const int q = qt * 32 + qi;
                        const bool ok = kok && q < a.Nq && (!CAUSAL || key <= q);
                        asm volatile("" : "+v"(x1), "+v"(x2));
                        x1 = ok ? x1 : -INFINITY;
                        x2 = ok ? x2 : -INFINITY;
                    }
                    const float p1 = __builtin_amdgcn_exp2f(x1);
                    const float p2 = __builtin_amdgcn_exp2f(x2);
                    wa[4 * b + r] = (__bf16)(p1 - lam * p2);
                    da1[4 * b + r] = (__bf16)(p1 * (dp[b][r] - t.z));
                    da2[4 * b + r] = (__bf16)(-lam * p2 * (dp[b][r] - t.w));
                }
            }
        };
        if (full)
            probs(std::false_type{});
        else
            probs(std::true_type{});
        // dV += W dD, dK_k += dS_k Q_k (k = the eight queries of lane group g)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bq1[c] = rd_qcol<D>(sq1, 16 * c, lane);
            bq2[c] = rd_qcol<D>(sq2, 16 * c, lane);
        }
#pragma unroll
        for (int c = 0; c < NCV; ++c) dvv[c] = mfma16(wa, bd[c], dvv[c]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            dk1[c] = mfma16(da1, bq1[c], dk1[c]);
            dk2[c] = mfma16(da2, bq2[c], dk2[c]);
        }
        // the other buffer was last read before the previous barrier
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // accumulator register r of block c: key kw0 + 4 g + r, channel 16 c + i
    const float tau = 1.f / sqrtf((float)D);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int kr = kw0 + 4 * g + r;
        if (kr >= a.Nk) continue;
        __bf16* o1 = (__bf16*)a.dk1 + ((size_t)bh * a.Nk + kr) * D;
        __bf16* o2 = (__bf16*)a.dk2 + ((size_t)bh * a.Nk + kr) * D;
        __bf16* ov = (__bf16*)a.dv + ((size_t)bh * a.Nk + kr) * DV;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            o1[16 * c + i16] = (__bf16)(tau * dk1[c][r]);
            o2[16 * c + i16] = (__bf16)(tau * dk2[c][r]);
        }
#pragma unroll
        for (int c = 0; c < NCV; ++c) ov[16 * c + i16] = (__bf16)dvv[c][r];
    }
}

// ---------------------------------------------------------------------------
// dlam: dlambda_h = -sum over batch and rows of delta_2 (fixed order)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads) void bwd_dlam_kernel(BackwardArgs a) {
    __shared__ float part[kBwdThreads / 64];
    const int h = blockIdx.x;
    const int64_t BH = (int64_t)a.B * a.H;
    // eight independent partial sums per thread (their loads in flight
    // together), added in a fixed order: the result does not depend on timing
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < a.B; ++b) {
        const float* d2 = a.delta + (BH + (int64_t)b * a.H + h) * a.Nq;
        int i = threadIdx.x;
        for (; i + 7 * kBwdThreads < a.Nq; i += 8 * kBwdThreads) {
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] += d2[i + u * kBwdThreads];
        }
        for (; i < a.Nq; i += kBwdThreads) acc[0] += d2[i];
    }
    float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int w = 0; w < kBwdThreads / 64; ++w) t += part[w];
        a.dlam[h] = -t;
    }
}

template <int D, int DV>
hipError_t launch_dims(const BackwardArgs& a, bool causal, hipStream_t stream) {
    BackwardArgs copy = a;
    void* args[] = {&copy};
    const int64_t rows = (int64_t)a.B * a.H * a.Nq;
    const int64_t BH = (int64_t)a.B * a.H;
    const int64_t g_prep = (rows + 4 * kPrepRows - 1) / (4 * kPrepRows);
    const int64_t g_dq = (int64_t)((a.Nq + 63) / 64) * BH;
    const int64_t g_kv = (int64_t)((a.Nk + 127) / 128) * BH;
    if (g_prep > 0x7fffffff || g_dq > 0x7fffffff || g_kv > 0x7fffffff) return hipErrorInvalidValue;
    hipError_t e = hipLaunchKernel((const void*)bwd_prep_kernel<DV>, dim3((unsigned)g_prep),
                                   dim3(kBwdThreads), args, 0, stream);
    if (e != hipSuccess) return e;
    e = hipLaunchKernel(causal ? (const void*)bwd_dq_kernel<D, DV, true>
                               : (const void*)bwd_dq_kernel<D, DV, false>,
                        dim3((unsigned)g_dq), dim3(kBwdThreads), args, 0, stream);
    if (e != hipSuccess) return e;
    if constexpr (D == 64 && DV == 128)
        e = hipLaunchKernel(causal ? (const void*)bwd_dkdv16_kernel<true>
                                   : (const void*)bwd_dkdv16_kernel<false>,
                            dim3((unsigned)g_kv), dim3(kKv16Threads), args, 0, stream);
    else
        e = hipLaunchKernel(causal ? (const void*)bwd_dkdv_kernel<D, DV, true>
                                   : (const void*)bwd_dkdv_kernel<D, DV, false>,
                            dim3((unsigned)g_kv), dim3(kBwdThreads), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel((const void*)bwd_dlam_kernel, dim3((unsigned)a.H), dim3(kBwdThreads),
                           args, 0, stream);
}

}  // namespace

size_t backward_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int dv) {
    const size_t dd = ((size_t)(B * H * Nq * dv * 2) + 255) / 256 * 256;
    const size_t delta = ((size_t)(2 * B * H * Nq) * sizeof(float) + 255) / 256 * 256;
    return dd + delta + (size_t)(B * H * Nq) * 4 * sizeof(float);
}

hipError_t launch_backward_bf16(const BackwardArgs& a, int d, int dv, bool causal,
                                hipStream_t stream) {
    if (d == 32 && dv == 64) return launch_dims<32, 64>(a, causal, stream);
    if (d == 64 && dv == 128) return launch_dims<64, 128>(a, causal, stream);
    if (d == 128 && dv == 256) {
        BackwardArgs copy = a;
        void* args[] = {&copy};
        const int64_t g_prep = ((int64_t)a.B * a.H * a.Nq + 4 * kPrepRows - 1) / (4 * kPrepRows);
        if (g_prep > 0x7fffffff) return hipErrorInvalidValue;
        hipError_t e = hipLaunchKernel((const void*)bwd_prep_kernel<256>, dim3((unsigned)g_prep),
                                       dim3(kBwdThreads), args, 0, stream);
        if (e != hipSuccess) return e;
        e = launch_backward_ring(a, causal, stream);
        if (e != hipSuccess) return e;
        return hipLaunchKernel((const void*)bwd_dlam_kernel, dim3((unsigned)a.H),
                               dim3(kBwdThreads), args, 0, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace diffattn
