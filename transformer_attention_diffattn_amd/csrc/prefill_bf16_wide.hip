// Fused Differential Attention prefill for bf16 inputs with head_dim 128 and
// v_dim 256 on gfx950 (CDNA4).
//
// Operator: the DiffAttn formula (iloveeagents.com, "Mathematical Formula")
// with the GroupNorm and (1 - lambda_init) scale of step 4 on llmbytes.dev
// ("How Differential Attention Cancels Common-Mode Noise"), fused into one
// memory pass ("Throughput and Hardware Realities").  This is the variant for
// the widest heads: the two O^T accumulators alone fill the 256 accumulation
// registers (AGPRs), the score tiles accumulate in VGPRs (inline-asm
// products, see mfma_v0), and the loop differs from the narrow-head kernel
// in prefill_core.h.
//
// Work decomposition
//   One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
//   wave owns 32 rows.  K1, K2 and V stream through a 3-stage LDS ring in tiles
//   of 32 keys; one wave per SIMD.  Iteration j of the key loop is
//   software-pipelined:
//     step 0  row maxima of tile j's scores, rare rescale (see below);
//     step 1  MFMA: scores of tile j+1        | VALU: probabilities of tile j
//     step 2  MFMA: P.V of tile j, both maps, each V operand read once
//                                             | LDS store of tile j+2, global
//                                               loads of tile j+3, masking
//   Tile j+1 must already be in LDS while tile j is consumed, hence 3 stages;
//   one barrier per tile.
//
// Per tile and wave, on MFMA v_mfma_f32_32x32x16_bf16:
//   S_k^T = K_k Q_k^T          (keys on the M axis, the wave's 32 queries on N),
//   O_k^T = alpha_k O_k^T + V^T P_k^T   for k = 1, 2,
// with the operand layouts, the swap23 key permutation that turns score
// accumulators directly into P^T B operands, the transposing V reads and the
// lazy running maximum all as described in prefill_core.h.  The O rescale
// multiplies the accumulators where they live, in AGPRs.
//
// LDS per stage: K1 and K2 row-major [32][d + 8], V row-major [32][dv + 32].
// Global loads go through buffer descriptors that end at the last key, so rows
// past the end read as zero without a branch; their scores are masked.

#include "internal.h"
#include "tile_ops.h"

#include <math.h>

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBc = 32;                 // keys per tile
constexpr float kRescaleLog2 = 30.0f;   // lazy-maximum slack, log2 units (see maybe_rescale)

template <int D, int DV>
struct Cfg {
    static constexpr int kBr = kWaves * 32;
    static constexpr int kStages = 3;
    static constexpr int kKStride = D + 8;
    static constexpr int kVStride = DV + 32;
    static constexpr int kKElems = kBc * kKStride;
    static constexpr int kVElems = kBc * kVStride;
    static constexpr int kStage = 2 * kKElems + kVElems;  // bf16 elements per stage
    static constexpr int kKChunks = kBc * D / 8;           // 16-byte chunks per K tile
    static constexpr int kVChunks = kBc * DV / 8;
    static constexpr int kKLoads = (kKChunks + kThreads - 1) / kThreads;
    static constexpr int kVLoads = (kVChunks + kThreads - 1) / kThreads;
};

__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// a*b - c*d with both products rounded before the subtraction (no fused
// multiply-add), so equal operands cancel to exactly zero
__device__ __forceinline__ float diff_of_products(float a, float b, float c, float d) {
#pragma clang fp contract(off)
    return a * b - c * d;
}

__device__ __forceinline__ float max16(const f32x16& s) {
    float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
    float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
    float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, s[15]));
}

// Score products with their accumulators in VGPRs (where the softmax reads
// them), while the compiler keeps the O accumulators of the P.V builtins in
// AGPRs.  As builtins they would accumulate in AGPRs too, and with O1 and O2
// filling all 256 of them the compiler moved an O block out and back every
// tile (~160 extra instructions per tile).  mfma_v0 starts a chain from zero
// (two wait states first, for a VALU write of its destination just before),
// mfma_v continues one.  The compiler does not see an asm product's latency:
// VALU accesses to the scores come after wait_s (below).
__device__ __forceinline__ f32x16 mfma_v0(bf16x8 a, bf16x8 b) {
    f32x16 d;
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ void mfma_v(f32x16& c, bf16x8 a, bf16x8 b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// 24 wait states (more than a 32x32x16 product needs) before a VALU access
// to asm products' results, in an asm that takes the results as operands: no
// product can be scheduled after it, no access before it
__device__ __forceinline__ void wait_s(f32x16& s1, f32x16& s2) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s1), "+v"(s2));
}

// Multiplies every accumulator of o by alpha in place.  The accumulators live
// in AGPRs; doing the read-multiply-write here keeps the compiler from holding
// a VGPR copy of all of them around this rarely taken path.
template <int NDB>
__device__ __forceinline__ void scale_acc(f32x16 (&o)[NDB], float alpha) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = o[db][r];
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha));
            o[db][r] = x;
        }
    }
}

// Moves the running maximum of one map when some row needs it (lazy rule):
// only when a score exceeds the running maximum by more than 2^kRescaleLog2
// in probability.  Probabilities up to 2^30 keep l and O far inside fp32
// (O <= 2^30 * keys * max|V|) and lose nothing in bf16, whose precision is
// relative; heavy-tailed scores, whose row maxima creep up tile after tile,
// then almost never pay for the rescale of the 256 accumulators.
template <int NDB>
__device__ __forceinline__ void maybe_rescale(float mx, float& m, float& l, f32x16 (&o)[NDB]) {
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleLog2)) {
        const float mrow = fmaxf(mx, xor32(mx));
        const float mnew = fmaxf(m, mrow);
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        l *= alpha;
        scale_acc<NDB>(o, alpha);
    }
}

// Probabilities of one map: p = 2^(s * scale - base), packed to bf16 B
// operands (registers 8kb .. 8kb+7 per 16 keys) and summed into l.  The sum
// is taken over the rounded values that enter P.V (a dot product of each
// packed pair with (1, 1)), so O / l stays an exact weighted mean of V.
__device__ __forceinline__ void probabilities(const f32x16& s, float sl2, float base, float& l,
                                              bf16x8 (&pb)[2]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float pa = __builtin_amdgcn_exp2f(fmaf(s[8 * kb + e], sl2, -base));
            const float pc = __builtin_amdgcn_exp2f(fmaf(s[8 * kb + e + 1], sl2, -base));
            const bf16x2 pr = {(__bf16)pa, (__bf16)pc};
            pb[kb][e] = pr[0];
            pb[kb][e + 1] = pr[1];
            if (e & 2)
                sum1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum1, false);
            else
                sum0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum0, false);
        }
    }
    l += sum0 + sum1;
}

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_bf16_wide_kernel(PrefillArgs a) {
    using C = Cfg<D, DV>;
    constexpr int NDB = DV / 32;
    constexpr int NKB = D / 16;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::kStages * C::kStage];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int lh = lane >> 5;

    // longest causal tiles first: the first B*H blocks take the last query tile
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + C::kBr - 1) / C::kBr;
    const int t = blockIdx.x / BH;
    const int bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? (nqt - 1 - t) : t;
    const int h = bh % a.H;

    const uint16_t* gq1 = (const uint16_t*)a.q1 + (size_t)bh * a.Nq * D;
    const uint16_t* gq2 = (const uint16_t*)a.q2 + (size_t)bh * a.Nq * D;
    const uint16_t* gk1 = (const uint16_t*)a.k1 + (size_t)bh * a.Nk * D;
    const uint16_t* gk2 = (const uint16_t*)a.k2 + (size_t)bh * a.Nk * D;
    const uint16_t* gv = (const uint16_t*)a.v + (size_t)bh * a.Nk * DV;
    __bf16* gout = (__bf16*)a.out + (size_t)bh * a.Nq * DV;

    const int wq0 = qt * C::kBr + wave * 32;  // first query row of this wave
    const int qrow = wq0 + l32;               // this lane's query row

    // Q fragments as B operands: column = query, k-slots = channels 16kb + 8lh ..
    bf16x8 qf1[NKB], qf2[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        if (qrow < a.Nq) {
            qf1[kb] = *(const bf16x8*)(gq1 + (size_t)qrow * D + 16 * kb + 8 * lh);
            qf2[kb] = *(const bf16x8*)(gq2 + (size_t)qrow * D + 16 * kb + 8 * lh);
        } else {
            qf1[kb] = bf16x8{};
            qf2[kb] = bf16x8{};
        }
    }

    const int nkt_all = (a.Nk + kBc - 1) / kBc;
    const int nkt = CAUSAL ? min(nkt_all, (qt * C::kBr + C::kBr + kBc - 1) / kBc) : nkt_all;

    u32x4 rk1[C::kKLoads], rk2[C::kKLoads], rv[C::kVLoads];

    // global -> registers through buffer loads: one descriptor per tensor and
    // tile (scalar work) starting at the tile's first key, per-lane byte
    // offsets fixed for the whole item; rows past the last key read as zero
    // (their scores are masked, so they contribute nothing)
    uint32_t k_voff[C::kKLoads], v_voff[C::kVLoads];
#pragma unroll
    for (int i = 0; i < C::kKLoads; ++i) {
        const int c = tid + i * kThreads;
        k_voff[i] = (uint32_t)(((c / (D / 8)) * D + (c % (D / 8)) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < C::kVLoads; ++i) {
        const int c = tid + i * kThreads;
        v_voff[i] = (uint32_t)(((c / (DV / 8)) * DV + (c % (DV / 8)) * 8) * 2);
    }
    auto load_tile = [&](int kt) {
        const int key0 = kt * kBc;
        const int64_t left = (int64_t)a.Nk - key0;  // <= 0 past the end: all zeros
        const __amdgpu_buffer_rsrc_t r1 = tile::buffer_rsrc(gk1 + (size_t)key0 * D, left * D * 2);
        const __amdgpu_buffer_rsrc_t r2 = tile::buffer_rsrc(gk2 + (size_t)key0 * D, left * D * 2);
        const __amdgpu_buffer_rsrc_t r3 = tile::buffer_rsrc(gv + (size_t)key0 * DV, left * DV * 2);
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
            rk1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, k_voff[i], 0, 0));
            rk2[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, k_voff[i], 0, 0));
        }
#pragma unroll
        for (int i = 0; i < C::kVLoads; ++i)
            rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r3, v_voff[i], 0, 0));
    };

    auto store_tile = [&](int buf) {
        uint16_t* k1s = smem + buf * C::kStage;
        uint16_t* k2s = k1s + C::kKElems;
        uint16_t* vs = k2s + C::kKElems;
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
            const int c = tid + i * kThreads;
            if (C::kKChunks % kThreads == 0 || c < C::kKChunks) {
                const int row = c / (D / 8), ch = c % (D / 8);
                *(u32x4*)(k1s + row * C::kKStride + ch * 8) = rk1[i];
                *(u32x4*)(k2s + row * C::kKStride + ch * 8) = rk2[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::kVLoads; ++i) {
            const int c = tid + i * kThreads;
            if (C::kVChunks % kThreads == 0 || c < C::kVChunks) {
                const int row = c / (DV / 8), ch = c % (DV / 8);
                *(u32x4*)(vs + row * C::kVStride + ch * 8) = rv[i];
            }
        }
    };

    const int krow = swap23(l32);
    auto scores = [&](int buf, f32x16& s1, f32x16& s2) {
        const uint16_t* k1s = smem + buf * C::kStage;
        const uint16_t* k2s = k1s + C::kKElems;
        // all K operand reads first: with one wave per SIMD nothing else would
        // hide the LDS latency of a read issued right before its product
        bf16x8 ka1[NKB], ka2[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            ka1[kb] = *(const bf16x8*)(k1s + krow * C::kKStride + 16 * kb + 8 * lh);
            ka2[kb] = *(const bf16x8*)(k2s + krow * C::kKStride + 16 * kb + 8 * lh);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if (kb == 0) {
                s1 = mfma_v0(ka1[kb], qf1[kb]);
                s2 = mfma_v0(ka2[kb], qf2[kb]);
            } else {
                mfma_v(s1, ka1[kb], qf1[kb]);
                mfma_v(s2, ka2[kb], qf2[kb]);
            }
        }
    };

    // keys past the end, and keys after the query under the causal mask, to -inf
    auto mask = [&](int kt, f32x16& s1, f32x16& s2) {
        const int key0 = kt * kBc;
        const bool need = (CAUSAL && key0 + kBc - 1 > wq0) || (key0 + kBc > a.Nk);
        if (need) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 16 * (r >> 3) + 8 * lh + (r & 7);
                const bool ok = key < a.Nk && (!CAUSAL || key <= qrow);
                s1[r] = ok ? s1[r] : -INFINITY;
                s2[r] = ok ? s2[r] : -INFINITY;
            }
        }
    };

    // per-lane pieces of the transposing V read: key e of 4, channel offset 4r
    const int vg = lane >> 4;
    const int v_lane_off = (8 * (vg >> 1) + ((lane & 15) >> 2)) * C::kVStride +
                           16 * (vg & 1) + 4 * (lane & 3);
    auto v_operand = [&](int buf, int db, int kb) {
        const uint16_t* vp = smem + buf * C::kStage + 2 * C::kKElems + v_lane_off +
                             16 * kb * C::kVStride + 32 * db;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)vp);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(vp + 4 * C::kVStride));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    const float sl2 = a.scale_log2;
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    f32x16 o1[NDB], o2[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        o1[db] = f32x16{};
        o2[db] = f32x16{};
    }

    // prologue: tiles 0 and 1 into LDS, tile 2 into registers, scores of tile 0
    load_tile(0);
    store_tile(0);
    load_tile(1);
    store_tile(1);
    __syncthreads();
    load_tile(2);
    // n1, n2: score accumulators of the next tile; s1, s2: tile j's scores
    f32x16 n1, n2, s1, s2;
    scores(0, s1, s2);
    wait_s(s1, s2);
    mask(0, s1, s2);

    int bj = 0;  // stage of tile j; tile j+1 is in (bj+1)%3, tile j+2 goes to (bj+2)%3
    for (int j = 0; j < nkt; ++j) {
        const int bn = bj == 2 ? 0 : bj + 1;
        const int bw = bn == 2 ? 0 : bn + 1;

        // step 0: row maxima of tile j and the rare rescale
        maybe_rescale<NDB>(max16(s1) * sl2, m1, l1, o1);
        maybe_rescale<NDB>(max16(s2) * sl2, m2, l2, o2);
        const float base1 = m1 == -INFINITY ? 0.f : m1;
        const float base2 = m2 == -INFINITY ? 0.f : m2;

        // step 1: scores of tile j+1 on MFMA while the VALU turns tile j into P
        scores(bn, n1, n2);
        bf16x8 p1[2], p2[2];
        probabilities(s1, sl2, base1, l1, p1);
        probabilities(s2, sl2, base2, l2, p2);
        // step 2: P.V for both maps, each V operand read once; the reads in
        // groups of four operands, each group issued before the previous
        // group's products
        constexpr int kGrp = 4;
        bf16x8 vcur[kGrp], vnxt[kGrp];
#pragma unroll
        for (int u = 0; u < kGrp; ++u) vnxt[u] = v_operand(bj, u >> 1, u & 1);
#pragma unroll
        for (int g0 = 0; g0 < 2 * NDB; g0 += kGrp) {
#pragma unroll
            for (int u = 0; u < kGrp; ++u) vcur[u] = vnxt[u];
            if (g0 + kGrp < 2 * NDB) {
#pragma unroll
                for (int u = 0; u < kGrp; ++u)
                    vnxt[u] = v_operand(bj, (g0 + kGrp + u) >> 1, (g0 + kGrp + u) & 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kGrp; ++u) {
                const int db = (g0 + u) >> 1, kb = (g0 + u) & 1;
                o1[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[u], p1[kb], o1[db], 0, 0, 0);
                o2[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[u], p2[kb], o2[db], 0, 0, 0);
            }
        }

        store_tile(bw);      // tile j+2 (stale and unused once past the end)
        load_tile(j + 3);    // clamped rows once past the end
        wait_s(n1, n2);  // before the masking and the copies read them
        mask(j + 1, n1, n2);
        __syncthreads();
        s1 = n1;
        s2 = n2;
        bj = bn;
    }

    // epilogue: D = O1/l1 - lambda O2/l2, then GroupNorm over the dv channels
    const float lam = a.lam[h];
    const float L1 = l1 + xor32(l1);
    const float L2 = l2 + xor32(l2);
    const float c1 = 1.f / L1;
    const float c2 = lam / L2;
    float dsum = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float dval = diff_of_products(o1[db][r], c1, o2[db][r], c2);
            o1[db][r] = dval;
            dsum += dval;
        }
    }
    if (!(a.flags & 1u)) {
        dsum += xor32(dsum);
        const float mean = dsum * (1.f / DV);
        float vsum = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float c = o1[db][r] - mean;
                vsum = fmaf(c, c, vsum);
            }
        }
        vsum += xor32(vsum);
        const float var = vsum * (1.f / DV);
        const float scale = (1.f - a.lambda_init) / sqrtf(var + a.eps);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o1[db][r] = (o1[db][r] - mean) * scale;
        }
    }

    if (qrow < a.Nq) {
        __bf16* orow = gout + (size_t)qrow * DV;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)o1[db][4 * g + e];
                *(bf16x4*)(orow + 32 * db + 8 * g + 4 * lh) = w;
            }
        }
    }
}

template <int D, int DV>
hipError_t launch_dims(const PrefillArgs& a, bool causal, hipStream_t stream) {
    const int nqt = (a.Nq + Cfg<D, DV>::kBr - 1) / Cfg<D, DV>::kBr;
    const dim3 grid((unsigned)((int64_t)nqt * a.B * a.H));
    PrefillArgs copy = a;
    void* args[] = {&copy};
    const void* fn = causal ? (const void*)prefill_bf16_wide_kernel<D, DV, true>
                            : (const void*)prefill_bf16_wide_kernel<D, DV, false>;
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill_bf16_wide(const PrefillArgs& a, int d, int dv, bool causal,
                                    hipStream_t stream) {
    if (d == 128 && dv == 256) return launch_dims<128, 256>(a, causal, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
