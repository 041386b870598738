// Fused Differential Attention prefill for bf16 inputs on gfx950 (CDNA4).
//
// Operator: the DiffAttn formula (iloveeagents.com, "Mathematical Formula")
// with the GroupNorm and (1 - lambda_init) scale of step 4 on llmbytes.dev
// ("How Differential Attention Cancels Common-Mode Noise").  The pages note
// that a custom kernel can fuse the two softmax maps and the subtraction into
// one memory pass ("Throughput and Hardware Realities"); this is that kernel.
//
// Work decomposition
//   One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
//   wave owns 32 rows.  K1, K2 and V stream through LDS in tiles of 64 keys,
//   double-buffered: the next tile's global loads are issued into registers
//   before the current tile's math and written to the other LDS buffer after
//   it, so one barrier per tile suffices.
//
// Per tile and wave, on MFMA v_mfma_f32_32x32x16_bf16:
//   S_k^T = K_k Q_k^T          (keys on the M axis, the wave's queries on N),
//   O_k^T = alpha_k O_k^T + V^T P_k^T   for k = 1, 2.
//   Computing the transposed score tile puts every query in one lane pair
//   (lanes l and l+32), so the row max and row sum of the online softmax are
//   in-lane reductions plus one exchange, and the alpha rescale of O^T is a
//   per-lane scalar.  The two maps keep separate (max, sum, O) states; the
//   lambda-weighted subtraction happens once, in the epilogue, followed by the
//   per-head GroupNorm over the dv channels and the (1 - lambda_init) scale.
//
// Operand layouts (32x32x16 MFMA; lane l, lh = l / 32, l32 = l % 32):
//   A operand: row l32, k-slots 8*lh .. 8*lh+7;  B operand: column l32, the same
//   k-slots; accumulator register r: row 8*(r/4) + 4*lh + r%4, column l32.
//   The k-slot order is the same for A and B, so any consistent assignment of
//   keys (or channels) to k-slots gives the right contraction.
//   The score tile's A operand loads key row swap23(l32) (bits 2 and 3 of the
//   row index exchanged), which makes accumulator register r of lane l hold
//   key 16*(r/8) + 8*lh + r%8 of the 32-key block.  Registers 8c .. 8c+7 of the
//   score accumulator then form, after conversion to bf16, exactly the B
//   operand P^T for keys 16c + 8*lh .. +7, matching an A operand that reads 8
//   consecutive keys of a V^T row: the probabilities never leave registers.
//
// LDS per stage: K1 and K2 row-major [64][d + 8] (the pad keeps 16-byte row
// reads conflict-free), V transposed [dv][64] with its 16-byte chunks XOR-
// swizzled by (row + row/8) & 7 so both the transposing 8-byte writes and the
// 16-byte operand reads spread over the banks.

#include "internal.h"

#include <math.h>

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBr = 128;  // query rows per workgroup
constexpr int kBc = 64;   // keys per tile

template <int D, int DV>
struct Layout {
    static constexpr int kKStride = D + 8;  // elements per K row in LDS
    static constexpr int kKElems = kBc * kKStride;
    static constexpr int kVtElems = DV * kBc;
    static constexpr int kStage = 2 * kKElems + kVtElems;  // bf16 elements per stage
    static constexpr int kKChunks = D / 8;                   // 16-byte chunks per K row
    static constexpr int kKLoads = kBc * kKChunks / kThreads;
    static constexpr int kVGroups = (kBc / 4) * (DV / 8);   // 4 keys x 8 channels each
    static constexpr int kVLoads = (kVGroups + kThreads - 1) / kThreads;
    static_assert(kBc * kKChunks % kThreads == 0, "K tile must split evenly");
};

__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ int vt_swizzle(int row) { return (row + (row >> 3)) & 7; }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// a*b - c*d with both products rounded before the subtraction (no fused
// multiply-add), so equal operands cancel to exactly zero
__device__ __forceinline__ float diff_of_products(float a, float b, float c, float d) {
#pragma clang fp contract(off)
    return a * b - c * d;
}

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
    using LY = Layout<D, DV>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * LY::kStage];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int lh = lane >> 5;

    // longest causal tiles first: the first B*H blocks take the last query tile
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + kBr - 1) / kBr;
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

    const int qrow0 = qt * kBr + wave * 32;  // first query row of this wave
    const int qrow = qrow0 + l32;            // this lane's query row

    // Q fragments as B operands: column = query, k-slots = channels 16kb + 8lh ..
    bf16x8 qf1[D / 16], qf2[D / 16];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
        if (qrow < a.Nq) {
            qf1[kb] = *(const bf16x8*)(gq1 + (size_t)qrow * D + 16 * kb + 8 * lh);
            qf2[kb] = *(const bf16x8*)(gq2 + (size_t)qrow * D + 16 * kb + 8 * lh);
        } else {
            qf1[kb] = bf16x8{};
            qf2[kb] = bf16x8{};
        }
    }

    const int nkt_all = (a.Nk + kBc - 1) / kBc;
    const int nkt = CAUSAL ? min(nkt_all, (qt * kBr + kBr + kBc - 1) / kBc) : nkt_all;

    u32x4 rk1[LY::kKLoads], rk2[LY::kKLoads], rv[LY::kVLoads][4];

    auto load_tile = [&](int kt) {
        const int key0 = kt * kBc;
#pragma unroll
        for (int i = 0; i < LY::kKLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / LY::kKChunks, ch = c % LY::kKChunks;
            const int key = key0 + row;
            if (key < a.Nk) {
                rk1[i] = *(const u32x4*)(gk1 + (size_t)key * D + ch * 8);
                rk2[i] = *(const u32x4*)(gk2 + (size_t)key * D + ch * 8);
            } else {
                rk1[i] = u32x4{0, 0, 0, 0};
                rk2[i] = u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < LY::kVLoads; ++i) {
            const int g = tid + i * kThreads;
            if (g < LY::kVGroups) {
                const int rg = g / (DV / 8), cc = g % (DV / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key0 + 4 * rg + r;
                    rv[i][r] = key < a.Nk ? *(const u32x4*)(gv + (size_t)key * DV + cc * 8)
                                          : u32x4{0, 0, 0, 0};
                }
            }
        }
    };

    auto store_tile = [&](int buf) {
        uint16_t* k1s = smem + buf * LY::kStage;
        uint16_t* k2s = k1s + LY::kKElems;
        uint16_t* vts = k2s + LY::kKElems;
#pragma unroll
        for (int i = 0; i < LY::kKLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / LY::kKChunks, ch = c % LY::kKChunks;
            *(u32x4*)(k1s + row * LY::kKStride + ch * 8) = rk1[i];
            *(u32x4*)(k2s + row * LY::kKStride + ch * 8) = rk2[i];
        }
#pragma unroll
        for (int i = 0; i < LY::kVLoads; ++i) {
            const int g = tid + i * kThreads;
            if (g < LY::kVGroups) {
                const int rg = g / (DV / 8), cc = g % (DV / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = 8 * cc + e;
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    // channel `col` of keys 4rg .. 4rg+3, two keys per dword
                    const uint32_t lo = __builtin_amdgcn_perm(rv[i][1][e >> 1], rv[i][0][e >> 1], sel);
                    const uint32_t hi = __builtin_amdgcn_perm(rv[i][3][e >> 1], rv[i][2][e >> 1], sel);
                    const int off = col * kBc + (((rg >> 1) ^ vt_swizzle(col)) << 3) + ((rg & 1) << 2);
                    *(u32x2*)(vts + off) = u32x2{lo, hi};
                }
            }
        }
    };

    const float NEG_INF = -INFINITY;
    const float sl2 = a.scale_log2;
    float m1 = NEG_INF, m2 = NEG_INF;  // running max of scaled log2 scores
    float l1 = 0.f, l2 = 0.f;          // running sums, this lane's half of the keys
    f32x16 o1[DV / 32], o2[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) {
        o1[db] = f32x16{};
        o2[db] = f32x16{};
    }

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool has_next = kt + 1 < nkt;
        if (has_next) load_tile(kt + 1);

        const int key0 = kt * kBc;
        // a wave whose rows all precede the tile's first key has nothing to do
        const bool active = !CAUSAL || key0 <= qrow0 + 31;
        if (active) {
            const uint16_t* k1s = smem + buf * LY::kStage;
            const uint16_t* k2s = k1s + LY::kKElems;
            const uint16_t* vts = k2s + LY::kKElems;

            f32x16 s1[2], s2[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                s1[sb] = f32x16{};
                s2[sb] = f32x16{};
                const int krow = 32 * sb + swap23(l32);
#pragma unroll
                for (int kb = 0; kb < D / 16; ++kb) {
                    const bf16x8 ka1 = *(const bf16x8*)(k1s + krow * LY::kKStride + 16 * kb + 8 * lh);
                    const bf16x8 ka2 = *(const bf16x8*)(k2s + krow * LY::kKStride + 16 * kb + 8 * lh);
                    s1[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qf1[kb], s1[sb], 0, 0, 0);
                    s2[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka2, qf2[kb], s2[sb], 0, 0, 0);
                }
            }

            // mask keys past the end, and keys after the query under the causal mask
            const bool need_mask = (CAUSAL && key0 + kBc - 1 > qrow0) || (key0 + kBc > a.Nk);
            if (need_mask) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + 32 * sb + 16 * (r >> 3) + 8 * lh + (r & 7);
                        const bool ok = key < a.Nk && (!CAUSAL || key <= qrow);
                        if (!ok) {
                            s1[sb][r] = NEG_INF;
                            s2[sb][r] = NEG_INF;
                        }
                    }
                }
            }

            float mx1 = NEG_INF, mx2 = NEG_INF;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    mx1 = fmaxf(mx1, s1[sb][r]);
                    mx2 = fmaxf(mx2, s2[sb][r]);
                }
            }
            mx1 = fmaxf(mx1, xor32(mx1));
            mx2 = fmaxf(mx2, xor32(mx2));

            const float mn1 = fmaxf(m1, mx1 * sl2);
            const float mn2 = fmaxf(m2, mx2 * sl2);
            const float base1 = mn1 == NEG_INF ? 0.f : mn1;
            const float base2 = mn2 == NEG_INF ? 0.f : mn2;
            const float al1 = __builtin_amdgcn_exp2f(m1 - base1);
            const float al2 = __builtin_amdgcn_exp2f(m2 - base2);
            m1 = mn1;
            m2 = mn2;

            float rs1 = 0.f, rs2 = 0.f;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s1[sb][r], sl2, -base1));
                    const float p2 = __builtin_amdgcn_exp2f(fmaf(s2[sb][r], sl2, -base2));
                    s1[sb][r] = p1;
                    s2[sb][r] = p2;
                    rs1 += p1;
                    rs2 += p2;
                }
            }
            l1 = fmaf(l1, al1, rs1);
            l2 = fmaf(l2, al2, rs2);

#pragma unroll
            for (int db = 0; db < DV / 32; ++db) {
                o1[db] *= al1;
                o2[db] *= al2;
            }

#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bf16x8 p1b, p2b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p1b[e] = (__bf16)s1[kb >> 1][8 * (kb & 1) + e];
                    p2b[e] = (__bf16)s2[kb >> 1][8 * (kb & 1) + e];
                }
#pragma unroll
                for (int db = 0; db < DV / 32; ++db) {
                    const int vrow = 32 * db + l32;
                    const bf16x8 va = *(const bf16x8*)(vts + vrow * kBc +
                                                       (((2 * kb + lh) ^ vt_swizzle(vrow)) << 3));
                    o1[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1b, o1[db], 0, 0, 0);
                    o2[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p2b, o2[db], 0, 0, 0);
                }
            }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue: D = O1/l1 - lambda O2/l2, then GroupNorm over the dv channels
    l1 += xor32(l1);
    l2 += xor32(l2);
    const float lam = a.lam[h];
    const float c1 = 1.f / l1;
    const float c2 = lam / l2;
    float dsum = 0.f;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) {
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
        for (int db = 0; db < DV / 32; ++db) {
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
        for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o1[db][r] = (o1[db][r] - mean) * scale;
        }
    }

    if (qrow < a.Nq) {
        __bf16* orow = gout + (size_t)qrow * DV;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
    const int nqt = (a.Nq + kBr - 1) / kBr;
    const dim3 grid((unsigned)((int64_t)nqt * a.B * a.H));
    PrefillArgs copy = a;
    void* args[] = {&copy};
    const void* fn = causal ? (const void*)prefill_bf16_kernel<D, DV, true>
                            : (const void*)prefill_bf16_kernel<D, DV, false>;
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, int dv, bool causal,
                               hipStream_t stream) {
    if (d == 32 && dv == 64) return launch_dims<32, 64>(a, causal, stream);
    if (d == 64 && dv == 128) return launch_dims<64, 128>(a, causal, stream);
    if (d == 128 && dv == 256) return launch_dims<128, 256>(a, causal, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
