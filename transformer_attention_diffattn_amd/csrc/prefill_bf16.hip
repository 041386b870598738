// Fused Differential Attention prefill for bf16 inputs on gfx950 (CDNA4),
// head_dim 32 or 64 (head_dim 128 is in prefill_bf16_wide.hip).
//
// Operator: the DiffAttn formula (iloveeagents.com, "Mathematical Formula")
// with the GroupNorm and (1 - lambda_init) scale of step 4 on llmbytes.dev
// ("How Differential Attention Cancels Common-Mode Noise").  The pages note
// that a custom kernel can fuse the two softmax maps and the subtraction into
// one memory pass ("Throughput and Hardware Realities"); this is that kernel.
//
// Work decomposition
//   One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
//   wave owns 32 rows.  K1, K2 and V stream through a 4-stage LDS ring in tiles
//   of 32 keys.  The kernel needs more than 256 registers per lane, so there is
//   one wave per SIMD and the overlap of matrix and vector work has to come
//   from inside the wave.  At d = 64 the vector work of the two softmaxes
//   (exp2, scale, sums, bf16 packing) costs about as many cycles as the six
//   matrix products of a tile, so the loop is arranged to keep both pipes busy:
//   iteration j issues, in one branch-free block,
//     MFMA  scores of tile j+1 (both maps), P.V of tile j-1 (both maps);
//     VALU  probabilities of tile j (both maps), row sums;
//     memory  global loads of tile j+3, LDS stores of tile j+2;
//   and ends with the masking of tile j+1 (tiles on the causal diagonal and
//   the ragged last tile only) and the lazy-maximum test of tile j (below),
//   whose body almost never runs.  Tile j-1's V is read in
//   iteration j and tile j+1's K too, hence 4 stages; one barrier per tile.
//
// Per tile and wave, on MFMA v_mfma_f32_32x32x16_bf16:
//   S_k^T = K_k Q_k^T          (keys on the M axis, the wave's 32 queries on N),
//   O_k^T = alpha_k O_k^T + V^T P_k^T   for k = 1, 2.
//   With the transposed score tile every query lives in one lane pair (lanes
//   l and l+32), so online-softmax row statistics are in-lane reductions plus
//   one exchange, and the rescale of O^T is a per-lane scalar.  The two maps
//   keep separate (max, sum, O) states; the lambda-weighted subtraction happens
//   once, in the epilogue, followed by the per-head GroupNorm over the dv
//   channels and the (1 - lambda_init) scale.
//
// Online softmax with a lazy maximum: the running maximum m of a row is set
// exactly from the first tile and afterwards moves only when needed.  Each
// tile's probabilities are formed against the current, possibly stale, m and
// may then exceed 1; the sum l and O share that m, so O / l is unchanged.  A
// lane whose partial sum over the tile (16 of the row's 32 keys) exceeds
// kSumLimit flags the tile: its exact row maxima are taken, O and l are
// rescaled, and its probabilities are formed again.  So no probability
// exceeds kSumLimit, and the O rescale (the only VALU work proportional to dv)
// and the row maxima (two 16-element reductions per tile) run only when some
// row's scores climb well past their running maximum, which after the first
// tile is rare.  The test reuses the row sums the softmax needs anyway.
//
// Operand layouts (32x32x16 MFMA; lane l, lh = l / 32, l32 = l % 32):
//   A operand: row l32, k-slots 8*lh .. 8*lh+7;  B operand: column l32, the same
//   k-slots; accumulator register r: row 8*(r/4) + 4*lh + r%4, column l32.
//   The k-slot order is the same for A and B, so any consistent assignment of
//   keys (or channels) to k-slots gives the right contraction.
//   The score tile's A operand loads key row swap23(l32) (bits 2 and 3 of the
//   row index exchanged), which makes accumulator register r of lane l hold
//   key 16*(r/8) + 8*lh + r%8 of the tile.  Registers 8c .. 8c+7, converted to
//   bf16, are then exactly the B operand P^T for keys 16c + 8*lh .. +7: the
//   probabilities never leave registers.
//   The P.V A operand (V^T: channel rows, key k-slots) comes from a row-major
//   V tile through ds_read_b64_tr_b16, the gfx950 transposing LDS read: within
//   each 16-lane group, lane i receives element i%4 of the 8-byte pieces that
//   lanes 4e + i/4 (e = 0..3) address.  Lane j = 4e + r of a group addresses
//   key e (of 4 consecutive keys) at channel base + 4r, so lane i gets channel
//   base + i of those 4 keys; two such reads give the 8 keys of a k-slot half.
//
// LDS per stage: K1 and K2 row-major [32][d + 8] (the pad keeps the 16-byte
// operand reads conflict-free), V row-major [32][dv + 32] (a 64-byte pad puts
// the 4 rows a half-wave of transposing reads touches in distinct banks).
// Global loads are raw buffer loads whose descriptor ends at the last key of
// the (batch, head): rows past the end read as zeros without a branch or a
// clamp, and their scores are masked, so they contribute nothing.

#include "internal.h"

#include <math.h>

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBc = 32;                 // keys per tile
constexpr float kSumLimit = 4096.0f;    // lazy-maximum bound on a lane's partial tile sum
constexpr int kBufferDword3 = 0x00020000;  // raw buffer descriptor word 3 for gfx9 parts

template <int D, int DV>
struct Cfg {
    static constexpr int kBr = kWaves * 32;
    static constexpr int kStages = 4;
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

// Descriptor of `bytes` bytes from `base`; loads at offsets past the end
// return zeros.  The record count is a 32-bit field, so it is clamped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, kBufferDword3);
}

// acc += a * b on MFMA with the accumulator held in AGPRs.  Written as inline
// asm so that this product, alone in the kernel, keeps the AGPR form while
// the score products (compiler builtins) accumulate in ordinary VGPRs, where
// the softmax reads them.  The compiler does not see this instruction as an
// MFMA, so the wait states it would insert are provided by hand: two before
// the product (a VALU write of an operand register needs them), and
// mfma_drain before any other instruction touches the accumulators.  Inputs
// a and b come from LDS reads (ordered by the compiler's s_waitcnt) and from
// VALU results of the previous tile.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states that let the last mfma_agpr products retire before the
// accumulators are read or written by other instructions.
template <int NDB>
__device__ __forceinline__ void mfma_drain(f32x16 (&o1)[NDB], f32x16 (&o2)[NDB]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o1[db]), "+a"(o2[db]));
}

// Multiplies every accumulator of o by alpha where it lives, in AGPRs, one
// register at a time (a plain multiply would stage all of them in VGPRs).
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

// The bf16 probabilities p[e], p[e+1] of a tile packed into pb, added to a
// row partial sum with one dot product against (1, 1): the sum is taken over
// the same rounded values that enter P.V.
__device__ __forceinline__ void pack_pair(bf16x8 (&pb)[2], int e, float pa, float pc, float& sum) {
    const bf16x2 pr = {(__bf16)pa, (__bf16)pc};
    u32x4 w = __builtin_bit_cast(u32x4, pb[e >> 3]);
    w[(e & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
    pb[e >> 3] = __builtin_bit_cast(bf16x8, w);
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
}

// Probabilities p = 2^(s * scale - base) of accumulator registers e, e+1 of a
// score tile, packed and summed (see pack_pair).
__device__ __forceinline__ void prob_pair(const f32x16& s, int e, float sl2, float base,
                                          bf16x8 (&pb)[2], float& sum) {
    const float pa = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -base));
    const float pc = __builtin_amdgcn_exp2f(fmaf(s[e + 1], sl2, -base));
    pack_pair(pb, e, pa, pc, sum);
}

template <bool B>
using bool_c = std::integral_constant<bool, B>;

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
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
    // leading tiles in which no row of this wave masks a key
    const int nfull = CAUSAL ? min(a.Nk / kBc, (wq0 + 1) / kBc) : a.Nk / kBc;

    u32x4 rk1[C::kKLoads], rk2[C::kKLoads], rv[C::kVLoads];

    // global -> registers through descriptors that start at the tile
    auto load_tile = [&](int kt) {
        const int64_t key0 = (int64_t)kt * kBc;
        const int64_t left = (int64_t)a.Nk - key0;
        const __amdgpu_buffer_rsrc_t r1 = buffer_rsrc(gk1 + key0 * D, left * D * 2);
        const __amdgpu_buffer_rsrc_t r2 = buffer_rsrc(gk2 + key0 * D, left * D * 2);
        const __amdgpu_buffer_rsrc_t rvv = buffer_rsrc(gv + key0 * DV, left * DV * 2);
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
            const int off = 16 * (tid + i * kThreads);  // key c / (D/8), channel chunk c % (D/8)
            rk1[i] = __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, 0);
            rk2[i] = __builtin_amdgcn_raw_buffer_load_b128(r2, off, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::kVLoads; ++i) {
            const int off = 16 * (tid + i * kThreads);
            rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rvv, off, 0, 0);
        }
    };

    auto stage_of = [](int kt) { return kt & (C::kStages - 1); };

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
        s1 = f32x16{};
        s2 = f32x16{};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const bf16x8 ka1 = *(const bf16x8*)(k1s + krow * C::kKStride + 16 * kb + 8 * lh);
            const bf16x8 ka2 = *(const bf16x8*)(k2s + krow * C::kKStride + 16 * kb + 8 * lh);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qf1[kb], s1, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka2, qf2[kb], s2, 0, 0, 0);
        }
    };

    // keys past the end, and keys after the query under the causal mask, to -inf
    auto mask = [&](int kt, f32x16& s1, f32x16& s2) {
        const int key0 = kt * kBc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = key0 + 16 * (r >> 3) + 8 * lh + (r & 7);
            const bool ok = key < a.Nk && (!CAUSAL || key <= qrow);
            s1[r] = ok ? s1[r] : -INFINITY;
            s2[r] = ok ? s2[r] : -INFINITY;
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
    float m1, m2, l1 = 0.f, l2 = 0.f;
    f32x16 o1[NDB], o2[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        o1[db] = f32x16{};
        o2[db] = f32x16{};
    }

    // P.V of one tile for both maps (the last tile; inside the loop the same
    // products are spread over the issue slots)
    auto pv = [&](int buf, const bf16x8 (&p1)[2], const bf16x8 (&p2)[2]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 va = v_operand(buf, db, kb);
                mfma_agpr(o1[db], va, p1[kb]);
                mfma_agpr(o2[db], va, p2[kb]);
            }
        }
    };

    // Per-tile state, two copies used alternately (tile j in X[j % 2]): the
    // masked scores of the tile and, once formed, its probabilities.  In
    // iteration j the other copy still holds tile j-1's probabilities (read by
    // its P.V) and receives tile j+1's scores, so nothing is copied between
    // iterations and the new probabilities never have to wait for the
    // previous tile's products to be issued.
    struct TileState {
        f32x16 s1, s2;
        bf16x8 p1[2], p2[2];
    };
    TileState A, B;

    // prologue: tiles 0 and 1 into LDS, tile 2 into registers, scores of tile 0
    load_tile(0);
    store_tile(0);
    load_tile(1);
    store_tile(1);
    __syncthreads();
    load_tile(2);
    scores(0, A.s1, A.s2);
    if (nfull < 1) mask(0, A.s1, A.s2);
    {
        // exact row maxima of tile 0 start the running maxima
        const float x1 = max16(A.s1) * sl2, x2 = max16(A.s2) * sl2;
        m1 = fmaxf(x1, xor32(x1));
        m2 = fmaxf(x2, xor32(x2));
    }

    // Issue plan of one iteration.  The body is a fixed sequence of kSlots
    // slots, each holding one MFMA and a planned share of the vector work,
    // fenced by scheduling barriers, so that the compiler cannot bunch the
    // matrix products together and leave the softmax to run after them (it
    // otherwise does, and both pipes then idle half of the time):
    //   slots 0 .. kScore-1     score products of tile j+1, each K operand
    //                           read kKAhead products ahead;
    //   slots kScore ..         P.V products of tile j-1, each V operand read
    //                           kLookahead operand pairs ahead;
    //   vector work             the 16 probability pairs of tile j spread
    //                           over the slots (starting in a slot -1 that
    //                           has no product and covers the first K read),
    //                           the LDS store of tile j+2 and the global loads
    //                           of tile j+3 early.
    constexpr int kScore = 2 * NKB;
    constexpr int kPairsV = 2 * NDB;           // V operands (db, kb)
    constexpr int kSlots = kScore + 2 * kPairsV;
    constexpr int kLookahead = 3;              // V operands read ahead
    constexpr int kKAhead = 4;                 // K operands read ahead
    constexpr int kStoreSlot = 1, kLoadSlot = 2;
    // probability pair k (map k / 8, registers 2 (k % 8) and +1) starts in slot
    auto pair_slot = [](int k) { return k * (kSlots - 3) / 16 - 1; };
    static_assert(15 * (kSlots - 3) / 16 - 1 + 2 < kSlots, "pairs must finish in the slots");

    // One iteration j (see the header); cur holds tile j, oth tile j-1 and
    // then j+1.  PREV: tile j-1 exists; NEXT: tile j+1 exists.
    auto iteration = [&](auto prev, auto next, int j, TileState& cur, TileState& oth) {
        constexpr bool PREV = decltype(prev)::value;
        constexpr bool NEXT = decltype(next)::value;
        const float base1 = m1 == -INFINITY ? 0.f : m1;
        const float base2 = m2 == -INFINITY ? 0.f : m2;

        bf16x8 ka[kScore], va[kPairsV];
        const uint16_t* k1s = smem + stage_of(j + 1) * C::kStage + krow * C::kKStride + 8 * lh;
        // K operand i: map i % 2, channels 16 (i / 2) + 8 lh ..
        auto read_k = [&](int i) {
            ka[i] = *(const bf16x8*)(k1s + (i & 1) * C::kKElems + 16 * (i >> 1));
        };
        if constexpr (NEXT) {
#pragma unroll
            for (int i = 0; i < kKAhead; ++i) read_k(i);
        }
        const int vbuf = stage_of(j - 1);
        if constexpr (PREV) {
#pragma unroll
            for (int q = 0; q < kLookahead; ++q) va[q] = v_operand(vbuf, q >> 1, q & 1);
        }
        float t1a = 0.f, t1b = 0.f, t2a = 0.f, t2b = 0.f;
        float xs[32];  // probabilities in flight, element 16 map + register
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int slot = -1; slot < kSlots; ++slot) {
            if (slot < 0) {
                // no product: the first K operands are still on their way
            } else if (slot < kScore) {
                if constexpr (NEXT) {
                    const int kb = slot >> 1;
                    if (slot + kKAhead < kScore) read_k(slot + kKAhead);
                    if ((slot & 1) == 0)
                        oth.s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            ka[slot], qf1[kb], kb == 0 ? f32x16{} : oth.s1, 0, 0, 0);
                    else
                        oth.s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            ka[slot], qf2[kb], kb == 0 ? f32x16{} : oth.s2, 0, 0, 0);
                }
            } else {
                if constexpr (PREV) {
                    const int i = slot - kScore, q = i >> 1;
                    if ((i & 1) == 0) {
                        if (q + kLookahead < kPairsV)
                            va[q + kLookahead] = v_operand(vbuf, (q + kLookahead) >> 1, (q + kLookahead) & 1);
                        mfma_agpr(o1[q >> 1], va[q], oth.p1[q & 1]);
                    } else {
                        mfma_agpr(o2[q >> 1], va[q], oth.p2[q & 1]);
                    }
                }
            }
            // probability pair k: scale at pair_slot(k), exp2 one slot later,
            // sums and bf16 packing one slot after that, so that the work of
            // a slot is independent and no chain latency stalls the wave
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int e = 2 * (k & 7);
                const f32x16& sk = k < 8 ? cur.s1 : cur.s2;
                const float bk = k < 8 ? base1 : base2;
                if (pair_slot(k) == slot) {
                    xs[2 * k] = fmaf(sk[e], sl2, -bk);
                    xs[2 * k + 1] = fmaf(sk[e + 1], sl2, -bk);
                }
                if (pair_slot(k) + 1 == slot) {
                    xs[2 * k] = __builtin_amdgcn_exp2f(xs[2 * k]);
                    xs[2 * k + 1] = __builtin_amdgcn_exp2f(xs[2 * k + 1]);
                }
                if (pair_slot(k) + 2 == slot) {
                    if (k < 8)
                        pack_pair(cur.p1, e, xs[2 * k], xs[2 * k + 1], (k & 1) ? t1b : t1a);
                    else
                        pack_pair(cur.p2, e, xs[2 * k], xs[2 * k + 1], (k & 1) ? t2b : t2a);
                }
            }
            if (slot == kStoreSlot) store_tile(stage_of(j + 2));  // zeros once past the end
            if (slot == kLoadSlot) load_tile(j + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Keep the common-path probabilities ahead of the rare branch below
        // (which forms them again) rather than sunk into its other side.
        asm volatile("" ::"v"(cur.p1[0]), "v"(cur.p1[1]), "v"(cur.p2[0]), "v"(cur.p2[1]),
                     "v"(t1a), "v"(t1b), "v"(t2a), "v"(t2b));

        // causal diagonal or ragged last tile: mask tile j+1 before its
        // probabilities are formed in the next iteration
        if constexpr (NEXT) {
            if (j + 1 >= nfull) mask(j + 1, oth.s1, oth.s2);
        }
        // lazy-maximum test on tile j: a large partial sum means that some
        // scores passed the stale maximum; take the exact maxima of the tile,
        // rescale, and form its probabilities again
        float t1 = t1a + t1b, t2 = t2a + t2b;
        if (__builtin_amdgcn_ballot_w64(t1 > kSumLimit || t2 > kSumLimit)) {
            const float x1 = max16(cur.s1) * sl2, x2 = max16(cur.s2) * sl2;
            const float mn1 = fmaxf(m1, fmaxf(x1, xor32(x1)));
            const float mn2 = fmaxf(m2, fmaxf(x2, xor32(x2)));
            const float al1 = mn1 == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m1 - mn1);
            const float al2 = mn2 == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m2 - mn2);
            m1 = mn1;
            m2 = mn2;
            l1 *= al1;
            l2 *= al2;
            mfma_drain<NDB>(o1, o2);
            scale_acc<NDB>(o1, al1);
            scale_acc<NDB>(o2, al2);
            const float nb1 = m1 == -INFINITY ? 0.f : m1;
            const float nb2 = m2 == -INFINITY ? 0.f : m2;
            t1 = t2 = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                prob_pair(cur.s1, e, sl2, nb1, cur.p1, t1);
                prob_pair(cur.s2, e, sl2, nb2, cur.p2, t2);
            }
        }
        l1 += t1;
        l2 += t2;
        __syncthreads();
    };

    const bool_c<true> T;
    const bool_c<false> F;
    if (nkt == 1) {
        iteration(F, F, 0, A, B);
        pv(stage_of(0), A.p1, A.p2);
    } else {
        iteration(F, T, 0, A, B);
        // tile j lives in A for even j and in B for odd j
        int j = 1;
        for (; j + 1 < nkt - 1; j += 2) {
            iteration(T, T, j, B, A);
            iteration(T, T, j + 1, A, B);
        }
        if (j < nkt - 1) {
            iteration(T, T, j, B, A);
            iteration(T, F, j + 1, A, B);
            pv(stage_of(j + 1), A.p1, A.p2);
        } else {
            iteration(T, F, j, B, A);
            pv(stage_of(j), B.p1, B.p2);
        }
    }

    // epilogue: D = O1/l1 - lambda O2/l2, then GroupNorm over the dv channels
    mfma_drain<NDB>(o1, o2);
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
    const void* fn = causal ? (const void*)prefill_bf16_kernel<D, DV, true>
                            : (const void*)prefill_bf16_kernel<D, DV, false>;
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, int dv, bool causal,
                               hipStream_t stream) {
    if (d == 32 && dv == 64) return launch_dims<32, 64>(a, causal, stream);
    if (d == 64 && dv == 128) return launch_dims<64, 128>(a, causal, stream);
    if (d == 128 && dv == 256) return launch_prefill_bf16_wide(a, d, dv, causal, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
