// Fused Differential Attention prefill for bf16 inputs with head_dim 128 and
// v_dim 256 on gfx950 (CDNA4), in two sweeps over the keys.
//
// Operator: the DiffAttn formula (iloveeagents.com, "Mathematical Formula")
// with the GroupNorm and (1 - lambda_init) scale of step 4 on llmbytes.dev
// ("How Differential Attention Cancels Common-Mode Noise"), fused into one
// kernel ("Throughput and Hardware Realities").
//
// Why two sweeps.  The one-sweep form keeps O1 = P1 V and O2 = P2 V apart and
// subtracts O1/l1 - lambda O2/l2 at the end; each map's probabilities are
// rounded to bf16 on their own before P.V.  When lambda is near 1 and the two
// maps nearly agree (the common-mode noise the subtraction exists to remove),
// D is a small difference of two large sums and the GroupNorm scales it back
// to unit spread, so each map's bf16 rounding (relative 2^-9) can reach the
// output at several percent.  Here the weights of both maps are formed first
// and subtracted before any rounding to bf16:
//
//   sweep 1   S_k = Q_k K_k^T (k = 1, 2) for every key tile; per row and map
//             the running maximum m_k and l_k = sum_j 2^(S_k scale - m_k);
//   sweep 2   S_k again; a_k = 2^(S_k scale - m_k) / l_k (the final softmax
//             weights), P = a_1 - lambda a_2, then O = P V, one P.V product.
//
// The matrix work per unmasked pair is 2*2d (sweep 1) + 2*2d + 2 dv (sweep 2)
// = 4 (d + dv) flops when dv = 2d, the same as the one-sweep form; the
// exponentials double.  At head_dim 128 the kernel is bound by the matrix
// cores (3,072 flops per byte), so the second set of exponentials is cheap.
//
// Work decomposition
//   A work item is 128 query rows of one (batch, head), taken by one
//   workgroup of 8 wavefronts; the grid is persistent and deals items out
//   head by head within each XCD, longest-first in a snake (schedule.h): the
//   XCD's workgroups sweep one head's K and V together, through its L2.  Wave w owns query block w % 4 (32 rows) and map
//   w / 4: it computes that map's scores and statistics, and in sweep 2 the
//   P.V of half of the dv channels (map 1's wave channels 0..127, map 2's
//   wave 128..255).  Both waves of a query block need the full P, so each
//   writes its map's weights, scaled by 2^15 and rounded toward zero to fp16
//   (the lambda map's negated), to LDS and keeps them; after the tile's
//   barrier each reads the other's and forms P = x1 - x2 in fp16 arithmetic,
//   then rounds P to bf16 for the product.
//   The two waves compute bit-identical P, so the two halves of a row agree.
//   The weights are at most 1 (times 2^15 < 65504), fp16 keeps 11 bits where
//   bf16 keeps 8, and the difference is rounded relative to itself: the
//   rounding error that reaches D is relative to D, not to the two maps.
//   Per wave: one O^T accumulator of 32 rows x 128 channels (64 registers)
//   instead of two of 256 channels; two waves share each SIMD.
//
// Per tile and wave, on MFMA v_mfma_f32_32x32x16_bf16:
//   S^T = K_k Q_k^T              8 products (keys on M, the wave's 32 queries on N)
//   O^T += V_half^T P^T          8 products (sweep 2)
// with the operand layouts of the narrow-head kernel: the score tile's A
// operand loads key row swap23(l), so accumulator register r of lane l holds
// key 16 (r/8) + 8 (l/32) + r%8 of query l%32 and registers 8c .. 8c+7 are
// the B operand P^T of keys 16c ..; V^T comes from ds_read_b64_tr_b16.
//
// With e4m3 queries and keys (prefill_fp8qk_twopass_kernel, the low-bit
// variant of "Throughput and Hardware Realities"), the scores of a tile are
// two v_mfma_scale_f32_32x32x64_f8f6f4 products (unit block scales; the
// per-tensor scales multiply the exponent's scale), a K row is 128 bytes and
// a K stage 8 KB; the weights, P and the P.V product are as above.
//
// Tiles stream through two 4-stage LDS rings (K1 and K2 of a tile in one
// 16 KB stage, V in another), filled by buffer loads with the LDS
// destination (no registers, no LDS store instructions), three tiles ahead
// of use.  The two sweeps form one sequence of K tiles (sweep 1's, then sweep
// 2's), so the ring runs on across the boundary and sweep 1's last iteration
// already computes sweep 2's first scores.  V tiles are loaded in sweep 2
// only (its first two at the item's start).  One barrier per tile.
//
// LDS (160 KB): K ring 64 KB, V ring 64 KB, two 16 KB weight-exchange slots
// (the slot written for tile t is read for tile t in the next iteration while
// the next tile's weights go to the other slot).  Rows are XOR-swizzled by
// 16-byte chunk so that the operand reads hit distinct banks.

#include "internal.h"
#include "schedule.h"

#include <math.h>

// The direct-to-LDS loads set M0 in inline asm; nothing else in this file
// uses M0, so the reserved-register clobber is safe here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 512;
constexpr int kBlocks = 4;               // query blocks of 32 rows per item
constexpr int kBc = 32;                  // keys per tile
constexpr int kD = 128;
constexpr int kDV = 256;
constexpr int kBr = 32 * kBlocks;
constexpr int kNKB = kD / 16;            // score products per tile (k = 16 each)
constexpr int kNDB = kDV / 2 / 32;       // channel blocks of a wave's half of dv
constexpr int kStages = 4;               // K ring and V ring
constexpr int kVRow = 2 * kDV;           // bytes per V row
constexpr int kVStage = kBc * kVRow;     // 16 KB
constexpr int kXchgWave = 64 * 32;                    // 16 fp16 per lane
constexpr int kXchgSlot = (kThreads / 64) * kXchgWave;
constexpr int kVLoads = kVStage / (16 * kThreads);    // V load instructions per wave and tile
constexpr float kSumLimit = 4096.0f;     // lazy-maximum bound on a lane's partial tile sum
constexpr int kXScale = 15;              // exchanged weights are a * 2^15
constexpr int kBufferDword3 = 0x00020000;

// The K side, by operand format: bf16 (F8 = false) or e4m3 queries and keys
// (one byte per element, per-tensor scales; the scores then run on
// v_mfma_scale_f32_32x32x64_f8f6f4, two products per tile instead of eight).
template <bool F8>
struct KSide {
    static constexpr int kRow = F8 ? kD : 2 * kD;        // bytes per Q or K row
    static constexpr int kCpr = kRow / 16;               // 16-byte chunks per row
    static constexpr int kTile = kBc * kRow;             // one map's K tile
    static constexpr int kStage = 2 * kTile;             // K1 then K2
    static constexpr int kLoads = kStage / (16 * kThreads);
    static constexpr int kVRing = kStages * kStage;      // V ring start
    static constexpr int kXchg = kVRing + kStages * kVStage;
    static constexpr int kSmem = kXchg + 2 * kXchgSlot;  // 160 KB (bf16), 128 KB (e4m3)
    static constexpr int kNKS = F8 ? kD / 64 : kD / 16;  // score products per tile
    static constexpr int kOps = F8 ? 2 * kNKS : kNKS;    // 16-byte K operand reads per tile
    static_assert(kStage % (16 * kThreads) == 0, "a K stage splits into whole loads per wave");
    // chunk swizzle of a K row: 16 chunks (one pass over the 64 banks) or 8
    static __device__ __forceinline__ int swz(int r) { return F8 ? (r >> 1) & 7 : r & 15; }
};
static_assert(kVStage == kVLoads * 16 * kThreads, "a V stage splits into whole loads per wave");

__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ float max16(const f32x16& s) {
    float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
    float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
    float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, s[15]));
}

// Raw buffer descriptor of `bytes` bytes from `base` (wave-uniform values):
// loads at offsets past the end return zeros.  The record count is a 32-bit
// field, so it is clamped.
__device__ __forceinline__ i32x4 sgpr_rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
    const uint64_t p = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = kBufferDword3;
    return r;
}

// P = x1 - x2 for the 8 weight pairs of a tile as own + partner: the first
// map's wave stores x1, the lambda map's wave -x2, each keeps its own values
// and reads the other's (two 16-byte reads).  Each sum is formed in fp32 as
// fma(own, one, other) on the fp16 halves -- the compiler selects
// v_fma_mix_f32, which converts and adds in one instruction, when the fp16
// one is not a constant it could fold -- exactly (two fp16 values sum
// exactly in fp32 unless their exponents differ by more than 12); fp32
// addition commutes, so both waves get the same bits.  Rounded once to bf16
// in B-operand order (registers 8kb .. 8kb+7).
__device__ __forceinline__ void combine(const u32x4 (&own)[2], const u32x4 (&other)[2], bf16x8 (&pb)[2]) {
    uint32_t one_bits = 0x3c00u;  // fp16 1.0
    asm volatile("" : "+s"(one_bits));
    const float one = (float)__builtin_bit_cast(_Float16, (uint16_t)one_bits);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const u32x4 v1 = own[kb], v2 = other[kb];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w1 = v1[c], w2 = v2[c];
            const _Float16 a0 = __builtin_bit_cast(_Float16, (uint16_t)w1);
            const _Float16 a1 = __builtin_bit_cast(_Float16, (uint16_t)(w1 >> 16));
            const _Float16 b0 = __builtin_bit_cast(_Float16, (uint16_t)w2);
            const _Float16 b1 = __builtin_bit_cast(_Float16, (uint16_t)(w2 >> 16));
            pb[kb][2 * c] = (__bf16)__builtin_fmaf((float)a0, one, (float)b0);
            pb[kb][2 * c + 1] = (__bf16)__builtin_fmaf((float)a1, one, (float)b1);
        }
    }
}

// chunk swizzle of a V row (32 chunks); K rows: KSide::swz
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

template <bool B>
using bool_c = std::integral_constant<bool, B>;

// FLAT: each (batch, head) slice of K and V spans < 2 GiB (one descriptor per
// tensor); SAVE: training forward, also writes D and the log-sum-exp rows.
template <bool CAUSAL, bool FLAT, bool SAVE, bool F8>
__device__ __forceinline__ void twopass_items(const PrefillArgs& a) {
    using KS = KSide<F8>;
    constexpr int kKRow = KS::kRow, kKTile = KS::kTile, kKStage = KS::kStage;
    constexpr int kVRing = KS::kVRing, kXchg = KS::kXchg;
    __shared__ __attribute__((aligned(16))) uint8_t smem[KS::kSmem];

    const int BH = a.B * a.H;
    const int nqt = (a.Nq + kBr - 1) / kBr;
    const int G = gridDim.x;
    for (int r = 0;; ++r) {
    int t, bh;
    if (!prefill_item(r, blockIdx.x, G, nqt, BH, t, bh)) break;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int lh = lane >> 5;
    const int qb = wave & (kBlocks - 1);
    const int map = wave >> 2;  // 0: first softmax map, 1: the lambda map
    const int qt = CAUSAL ? (nqt - 1 - t) : t;
    const int h = bh % a.H;
    const float lam_h = a.lam[h];

    const char* gq = (const char*)(map ? a.q2 : a.q1) + (size_t)bh * a.Nq * kKRow;
    const char* gk1 = (const char*)a.k1 + (size_t)bh * a.Nk * kKRow;
    const char* gk2 = (const char*)a.k2 + (size_t)bh * a.Nk * kKRow;
    const char* gv = (const char*)a.v + (size_t)bh * a.Nk * kVRow;
    __bf16* gout = (__bf16*)a.out + (size_t)bh * a.Nq * kDV;

    const int wq0 = qt * kBr + qb * 32;
    const int qrow = wq0 + l32;

    // Q fragments of the wave's map as B operands: column = query, k-slots =
    // channels 16 kb + 8 lh ..
    // (e4m3: k-step s of 64 bytes, this lane's bytes 64 s + 32 lh .. + 31)
    bf16x8 qf[F8 ? 1 : kNKB];
    i32x8 qf8[F8 ? kD / 64 : 1];
    if constexpr (F8) {
#pragma unroll
        for (int ks = 0; ks < kD / 64; ++ks)
            qf8[ks] = qrow < a.Nq ? *(const i32x8*)(gq + (size_t)qrow * kKRow + 64 * ks + 32 * lh)
                                  : i32x8{};
    } else {
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
            qf[kb] = qrow < a.Nq ? *(const bf16x8*)(gq + (size_t)qrow * kKRow + 2 * (16 * kb + 8 * lh))
                                 : bf16x8{};
    }

    const int nkt_all = (a.Nk + kBc - 1) / kBc;
    const int nkt = CAUSAL ? min(nkt_all, (qt * kBr + kBr + kBc - 1) / kBc) : nkt_all;
    const int nfull = __builtin_amdgcn_readfirstlane(CAUSAL ? min(a.Nk / kBc, (wq0 + 1) / kBc) : a.Nk / kBc);

    // ---- tile loads: global -> LDS ring, buffer_load_dwordx4 ... lds ----
    // Load instruction i of wave w covers the stage's chunk positions
    // 64 (w + 8 i) .. + 63.  K stage (K1's tile, then K2's): which map that
    // is follows from the position (bf16: instruction i reads K_{i+1};
    // e4m3: waves 0-3 K1, 4-7 K2); V stage: rows 2 (w + 8 i), + 1.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int k_ld_off[KS::kLoads], k_src[KS::kLoads];
#pragma unroll
    for (int i = 0; i < KS::kLoads; ++i) {
        const int pos = 64 * (wave_u + 8 * i) + lane;  // chunk position in the stage
        const int q = pos % (kKTile / 16);
        const int row = q / KS::kCpr;
        k_src[i] = __builtin_amdgcn_readfirstlane(pos / (kKTile / 16));  // 0: K1, 1: K2
        k_ld_off[i] = row * kKRow + 16 * ((q % KS::kCpr) ^ KS::swz(row));
    }
    int v_ld_off[kVLoads];
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
        const int vpos = 64 * (wave_u + 8 * i) + lane;
        v_ld_off[i] = (vpos >> 5) * kVRow + 16 * ((vpos & 31) ^ v_swz(vpos >> 5));
    }
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    const int64_t kbytes = (int64_t)a.Nk * kKRow, vbytes = (int64_t)a.Nk * kVRow;
    const i32x4 rs_k1 = sgpr_rsrc(gk1, kbytes), rs_k2 = sgpr_rsrc(gk2, kbytes);
    const i32x4 rs_v = sgpr_rsrc(gv, vbytes);
    auto load_lds = [](uint32_t m0, int voff, i32x4 rsrc) {
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(rsrc)
                     : "memory", "m0");
    };
    // K tiles of the two sweeps form one sequence: seq s < nkt is sweep 1's
    // key tile s, nkt <= s < 2 nkt sweep 2's key tile s - nkt; it goes to
    // ring stage s mod 4.  Past the sequence the loads write zeros (the
    // instruction count per iteration stays fixed for the waits).
    auto issue_k = [&](int s) {
        const int kt = s < nkt ? s : s - nkt;
        const bool real = s < 2 * nkt;
        const uint32_t st_off = (uint32_t)(s & (kStages - 1)) * kKStage;
#pragma unroll
        for (int i = 0; i < KS::kLoads; ++i) {
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(
                smem_base + st_off + (uint32_t)(16 * 64 * (wave_u + 8 * i)));
            if constexpr (FLAT) {
                const int voff = k_ld_off[i] + (real ? kt * kKTile : (int)kbytes);
                load_lds(m0, voff, k_src[i] == 0 ? rs_k1 : rs_k2);
            } else {
                const int64_t key0 = (int64_t)kt * kBc;
                const int64_t left = real ? (int64_t)a.Nk - key0 : 0;
                load_lds(m0, k_ld_off[i],
                         sgpr_rsrc((k_src[i] == 0 ? gk1 : gk2) + key0 * kKRow, left * kKRow));
            }
        }
    };
    // V tile j (sweep 2) goes to V stage (nkt + j) mod 4: the stage index of
    // the iteration that forms tile j's weights
    auto issue_v = [&](int j) {
        const bool real = j < nkt;
        const uint32_t st_off = kVRing + (uint32_t)((nkt + j) & (kStages - 1)) * kVStage;
#pragma unroll
        for (int i = 0; i < kVLoads; ++i) {
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(
                smem_base + st_off + (uint32_t)(16 * 64 * (wave_u + 8 * i)));
            if constexpr (FLAT) {
                const int voff = v_ld_off[i] + (real ? j * kVStage : (int)vbytes);
                load_lds(m0, voff, rs_v);
            } else {
                const int64_t key0 = (int64_t)j * kBc;
                const int64_t left = real ? (int64_t)a.Nk - key0 : 0;
                load_lds(m0, v_ld_off[i], sgpr_rsrc(gv + key0 * kVRow, left * kVRow));
            }
        }
    };
    // this wave's loads still in flight may number at most N (in order)
    auto wait_loads = [](auto n) {
        constexpr int N = decltype(n)::value;
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    };

    // ---- operands ----
    const int krow = swap23(l32);
    // this lane's 16-byte pieces of its map's K tile (A operand, row krow):
    // bf16, piece kb = channels 16 kb + 8 lh ..; e4m3, pieces 2 s, 2 s + 1 =
    // bytes 64 s + 32 lh .. + 31 of k-step s
    int k_off[KS::kOps];
#pragma unroll
    for (int kb = 0; kb < KS::kOps; ++kb) {
        const int ch = F8 ? 4 * (kb >> 1) + 2 * lh + (kb & 1) : 2 * kb + lh;
        k_off[kb] = map * kKTile + krow * kKRow + 16 * (ch ^ KS::swz(krow));
    }
    auto k_operand = [&](int st, int kb) {
        return *(const bf16x8*)(smem + st * kKStage + k_off[kb]);
    };
    // transposing V reads: in each 16-lane group g, lane 4e + r addresses key
    // row e (+ 8 for the upper half-wave) at channel base + 16 (g % 2) + 4 r
    const int vg = lane >> 4;
    const int ve = (lane & 15) >> 2;
    const int vr = lane & 3;
    int v_off[kNDB];
#pragma unroll
    for (int db = 0; db < kNDB; ++db)
        v_off[db] = kVRing + (8 * (vg >> 1) + ve) * kVRow +
                    16 * ((16 * map + 4 * db + 2 * (vg & 1) + (vr >> 1)) ^ v_swz(ve)) + 8 * (vr & 1);
    auto v_operand = [&](int st, int db, int kb) {
        const uint8_t* vp = smem + st * kVStage + v_off[db] + 16 * kb * kVRow;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint8_t*)vp);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint8_t*)(vp + 4 * kVRow));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // register r holds key kt*kBc + 8 lh + 16 (r/8) + r%8: one bound per lane
    // (the last key, and under the causal mask the query row), one compare
    // with a constant per register
    auto mask = [&](int kt, f32x16& s) {
        const int last = CAUSAL ? min(qrow, a.Nk - 1) : a.Nk - 1;
        const int lim = last - kt * kBc - 8 * lh;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 16 * (r >> 3) + (r & 7) <= lim ? s[r] : -INFINITY;
    };
    // key tile of sequence entry s
    auto tile_of = [&](int s) { return s < nkt ? s : s - nkt; };

    // e4m3: the product of the map's two dequantisation scales folds into exp2's
    const float sl2 = F8 ? a.scale_log2 * a.qk_scale[map] : a.scale_log2;
    float m, l = 0.f;
    f32x16 o[kNDB];
#pragma unroll
    for (int db = 0; db < kNDB; ++db) o[db] = f32x16{};

    // ---- prologue: V tiles 0, 1 and K sequence 0 .. 3 in flight ----
    issue_v(0);
    issue_v(1);
    issue_k(0);
    issue_k(1);
    // the compiler waits for the Q loads by counting its own loads only, which
    // also drains the tile loads issued so far (they are needed first anyway)
    if constexpr (F8) {
#pragma unroll
        for (int ks = 0; ks < kD / 64; ++ks) asm volatile("" ::"v"(qf8[ks]));
    } else {
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb) asm volatile("" ::"v"(qf[kb]));
    }
    issue_k(2);
    issue_k(3);
    __syncthreads();

    f32x16 sa, sb;  // score tiles: sequence entry s lives in sa for even s, sb for odd
    auto scores = [&](int st, f32x16& s) {
        bf16x8 ka[KS::kOps];
#pragma unroll
        for (int kb = 0; kb < KS::kOps; ++kb) ka[kb] = k_operand(st, kb);
        if constexpr (F8) {
#pragma unroll
            for (int ks = 0; ks < kD / 64; ++ks) {
                const i32x8 ka8 = __builtin_bit_cast(
                    i32x8, __builtin_shufflevector(__builtin_bit_cast(i32x4, ka[2 * ks]),
                                                   __builtin_bit_cast(i32x4, ka[2 * ks + 1]), 0, 1,
                                                   2, 3, 4, 5, 6, 7));
                // e4m3 A and B (format 0), unit block scales (127 = 2^0)
                s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka8, qf8[ks], ks == 0 ? f32x16{} : s,
                                                                    0, 0, 0, 127, 0, 127);
            }
        } else {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int kb = 1; kb < kNKB; ++kb)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb], qf[kb], s, 0, 0, 0);
        }
    };
    scores(0, sa);
    if (nfull < 1) mask(0, sa);
    {
        // exact row maxima of the first tile start the running maxima
        const float x = max16(sa) * sl2;
        m = fmaxf(x, xor32(x));
    }
    // iteration 0 refills ring stage 0, which every wave has just read
    __syncthreads();

    // ---- sweep 1: statistics.  Iteration g: scores of sequence entry g+1
    // (MFMA), the lazy-maximum sums of entry g (VALU), loads of entry g+4.
    auto sweep1 = [&](int g, f32x16& cur, f32x16& nxt) {
        scores((g + 1) & (kStages - 1), nxt);
        float ta = 0.f, tb = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            ta += __builtin_amdgcn_exp2f(fmaf(cur[e], sl2, -m));
            tb += __builtin_amdgcn_exp2f(fmaf(cur[e + 1], sl2, -m));
        }
        float tsum = ta + tb;
        // a large partial sum: some scores passed the running maximum; take the
        // tile's exact maxima, rescale l, and sum again
        if (__builtin_amdgcn_ballot_w64(tsum > kSumLimit)) {
            const float x = max16(cur) * sl2;
            const float mn = fmaxf(m, fmaxf(x, xor32(x)));
            l *= __builtin_amdgcn_exp2f(m - mn);
            m = mn;
            float ua = 0.f, ub = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                ua += __builtin_amdgcn_exp2f(fmaf(cur[e], sl2, -m));
                ub += __builtin_amdgcn_exp2f(fmaf(cur[e + 1], sl2, -m));
            }
            tsum = ua + ub;
        }
        l += tsum;
        issue_k(g + 4);
        if (tile_of(g + 1) >= nfull) mask(tile_of(g + 1), nxt);
        wait_loads(std::integral_constant<int, 2 * KS::kLoads>{});
        __syncthreads();
    };
    int g = 0;
    for (; g + 1 < nkt; g += 2) {
        sweep1(g, sa, sb);
        sweep1(g + 1, sb, sa);
    }
    if (g < nkt) {
        sweep1(g, sa, sb);
        // sweep 2's first scores (entry nkt, odd) landed in sb
        sa = sb;
    }

    // ---- sweep 2 constants: a_k 2^(15 - e) = 2^(S scale - base2) with
    // base2 = m + log2 l - (15 - e) - log2(c_k), c_1 = 1, c_2 = |lambda|; e
    // makes room for |lambda| > 1 (the exchanged values stay below 2^15)
    const float L = l + xor32(l);
    const float alam = fabsf(lam_h);
    int e_sc = 0;
    if (alam > 1.f) (void)frexpf(alam, &e_sc);
    const bool lambda_map = __builtin_amdgcn_readfirstlane(map) != 0;
    const float lc = lambda_map ? __builtin_amdgcn_logf(alam) : 0.f;  // log2: 0 for c = 1
    const float base2 = ((m + __builtin_amdgcn_logf(L)) - (float)(kXScale - e_sc)) - lc;
    // the lambda map's wave stores -x2 = -fp16(2^(15-e) lambda a_2): its
    // exponentials give |lambda| a_2, negated unless lambda < 0
    const bool flip = lambda_map && !(lam_h < 0.f);
    u32x4 own[2];  // this wave's stored weights of the previous tile

    // ---- sweep 2.  Iteration g (tile j = g - nkt): P of tile j-1 from the
    // exchange slot and its P.V (MFMA), scores of entry g+1 (MFMA), weights
    // of tile j into the other slot (VALU), loads of V tile j+2 and K entry g+4.
    auto xchg_at = [&](int slot, int w) { return smem + kXchg + slot * kXchgSlot + w * kXchgWave; };
    auto sweep2 = [&](auto prev, auto next, int j, f32x16& cur, f32x16& nxt) {
        constexpr bool PREV = decltype(prev)::value;
        constexpr bool NEXT = decltype(next)::value;
        const int gg = nkt + j;
        bf16x8 pb[2];
        u32x4 other[2];
        if constexpr (PREV) {
            const int slot = (gg - 1) & 1;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                other[i] = *(const u32x4*)(xchg_at(slot, wave ^ 4) + 1024 * i + 16 * lane);
        }
        if constexpr (NEXT) scores((gg + 1) & (kStages - 1), nxt);
        if constexpr (PREV) {
            combine(own, other, pb);
            const int vst = (gg - 1) & (kStages - 1);
#pragma unroll
            for (int db = 0; db < kNDB; ++db) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(vst, db, kb), pb[kb],
                                                                    o[db], 0, 0, 0);
            }
        }
        // this tile's weights, scaled and rounded toward zero to fp16
        uint32_t xw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(cur[2 * i], sl2, -base2));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(cur[2 * i + 1], sl2, -base2));
            xw[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
        }
        if (flip) {
#pragma unroll
            for (int i = 0; i < 8; ++i) xw[i] ^= 0x80008000u;
        }
        own[0] = u32x4{xw[0], xw[1], xw[2], xw[3]};
        own[1] = u32x4{xw[4], xw[5], xw[6], xw[7]};
        {
            uint8_t* dst = xchg_at(gg & 1, wave) + 16 * lane;
            *(u32x4*)dst = own[0];
            *(u32x4*)(dst + 1024) = own[1];
        }
        issue_v(j + 2);
        issue_k(gg + 4);
        if constexpr (NEXT) {
            if (j + 1 >= nfull) mask(j + 1, nxt);
        }
        wait_loads(std::integral_constant<int, 2 * KS::kLoads + kVLoads>{});
        __syncthreads();
    };
    const bool_c<true> T;
    const bool_c<false> F;
    int j = 0;
    if (nkt == 1) {
        sweep2(F, F, 0, sa, sb);
        j = 1;
    } else {
        sweep2(F, T, 0, sa, sb);
        for (j = 1; j + 2 < nkt; j += 2) {
            sweep2(T, T, j, sb, sa);
            sweep2(T, T, j + 1, sa, sb);
        }
        if (j + 1 < nkt) {
            sweep2(T, T, j, sb, sa);
            sweep2(T, F, j + 1, sa, sb);
        } else {
            sweep2(T, F, j, sb, sa);
        }
        j = nkt;
    }
    // P.V of the last tile
    {
        const int gg = 2 * nkt;
        const int slot = (gg - 1) & 1;
        bf16x8 pb[2];
        u32x4 other[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            other[i] = *(const u32x4*)(xchg_at(slot, wave ^ 4) + 1024 * i + 16 * lane);
        combine(own, other, pb);
        const int vst = (gg - 1) & (kStages - 1);
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(vst, db, kb), pb[kb], o[db],
                                                                0, 0, 0);
        }
    }

    // ---- epilogue: D = O 2^(e - 15) on the wave's half of the channels, the
    // GroupNorm over all dv channels (half-row statistics merged pairwise,
    // Chan, Golub and LeVeque), the (1 - lambda_init) scale, bf16 stores
    // through LDS as whole row segments
    wait_loads(std::integral_constant<int, 0>{});
    __syncthreads();  // the rings and the exchange slots are free from here
    const float dscale = ldexpf(1.f, e_sc - kXScale);
    float x[kNDB][16];
#pragma unroll
    for (int db = 0; db < kNDB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[db][r] = o[db][r] * dscale;
    }
    if constexpr (SAVE) {
        if (qrow < a.Nq) {
            float* drow = a.d_save + ((size_t)bh * a.Nq + qrow) * kDV + map * (kDV / 2);
#pragma unroll
            for (int db = 0; db < kNDB; ++db) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *(float4*)(drow + 32 * db + 8 * gq + 4 * lh) =
                        make_float4(x[db][4 * gq], x[db][4 * gq + 1], x[db][4 * gq + 2], x[db][4 * gq + 3]);
            }
            if (lh == 0)
                a.lse[((size_t)map * a.B * a.H + bh) * a.Nq + qrow] =
                    (m + __builtin_amdgcn_logf(L)) * 0.69314718055994531f;
        }
    }
    if (!(a.flags & 1u)) {
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) ps[r & 3] += x[db][r];
        }
        float hs = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        hs += xor32(hs);
        const float mh = hs * (2.f / kDV);  // mean of this half of the row
        float pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float c = x[db][r] - mh;
                pq[r & 3] = fmaf(c, c, pq[r & 3]);
            }
        }
        float hq = (pq[0] + pq[1]) + (pq[2] + pq[3]);
        hq += xor32(hq);
        float2* stats = (float2*)(smem + kXchg);
        stats[(qb * 2 + map) * 64 + lane] = make_float2(mh, hq);
        __syncthreads();
        const float2 ot = stats[(qb * 2 + (map ^ 1)) * 64 + lane];
        // both waves evaluate the same expressions in the same order
        const float mean = 0.5f * (mh + ot.x);
        const float dm = mh - ot.x;
        const float m2 = (hq + ot.y) + dm * dm * (0.25f * kDV);
        const float var = m2 * (1.f / kDV);
        const float sc = (1.f - a.lambda_init) / sqrtf(var + a.eps);
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[db][r] = (x[db][r] - mean) * sc;
        }
    }
    // Output: the wave's 32 rows by 128 channels go through LDS (bf16, 16
    // chunks per half row, chunk index swizzled by row) so that each store
    // instruction writes whole 256-byte row segments.
    {
        constexpr int kCpr = kDV / 16;  // chunks per half row
        uint16_t* so = (uint16_t*)smem + wave * (32 * (kDV / 2));
        const int swr = l32 % kCpr;
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)x[db][4 * gq + e];
                *(bf16x4*)(so + l32 * (kDV / 2) + 8 * ((4 * db + gq) ^ swr) + 4 * lh) = w;
            }
        }
        constexpr int kRowsPerStore = 64 / kCpr;
        __bf16* gbase = gout + (size_t)wq0 * kDV + map * (kDV / 2);
#pragma unroll
        for (int k = 0; k < 32 / kRowsPerStore; ++k) {
            const int row = k * kRowsPerStore + lane / kCpr;
            const int ch = lane % kCpr;
            const uint4 w = *(const uint4*)(so + row * (kDV / 2) + 8 * (ch ^ (row % kCpr)));
            if (wq0 + row < a.Nq) *(uint4*)(gbase + (size_t)row * kDV + 8 * ch) = w;
        }
    }
    __syncthreads();  // the LDS is reused by the next item
    }
}

template <bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kThreads) void prefill_bf16_twopass_kernel(PrefillArgs a) {
    twopass_items<CAUSAL, FLAT, false, false>(a);
}

template <bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kThreads) void prefill_train_twopass_kernel(PrefillArgs a) {
    twopass_items<CAUSAL, FLAT, true, false>(a);
}

// Scores from e4m3 queries and keys (per-tensor scales in a.qk_scale).
template <bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kThreads) void prefill_fp8qk_twopass_kernel(PrefillArgs a) {
    twopass_items<CAUSAL, FLAT, false, true>(a);
}

}  // namespace

hipError_t launch_prefill_twopass(const PrefillArgs& a, int d, int dv, bool causal, bool fp8qk,
                                  hipStream_t stream) {
    if (d != kD || dv != kDV) return hipErrorInvalidValue;
    const int nqt = (a.Nq + kBr - 1) / kBr;
    const int64_t items = (int64_t)nqt * a.B * a.H;
    if (items > (int64_t)0x7fffffff - 4096) return hipErrorInvalidValue;
    const int cus = device_cus();
    const dim3 grid((unsigned)(cus > 0 && items > cus ? cus : items));
    PrefillArgs copy = a;
    void* args[] = {&copy};
    // one descriptor per tensor when each (batch, head) slice spans < 2 GiB
    const bool flat = one_descriptor(a.flags, (int64_t)a.Nk * kVRow);
    const void* fn;
    if (fp8qk) {
        if (a.lse) return hipErrorInvalidValue;  // no training forward from e4m3 scores
        fn = causal ? (flat ? (const void*)prefill_fp8qk_twopass_kernel<true, true>
                            : (const void*)prefill_fp8qk_twopass_kernel<true, false>)
                    : (flat ? (const void*)prefill_fp8qk_twopass_kernel<false, true>
                            : (const void*)prefill_fp8qk_twopass_kernel<false, false>);
    } else if (a.lse)
        fn = causal ? (flat ? (const void*)prefill_train_twopass_kernel<true, true>
                            : (const void*)prefill_train_twopass_kernel<true, false>)
                    : (flat ? (const void*)prefill_train_twopass_kernel<false, true>
                            : (const void*)prefill_train_twopass_kernel<false, false>);
    else
        fn = causal ? (flat ? (const void*)prefill_bf16_twopass_kernel<true, true>
                            : (const void*)prefill_bf16_twopass_kernel<true, false>)
                    : (flat ? (const void*)prefill_bf16_twopass_kernel<false, true>
                            : (const void*)prefill_bf16_twopass_kernel<false, false>);
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace diffattn
