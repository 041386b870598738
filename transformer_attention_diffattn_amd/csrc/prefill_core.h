// The bf16 prefill forward for head_dim 32 and 64 as a template
// (prefill_items), kept apart from its instantiations in prefill_bf16.hip
// (the forward, the training forward, the e4m3-score variant).  head_dim 128
// is in prefill_twopass.hip.
//
// Fused Differential Attention prefill for bf16 inputs on gfx950 (CDNA4).
//
// Operator: the DiffAttn formula (iloveeagents.com, "Mathematical Formula")
// with the GroupNorm and (1 - lambda_init) scale of step 4 on llmbytes.dev
// ("How Differential Attention Cancels Common-Mode Noise").  The pages note
// that a custom kernel can fuse the two softmax maps and the subtraction into
// one memory pass ("Throughput and Hardware Realities"); this is that kernel.
//
// Work decomposition
//   A work item is 128 query rows of one (batch, head), taken by one
//   workgroup of 8 wavefronts.  The grid is persistent (one workgroup per
//   compute unit when there are more items than units): items are dealt out
//   longest-first in a snake, so the causal lengths even out and no
//   workgroup launches per item, and head by head within each XCD, so the
//   XCD's workgroups sweep one head's K and V together (schedule.h).  Wave
//   w owns query block w % 4 (32 rows) of map w / 4: the two softmax maps of
//   a row are computed by two waves, and the lambda-weighted subtraction is
//   done once, through LDS, in the epilogue.  Splitting by map halves the
//   registers of a wave (one O^T accumulator, one score tile), which lets two
//   waves share each SIMD; a wave waiting on LDS or on the barrier then
//   leaves the SIMD to the other.  Waves w and w + 4 run on the same SIMD, one
//   per map.  K1, K2 and V stream through an 8-stage LDS ring in tiles of 32
//   keys, loaded 5 tiles ahead of use; each wave reads the K tile of its own
//   map and the shared V tile.  The main loop is unrolled over one turn of
//   the ring, so every stage address is an instruction's immediate offset
//   (K and V sit in two rings of that depth, each under the 64 KB reach of
//   the offset) and the loop spends no instructions on stage arithmetic.
//
//   Iteration j of a wave issues, in one branch-free block,
//     MFMA  scores of tile j+1, P.V of tile j-1;
//     VALU  probabilities of tile j, row sums;
//     memory  the global-to-LDS loads of tile j+5 (all waves);
//   and ends with the masking of tile j+1 (tiles on the causal diagonal and
//   the ragged last tile only) and the lazy-maximum test of tile j (below),
//   whose body almost never runs.  None of the three streams waits for
//   another inside the block, so the two waves of a SIMD can overlap one's
//   matrix work with the other's vector work.  One barrier per two tiles.
//
// Per tile and wave, on MFMA v_mfma_f32_32x32x16_bf16 (k = the wave's map):
//   S_k^T = K_k Q_k^T          (keys on the M axis, the wave's 32 queries on N),
//   O_k^T = alpha O_k^T + V^T P_k^T.
//   With the transposed score tile every query lives in one lane pair (lanes
//   l and l+32), so online-softmax row statistics are in-lane reductions plus
//   one exchange, and the rescale of O^T is a per-lane scalar.  The epilogue
//   forms D = O_1 / l_1 - lambda O_2 / l_2, the per-head GroupNorm over the dv
//   channels and the (1 - lambda_init) scale; the two waves of a query block
//   each finish half of the channels and exchange half-row statistics, and
//   the output goes out through LDS as whole row segments.
//
// Online softmax with a lazy maximum: the running maximum m of a row is set
// exactly from the first tile and afterwards moves only when needed.  Each
// tile's probabilities are formed against the current, possibly stale, m and
// may then exceed 1; the sum l and O share that m, so O / l is unchanged.  A
// lane whose partial sum over the tile (16 of the row's 32 keys) exceeds
// kSumLimit flags the tile: its exact row maxima are taken, O and l are
// rescaled, and its probabilities are formed again.  So no probability
// exceeds kSumLimit, and the O rescale (the only VALU work proportional to dv)
// and the row maxima run only when some row's scores climb well past their
// running maximum, which after the first tile is rare.  The test reuses the
// row sums the softmax needs anyway.
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
// LDS per stage: K1, K2 and V tiles row-major without padding, 16-byte
// chunks XOR-swizzled within each row (see k_swz_rb, v_swz) so that operand
// reads hit distinct banks.  Tiles are copied from global memory straight
// into LDS by buffer loads with the LDS destination (no registers, no LDS
// store instructions), through descriptors that end at the last key of the
// (batch, head): rows past the end are filled with zeros without a branch or
// a clamp, and their scores are masked, so they contribute nothing.

#pragma once

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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 512;
constexpr int kBlocks = 4;              // query blocks of 32 rows per workgroup
constexpr int kBc = 32;                 // keys per tile
constexpr float kSumLimit = 4096.0f;    // lazy-maximum bound on a lane's partial tile sum
constexpr int kBufferDword3 = 0x00020000;  // raw buffer descriptor word 3 for gfx9 parts

// F8: Q1, Q2, K1, K2 are e4m3 bytes (per-tensor scales in PrefillArgs), V bf16
template <int D, int DV, bool F8 = false>
struct Cfg {
    static constexpr int kBr = kBlocks * 32;
    static constexpr int kStages = 8;                      // LDS ring (a power of two)
    static constexpr int kAhead = 5;                       // tiles loaded ahead of use
    static constexpr int kKRow = F8 ? D : 2 * D;           // bytes per K row
    static constexpr int kKElems = kBc * kKRow / 2;        // K tile, in 16-bit units
    static constexpr int kVElems = kBc * DV;
    static constexpr int kStage = 2 * kKElems + kVElems;  // 16-bit units per stage
    // the ring is two rings: K1 and K2 of stage s at s kKStage, V of stage s at
    // kVRing + s kVStage, so that any stage's operands sit less than 64 KB
    // past a per-lane base (the LDS instructions' immediate offset)
    static constexpr int kKStage = 2 * kKElems;
    static constexpr int kVStage = kVElems;
    static constexpr int kVRing = kStages * kKStage;
    static constexpr int kKChunks = kBc * kKRow / 16;      // 16-byte chunks per K tile
    static constexpr int kVChunks = kBc * DV / 8;
    static constexpr int kChunks = 2 * kKChunks + kVChunks;
    static constexpr int kWaves = kThreads / 64;
    // load instructions per wave and tile: bf16, 16-byte loads spread evenly;
    // e4m3, one 16-byte load of V and two 4-byte loads of K (K1 then K2)
    static constexpr int kLoads = F8 ? 3 : kChunks / 64 / kWaves;
    static_assert(F8 || kChunks % (64 * kWaves) == 0, "tile must split evenly over the waves");
    static_assert(F8 || kKChunks % 64 == 0, "K regions must start on an instruction boundary");
    static_assert(!F8 || (kVChunks == 64 * kWaves && kKChunks * 16 == 256 * kWaves),
                  "e4m3 tile: one V load and one K1 and one K2 load per wave");
    // a stage is refilled kAhead tiles after its tile, by iteration t + 8 -
    // kAhead for tile t, whose V is last read in iteration t + 1; with a
    // barrier after every odd iteration one always lies between the two
    static_assert(kAhead + 3 <= kStages, "ring too small for the load distance");
    // epilogue, reusing the ring: the two half-row exchanges (one float per
    // query block, accumulator and lane), the GroupNorm statistics (two
    // floats per wave and lane) and the bf16 output staging (32 rows by DV/2
    // channels per wave), in bf16 elements
    static constexpr int kXchgElems = 2 * kBlocks * (DV / 32) * 16 * 64;
    static constexpr int kStatElems = 4 * (kThreads / 64) * 64;
    static constexpr int kStageOutElems = (kThreads / 64) * 32 * (DV / 2);
    static constexpr int kEpiElems = kXchgElems + kStatElems + kStageOutElems;
    static constexpr int kSmemElems = kStages * kStage > kEpiElems ? kStages * kStage : kEpiElems;
};

__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// LDS tiles are stored without padding; 16-byte chunk ch of row r sits at
// chunk position ch ^ swz(r) of its row, which spreads the rows an MFMA
// operand read touches at once over distinct banks.  The LDS serves 256 bytes
// (64 banks) per cycle: 16 lanes of a 16-byte read, 32 lanes of an 8-byte
// read.  A K operand read gives 16 lanes 16 different rows at one chunk
// column; a transposing V read gives 32 lanes 4 consecutive rows at one
// 64-byte column.  The swizzles make those land on distinct banks.
// swizzle of a K row's 16-byte chunks, by row length in bytes
template <int RB>
__device__ __forceinline__ int k_swz_rb(int r) {
    if constexpr (RB == 128)
        return (r >> 1) & 7;  // 8 chunks per row, two rows per 256 bytes
    else
        return (r >> 2) & 3;  // 4 chunks per row, four rows per 256 bytes
}

template <int DV>
__device__ __forceinline__ int v_swz(int r) {
    if constexpr (DV == 128)
        return 4 * (r & 3);         // 16 chunks per row
    else
        return 4 * ((r >> 1) & 1);  // 8 chunks per row, two rows per 256 bytes
}

// a*b - c*d with both products rounded before the subtraction (no fused
// multiply-add), so equal operands cancel to exactly zero
__device__ __forceinline__ float diff_of_products(float a, float b, float c, float d) {
#pragma clang fp contract(off)
    return a * b - c * d;
}

// a*b rounded on its own (the second product of diff_of_products)
__device__ __forceinline__ float product(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

__device__ __forceinline__ float max16(const f32x16& s) {
    float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
    float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
    float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, s[15]));
}

// Raw buffer descriptor of `bytes` bytes from `base` (wave-uniform values),
// as four SGPRs: base address (48 bits, stride 0), record count in bytes,
// word 3.  Loads at offsets past the end return zeros.  The record count is
// a 32-bit field, so it is clamped.
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

// The bf16 probabilities p[e], p[e+1] of a tile packed into pb, added to a
// row partial sum with one dot product against (1, 1): the sum is taken over
// the same rounded values that enter P.V.
// The first pair of a sum: the bf16 dot product with a zero accumulator as
// one instruction (the compiler would zero a register and accumulate).
__device__ __forceinline__ void pack_pair_first(bf16x8 (&pb)[2], int e, float pa, float pc, float& sum) {
    const bf16x2 pr = {(__bf16)pa, (__bf16)pc};
    u32x4 w = __builtin_bit_cast(u32x4, pb[e >> 3]);
    w[(e & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
    pb[e >> 3] = __builtin_bit_cast(bf16x8, w);
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(sum) : "v"(__builtin_bit_cast(uint32_t, pr)), "s"(0x3f803f80u));
}

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

// The whole kernel; F8: Q1, Q2, K1, K2 are e4m3 codes (d = 64 only);
// SAVE: also write D and the log-sum-exp rows for the backward.
template <int D, int DV, bool CAUSAL, bool FLAT, bool F8, bool SAVE>
__device__ __forceinline__ void prefill_items(PrefillArgs a) {
    using C = Cfg<D, DV, F8>;
    static_assert(!F8 || D == 64, "the e4m3 variant is for head_dim 64");
    constexpr int NDB = DV / 32;
    constexpr int NKB = D / 16;               // bf16 score products (k = 16 each)
    constexpr int NKS = F8 ? D / 64 : NKB;    // score products of the variant in use
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::kSmemElems];


    // Work items (query tile, batch*head), taken by the persistent grid in the
    // order of prefill_item (schedule.h): head-major per XCD, longest causal
    // tiles first, in a snake.
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + C::kBr - 1) / C::kBr;
    const int G = gridDim.x;
    for (int r = 0;; ++r) {
    int t, bh;
    if (!prefill_item(r, blockIdx.x, G, nqt, BH, t, bh)) break;
    // opaque per item, so that nothing derived from the lane is hoisted out of
    // the item loop and held live across it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int lh = lane >> 5;
    const int qb = wave & (kBlocks - 1);  // query block
    const int map = wave >> 2;            // 0: first softmax map, 1: the lambda map
    const int qt = CAUSAL ? (nqt - 1 - t) : t;
    const int h = bh % a.H;
    const float lam_h = a.lam[h];

    constexpr int kQRow = F8 ? D : 2 * D;  // bytes per Q (and K) row
    const char* gq = (const char*)(map ? a.q2 : a.q1) + (size_t)bh * a.Nq * kQRow;
    const char* gk1 = (const char*)a.k1 + (size_t)bh * a.Nk * C::kKRow;
    const char* gk2 = (const char*)a.k2 + (size_t)bh * a.Nk * C::kKRow;
    const uint16_t* gv = (const uint16_t*)a.v + (size_t)bh * a.Nk * DV;
    __bf16* gout = (__bf16*)a.out + (size_t)bh * a.Nq * DV;

    const int wq0 = qt * C::kBr + qb * 32;  // first query row of this wave
    const int qrow = wq0 + l32;             // this lane's query row

    // Q fragments of the wave's map as B operands: column = query,
    // k-slots = channels 16kb + 8lh .. (bf16), or bytes 32 lh .. 32 lh + 31
    // of the row (e4m3: one k = 64 product covers d = 64)
    bf16x8 qf[F8 ? 1 : NKB];
    i32x8 qf8 = i32x8{};
    if constexpr (F8) {
        if (qrow < a.Nq) qf8 = *(const i32x8*)(gq + (size_t)qrow * kQRow + 32 * lh);
        qf[0] = bf16x8{};
    } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            qf[kb] = qrow < a.Nq ? *(const bf16x8*)(gq + (size_t)qrow * kQRow + 2 * (16 * kb + 8 * lh))
                                 : bf16x8{};
    }

    const int nkt_all = (a.Nk + kBc - 1) / kBc;
    const int nkt = CAUSAL ? min(nkt_all, (qt * C::kBr + C::kBr + kBc - 1) / kBc) : nkt_all;
    // leading tiles in which no row of this wave masks a key
    const int nfull = __builtin_amdgcn_readfirstlane(CAUSAL ? min(a.Nk / kBc, (wq0 + 1) / kBc) : a.Nk / kBc);

    // Tile loads go from global memory straight into the LDS ring
    // (buffer_load_dwordx4 ... lds: lane i of an instruction writes its 16
    // bytes at M0 + 16 i).  The tile's chunk positions, K1 then K2 then V, form
    // kChunks / 64 instructions; wave w issues instructions w, w + 8, ...  Each
    // lane loads the global chunk that belongs at its position under the
    // swizzle.  Regions start on instruction boundaries, so an instruction
    // reads one tensor; its descriptor ends at the last key, and lanes past
    // it write zeros.  With e4m3 K (64-byte rows) the K regions are 2 KB
    // each, which does not split into whole 16-byte instructions per wave:
    // there each wave loads one 1 KB group of V and 256 bytes of each K with
    // buffer_load_dword ... lds (lane i writes 4 bytes at M0 + 4 i), so every
    // wave issues the same three loads per tile.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // provably uniform copy
    // per instruction i of this wave: where its 64 lanes write in the stage
    // (bytes, lane 0; lane l writes 16 l or, for 4-byte loads, 4 l further),
    // which tensor it reads (0: K1, 1: K2, 2: V), and this lane's byte
    // offset in the tile of that tensor
    uint32_t m0_off[C::kLoads];
    int src[C::kLoads], ld_off[C::kLoads];
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
        if constexpr (F8) {
            if (i == 0) {  // V: chunk group wave_u
                const int pos = 64 * wave_u + lane;
                const int row = pos / (DV / 8);
                m0_off[i] = 2u * C::kVRing + 16u * 64u * (uint32_t)wave_u;
                src[i] = 2;
                ld_off[i] = row * DV * 2 + 16 * ((pos % (DV / 8)) ^ v_swz<DV>(row));
            } else {  // K1 (i = 1) or K2 (i = 2): 256 bytes, rows 4 wave_u ..
                const int row = 4 * wave_u + (lane >> 4);
                const int cp = (lane & 15) >> 2;  // chunk position in the row
                m0_off[i] = (uint32_t)((i - 1) * C::kKChunks * 16 + 256 * wave_u);
                src[i] = i - 1;
                ld_off[i] = row * C::kKRow + 16 * (cp ^ k_swz_rb<C::kKRow>(row)) + 4 * (lane & 3);
            }
        } else {
            const int c0 = 64 * (wave_u + i * (kThreads / 64));
            m0_off[i] = 16u * (uint32_t)c0;
            if (c0 < 2 * C::kKChunks) {
                constexpr int kCpr = C::kKRow / 16;  // chunks per K row
                const int pos = (c0 < C::kKChunks ? c0 : c0 - C::kKChunks) + lane;
                const int row = pos / kCpr;
                src[i] = c0 < C::kKChunks ? 0 : 1;
                ld_off[i] = row * C::kKRow + 16 * ((pos % kCpr) ^ k_swz_rb<C::kKRow>(row));
            } else {
                const int pos = c0 - 2 * C::kKChunks + lane;
                const int row = pos / (DV / 8);
                m0_off[i] = 2u * C::kVRing + 16u * (uint32_t)(c0 - 2 * C::kKChunks);
                src[i] = 2;
                ld_off[i] = row * DV * 2 + 16 * ((pos % (DV / 8)) ^ v_swz<DV>(row));
            }
        }
    }
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;  // LDS byte address
    auto stage_of = [](int kt) { return kt & (C::kStages - 1); };
    // FLAT: every tensor of the (batch, head) spans < 2 GiB, so one descriptor
    // per load instruction, built here, covers it and a tile is a byte offset
    // added to the lane offsets; otherwise each tile gets its own descriptor.
    i32x4 rs[C::kLoads];
    uint32_t tile_bytes[C::kLoads], region_bytes[C::kLoads];
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
        const bool in_k = src[i] < 2;
        const void* base = in_k ? (const void*)(src[i] == 0 ? gk1 : gk2) : (const void*)gv;
        const int row_bytes = in_k ? C::kKRow : DV * 2;
        const int64_t bytes = (int64_t)a.Nk * row_bytes;
        rs[i] = sgpr_rsrc(base, bytes);
        tile_bytes[i] = kBc * row_bytes;
        region_bytes[i] = FLAT ? (uint32_t)bytes : 0u;
    }
    static_assert(F8 || C::kKStage == C::kVStage, "bf16 loads share one stage stride");
    // tile kt into ring stage st (= kt mod kStages)
    auto issue_tile = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const uint32_t stride = 2u * (uint32_t)((F8 && i == 0) ? C::kVStage : C::kKStage);
            const uint32_t m0 =
                __builtin_amdgcn_readfirstlane(smem_base + m0_off[i] + (uint32_t)st * stride);
            const bool dw = F8 && i > 0;  // 4-byte load
            // Tiles past this workgroup's last one read out of range: the
            // instruction count per tile stays fixed (the waits count on it)
            // and the lanes just write zeros, without touching memory.
            int voff;
            i32x4 rsrc;
            if constexpr (FLAT) {
                const uint32_t toff = kt < nkt ? (uint32_t)kt * tile_bytes[i] : region_bytes[i];
                voff = ld_off[i] + (int)toff;
                rsrc = rs[i];
            } else {
                const int64_t key0 = (int64_t)kt * kBc;
                const int64_t left = kt < nkt ? (int64_t)a.Nk - key0 : 0;
                const bool in_k = src[i] < 2;
                const int row_bytes = in_k ? C::kKRow : DV * 2;
                const void* base = in_k ? (const void*)((src[i] == 0 ? gk1 : gk2) + key0 * C::kKRow)
                                        : (const void*)(gv + key0 * DV);
                voff = ld_off[i];
                rsrc = sgpr_rsrc(base, left * row_bytes);
            }
            if (dw)
                asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                             :
                             : "s"(m0), "v"(voff), "s"(rsrc)
                             : "memory", "m0");
            else
                asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                             :
                             : "s"(m0), "v"(voff), "s"(rsrc)
                             : "memory", "m0");
        }
    };
    // The loads above are invisible to the compiler's counters: before the
    // barrier that publishes tile t, each wave waits until at most N of its
    // own loads are still in flight (loads complete in order).
    auto wait_loads = [](auto n) {
        constexpr int N = decltype(n)::value;
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    };
    // at most T tiles' loads of this wave in flight
    auto wait_tiles = [&](auto t) {
        constexpr int T = decltype(t)::value;
        wait_loads(std::integral_constant<int, T * C::kLoads>{});
    };

    const int krow = swap23(l32);
    // this lane's pieces of the wave's K tile (A operand): row krow, chunk
    // 2 kb + lh under the swizzle, in bf16 elements from the stage start
    // (e4m3: bytes 32 lh .. 32 lh + 31 of the row, chunks 2 lh and 2 lh + 1)
    int k_off[F8 ? 2 : NKB];
#pragma unroll
    for (int kb = 0; kb < (F8 ? 2 : NKB); ++kb)
        k_off[kb] = map * C::kKElems + krow * (C::kKRow / 2) +
                    8 * ((F8 ? 2 * lh + kb : 2 * kb + lh) ^ k_swz_rb<C::kKRow>(krow));
    auto k_operand = [&](int buf, int kb) {
        return *(const bf16x8*)(smem + buf * C::kKStage + k_off[kb]);
    };
    // one score product: bf16 k = 16 step kb, or the whole e4m3 row (k = 64)
    auto score_mfma = [&](int buf, int kb, f32x16 c) {
        if constexpr (F8) {
            const bf16x8 lo = k_operand(buf, 0), hi = k_operand(buf, 1);
            const i32x8 ka8 = __builtin_bit_cast(
                i32x8, __builtin_shufflevector(__builtin_bit_cast(i32x4, lo),
                                               __builtin_bit_cast(i32x4, hi), 0, 1, 2, 3, 4, 5, 6, 7));
            return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka8, qf8, c, 0, 0, 0, 127, 0, 127);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(buf, kb), qf[kb], c, 0, 0, 0);
        }
    };
    auto scores = [&](int buf, f32x16& s) {
        s = f32x16{};
#pragma unroll
        for (int kb = 0; kb < NKS; ++kb) s = score_mfma(buf, kb, s);
    };

    // keys past the end, and keys after the query under the causal mask, to
    // -inf.  Register r holds key kt*kBc + 8 lh + idx(r), idx(r) = 16 (r/8) +
    // r%8, and a key is visible when it is at most the last key and (causal)
    // the query row: one bound per lane, one compare with a constant per
    // register.
    auto mask = [&](int kt, f32x16& s) {
        const int last = CAUSAL ? min(qrow, a.Nk - 1) : a.Nk - 1;
        const int lim = last - kt * kBc - 8 * lh;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 16 * (r >> 3) + (r & 7) <= lim ? s[r] : -INFINITY;
    };

    // per-lane pieces of the transposing V read: row e of 4 (e = (lane%16)/4,
    // plus 8 for the upper half-wave; further rows add multiples of 4, which
    // the swizzle does not see), channels 32 db + 16 (vg%2) + 4 (lane%4),
    // i.e. chunk 4 db + 2 (vg%2) + (lane%4)/2 and byte 8 (lane%2) in it
    const int vg = lane >> 4;
    const int ve = (lane & 15) >> 2;
    const int v_lane_row = C::kVRing + (8 * (vg >> 1) + ve) * DV + 4 * (lane & 1);  // 16-bit units
    int v_off[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        v_off[db] = v_lane_row + 8 * ((4 * db + 2 * (vg & 1) + ((lane & 3) >> 1)) ^ v_swz<DV>(ve));
    auto v_operand = [&](int buf, int db, int kb) {
        const uint16_t* vp = smem + buf * C::kVStage + v_off[db] + 16 * kb * DV;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)vp);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(vp + 4 * DV));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    const float sl2 = F8 ? a.scale_log2 * a.qk_scale[map] : a.scale_log2;
    float m, l = 0.f;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};

    // P.V of one tile (the last tile; inside the loop the same products are
    // spread over the issue slots)
    auto pv = [&](int buf, const bf16x8 (&p)[2]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(buf, db, kb), p[kb], o[db],
                                                                0, 0, 0);
        }
    };

    // Per-tile state, two copies used alternately (tile j in X[j % 2]): the
    // masked scores of the tile and, once formed, its probabilities.  In
    // iteration j the other copy still holds tile j-1's probabilities (read by
    // its P.V) and receives tile j+1's scores, so nothing is copied between
    // iterations and the new probabilities never have to wait for the
    // previous tile's products to be issued.
    struct TileState {
        f32x16 s;
        bf16x8 p[2];
    };
    TileState A, B;

    // prologue: tiles 0 .. kAhead-1 in flight; tiles 0, 1 and 2 complete (the
    // first barrier in the loop comes after iteration 1).  The
    // compiler waits for the Q loads before their first use by counting only
    // its own loads, which would also drain every tile load issued before that
    // use; so the Q fragments are taken (and waited for) right after tiles 0
    // and 1, which the first iteration needs anyway, and the rest follow.
    issue_tile(0, 0);
    issue_tile(1, 1);
    if constexpr (F8) {
        asm volatile("" ::"v"(qf8));
    } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) asm volatile("" ::"v"(qf[kb]));
    }
#pragma unroll
    for (int t0 = 2; t0 < C::kAhead; ++t0) issue_tile(t0, t0);
    wait_tiles(std::integral_constant<int, C::kAhead - 3>{});
    __syncthreads();
    scores(0, A.s);
    if (nfull < 1) mask(0, A.s);
    {
        // exact row maxima of tile 0 start the running maxima
        const float x = max16(A.s) * sl2;
        m = fmaxf(x, xor32(x));
    }
    // minus the exponent base: the running maximum, or 0 while it is -inf;
    // changes only where m does

    // Source order of one iteration: kSlots slots, each with one MFMA and a
    // share of the vector work (the compiler's scheduler takes it from there):
    //   slots 0 .. NKB-1     score products of tile j+1 (K operands read
    //                        before slot -1);
    //   slots NKB ..         P.V products of tile j-1, each V operand read
    //                        kLookahead products ahead;
    //   vector work          the 8 probability pairs of tile j, each in three
    //                        steps (scale, exp2, pack and sum) in consecutive
    //                        slots so that a slot's work is independent,
    //                        starting in a slot -1 that has no product;
    //   memory               the loads of tile j+5 (kAhead) in slot
    //                        kLoadSlot, late in the iteration: issued after
    //                        most of its LDS operand reads rather than among
    //                        them (slot 8 against slot 1, back to back on one
    //                        GPU: -1.6% and -2.4% on the 32K workload, -1.3%
    //                        on the 2K one).
    constexpr int kPairsV = 2 * NDB;  // V operands (db, kb)
    constexpr int kSlots = NKS + kPairsV;
    constexpr int kLookahead = 3;
    constexpr int kLoadSlot = kSlots > 8 ? 8 : kSlots - 1;
    // probability pair k (registers 2k, 2k+1) starts in slot pair_slot(k)
    auto pair_slot = [](int k) { return k * (kSlots - 3) / 8 - 1; };
    static_assert(7 * (kSlots - 3) / 8 - 1 + 2 < kSlots, "pairs must finish in the slots");

    // One iteration j (see the header); cur holds tile j, oth tile j-1 and
    // then j+1.  PREV: tile j-1 exists; NEXT: tile j+1 exists.
    // R: j mod kStages when known at compile time (stage offsets then fold into
    // the LDS instructions), else -1
    auto iteration = [&](auto res, auto prev, auto next, int j, TileState& cur, TileState& oth) {
        constexpr int R = decltype(res)::value;
        constexpr bool PREV = decltype(prev)::value;
        constexpr bool NEXT = decltype(next)::value;
        auto st = [&](int d) { return R >= 0 ? ((R + d) & (C::kStages - 1)) : stage_of(j + d); };
        const float nbase = -(m == -INFINITY ? 0.f : m);

        bf16x8 ka[F8 ? 2 : NKB], va[kPairsV];
        if constexpr (NEXT) {
#pragma unroll
            for (int kb = 0; kb < (F8 ? 2 : NKB); ++kb) ka[kb] = k_operand(st(1), kb);
        }
        const int vbuf = st(-1);
        if constexpr (PREV) {
#pragma unroll
            for (int q = 0; q < kLookahead; ++q) va[q] = v_operand(vbuf, q >> 1, q & 1);
        }
        float ta, tb;  // set by the first pair of each
        float xs[16];  // probabilities in flight, by accumulator register

#pragma unroll
        for (int slot = -1; slot < kSlots; ++slot) {
            if (slot < 0) {
                // no product: the first operands are still on their way
            } else if (slot < NKS) {
                if constexpr (NEXT) {
                    if constexpr (F8) {
                        const i32x8 ka8 = __builtin_bit_cast(
                            i32x8, __builtin_shufflevector(__builtin_bit_cast(i32x4, ka[0]),
                                                           __builtin_bit_cast(i32x4, ka[1]), 0, 1,
                                                           2, 3, 4, 5, 6, 7));
                        oth.s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            ka8, qf8, f32x16{}, 0, 0, 0, 127, 0, 127);
                        // keep it first: its result is the next iteration's
                        // first input (the scheduler would sink it to the end)
                        __builtin_amdgcn_sched_barrier(0);
                    } else {
                        oth.s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            ka[slot], qf[slot], slot == 0 ? f32x16{} : oth.s, 0, 0, 0);
                    }
                }
            } else {
                if constexpr (PREV) {
                    const int q = slot - NKS;
                    if (q + kLookahead < kPairsV)
                        va[q + kLookahead] =
                            v_operand(vbuf, (q + kLookahead) >> 1, (q + kLookahead) & 1);
                    o[q >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[q], oth.p[q & 1],
                                                                        o[q >> 1], 0, 0, 0);
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (pair_slot(k) == slot) {
                    xs[2 * k] = fmaf(cur.s[2 * k], sl2, nbase);
                    xs[2 * k + 1] = fmaf(cur.s[2 * k + 1], sl2, nbase);
                }
                if (pair_slot(k) + 1 == slot) {
                    xs[2 * k] = __builtin_amdgcn_exp2f(xs[2 * k]);
                    xs[2 * k + 1] = __builtin_amdgcn_exp2f(xs[2 * k + 1]);
                }
                if (pair_slot(k) + 2 == slot) {
                    if (k < 2)
                        pack_pair_first(cur.p, 2 * k, xs[2 * k], xs[2 * k + 1], (k & 1) ? tb : ta);
                    else
                        pack_pair(cur.p, 2 * k, xs[2 * k], xs[2 * k + 1], (k & 1) ? tb : ta);
                }
            }
            if (slot == kLoadSlot) issue_tile(j + C::kAhead, st(C::kAhead));  // zeros once past the end
        }
        // Keep the common-path probabilities ahead of the rare branch below
        // (which forms them again) rather than sunk into its other side.
        asm volatile("" ::"v"(cur.p[0]), "v"(cur.p[1]), "v"(ta), "v"(tb));

        // causal diagonal or ragged last tile: mask tile j+1 before its
        // probabilities are formed in the next iteration
        if constexpr (NEXT) {
            if (j + 1 >= nfull) mask(j + 1, oth.s);
        }
        // lazy-maximum test on tile j: a large partial sum means that some
        // scores passed the stale maximum; take the exact maxima of the tile,
        // rescale, and form its probabilities again
        float tsum = ta + tb;
        if (__builtin_amdgcn_ballot_w64(tsum > kSumLimit)) {
            const float x = max16(cur.s) * sl2;
            const float mn = fmaxf(m, fmaxf(x, xor32(x)));
            const float al = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
            m = mn;
            l *= al;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= al;
            const float nb = m == -INFINITY ? 0.f : m;
            tsum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 2) prob_pair(cur.s, e, sl2, nb, cur.p, tsum);
        }
        l += tsum;
        // a barrier after odd iterations only: tiles j+2 and j+3 (read by the
        // next two) must have landed; tiles j+4 .. j+kAhead may still be in flight
        const bool odd = R >= 0 ? (R & 1) : (j & 1);
        if (odd) {
            wait_tiles(std::integral_constant<int, C::kAhead - 3>{});
            __syncthreads();
        }
    };

    const bool_c<true> T;
    const bool_c<false> F;
    const std::integral_constant<int, -1> Rd;  // stage from j at run time
    auto Rs = [](auto r) { return std::integral_constant<int, decltype(r)::value>{}; };
    if (nkt == 1) {
        iteration(Rd, F, F, 0, A, B);
        pv(stage_of(0), A.p);
    } else {
        iteration(std::integral_constant<int, 0>{}, F, T, 0, A, B);
        // tile j lives in A for even j and in B for odd j; j = 1 mod kStages in
        // the unrolled loop, whose iterations are all followed by another
        int j = 1;
        static_assert(C::kStages == 8, "the unrolled loop covers one turn of the ring");
        for (; j + 7 < nkt - 1; j += 8) {
            iteration(Rs(std::integral_constant<int, 1>{}), T, T, j, B, A);
            iteration(Rs(std::integral_constant<int, 2>{}), T, T, j + 1, A, B);
            iteration(Rs(std::integral_constant<int, 3>{}), T, T, j + 2, B, A);
            iteration(Rs(std::integral_constant<int, 4>{}), T, T, j + 3, A, B);
            iteration(Rs(std::integral_constant<int, 5>{}), T, T, j + 4, B, A);
            iteration(Rs(std::integral_constant<int, 6>{}), T, T, j + 5, A, B);
            iteration(Rs(std::integral_constant<int, 7>{}), T, T, j + 6, B, A);
            iteration(Rs(std::integral_constant<int, 0>{}), T, T, j + 7, A, B);
        }
        for (; j + 1 < nkt - 1; j += 2) {
            iteration(Rd, T, T, j, B, A);
            iteration(Rd, T, T, j + 1, A, B);
        }
        if (j < nkt - 1) {
            iteration(Rd, T, T, j, B, A);
            iteration(Rd, T, F, j + 1, A, B);
            pv(stage_of(j + 1), A.p);
        } else {
            iteration(Rd, T, F, j, B, A);
            pv(stage_of(j), B.p);
        }
    }

    // epilogue: D = O1/l1 - lambda O2/l2, then GroupNorm over the dv channels
    // and the (1 - lambda_init) scale.  The two waves of a query block (one
    // per map) each finish half of the channels: the first map's wave the
    // accumulator blocks [0, NH), the lambda map's wave [NH, NDB).  Each sends
    // its scaled other half through LDS, forms D on its own half, and the
    // GroupNorm statistics are merged from the two halves' means and centred
    // sums of squares (pairwise merge of Chan, Golub and LeVeque).
    constexpr int NH = NDB / 2;
    const float L = l + xor32(l);
    // every wave is done with the tile ring, and no load (the last ones read
    // past the end and write zeros) may land on the epilogue's areas
    wait_tiles(std::integral_constant<int, 0>{});
    __syncthreads();
    const int other = map ^ 1;
    const float cs = map ? lam_h / L : 1.f / L;
    // exchange layout per (query block, receiving map): [db][g][lane] float4
    // holding registers 4g .. 4g+3 of block db, so each lane moves 16 bytes
    // per instruction and 16 lanes cover 256 contiguous bytes
    float* xchg = (float*)smem;
    // the map is wave-uniform: branch on it (a select would form both sides
    // of every element)
    const bool lambda_map = __builtin_amdgcn_readfirstlane(map) != 0;
    auto send = [&](auto h0) {  // blocks [H0, H0 + NH) go to the other wave
        constexpr int H0 = decltype(h0)::value;
        float* dst = xchg + (qb * 2 + other) * (NH * 16 * 64) + 4 * lane;
#pragma unroll
        for (int db = 0; db < NH; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16& src = o[H0 + db];
                *(float4*)(dst + (db * 4 + g) * 256) =
                    make_float4(product(src[4 * g], cs), product(src[4 * g + 1], cs),
                                product(src[4 * g + 2], cs), product(src[4 * g + 3], cs));
            }
        }
    };
    if (lambda_map)
        send(std::integral_constant<int, 0>{});
    else
        send(std::integral_constant<int, NH>{});
    __syncthreads();
    float x[NH][16];
    auto form = [&](auto lm) {  // D on the wave's own blocks
        constexpr bool LM = decltype(lm)::value;
        const float* src = xchg + (qb * 2 + (LM ? 1 : 0)) * (NH * 16 * 64) + 4 * lane;
#pragma unroll
        for (int db = 0; db < NH; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 got4 = *(const float4*)(src + (db * 4 + g) * 256);
                const float got[4] = {got4.x, got4.y, got4.z, got4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    x[db][r] = LM ? diff_of_products(got[e], 1.f, o[NH + db][r], cs)
                                  : diff_of_products(o[db][r], cs, got[e], 1.f);
                }
            }
        }
    };
    if (lambda_map)
        form(bool_c<true>{});
    else
        form(bool_c<false>{});
    if constexpr (SAVE) {
        // training forward: D before the normalisation, and each map's
        // log-sum-exp (m and l share the lazy maximum, so m + log2 l is exact)
        if (qrow < a.Nq) {
            float* drow = a.d_save + ((size_t)bh * a.Nq + qrow) * DV + map * (DV / 2);
#pragma unroll
            for (int db = 0; db < NH; ++db) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(float4*)(drow + 32 * db + 8 * g + 4 * lh) =
                        make_float4(x[db][4 * g], x[db][4 * g + 1], x[db][4 * g + 2], x[db][4 * g + 3]);
            }
            if (lh == 0)
                a.lse[((size_t)map * a.B * a.H + bh) * a.Nq + qrow] =
                    (m + __builtin_amdgcn_logf(L)) * 0.69314718055994531f;
        }
    }
    if (!(a.flags & 1u)) {
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NH; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) ps[r & 3] += x[db][r];
        }
        float hs = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        hs += xor32(hs);
        const float mh = hs * (2.f / DV);  // mean of this half of the row
        float pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NH; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float c = x[db][r] - mh;
                pq[r & 3] = fmaf(c, c, pq[r & 3]);
            }
        }
        float hq = (pq[0] + pq[1]) + (pq[2] + pq[3]);
        hq += xor32(hq);
        float2* stats = (float2*)(smem + C::kXchgElems);
        stats[(qb * 2 + map) * 64 + lane] = make_float2(mh, hq);
        __syncthreads();
        const float2 ot = stats[(qb * 2 + other) * 64 + lane];
        // both waves evaluate the same expressions in the same order
        const float mean = 0.5f * (mh + ot.x);
        const float dm = mh - ot.x;
        const float m2 = (hq + ot.y) + dm * dm * (0.25f * DV);
        const float var = m2 * (1.f / DV);
        const float scale = (1.f - a.lambda_init) / sqrtf(var + a.eps);
#pragma unroll
        for (int db = 0; db < NH; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[db][r] = (x[db][r] - mean) * scale;
        }
    }

    // Output: the wave's 32 rows by DV/2 channels go through LDS (bf16, rows
    // of kCpr 16-byte chunks, chunk index swizzled by the row's 256-byte line)
    // so that each store instruction writes whole row segments.
    {
        constexpr int kCpr = DV / 16;       // chunks per half row
        constexpr int kRpl = 256 / DV;      // half rows per 256 bytes
        uint16_t* so = smem + C::kXchgElems + C::kStatElems + wave * (32 * (DV / 2));
        const int swr = (l32 / kRpl) % kCpr;
#pragma unroll
        for (int db = 0; db < NH; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)x[db][4 * g + e];
                *(bf16x4*)(so + l32 * (DV / 2) + 8 * ((4 * db + g) ^ swr) + 4 * lh) = w;
            }
        }
        constexpr int kRowsPerStore = 64 / kCpr;
        __bf16* gbase = gout + (size_t)wq0 * DV + map * (DV / 2);
#pragma unroll
        for (int k = 0; k < 32 / kRowsPerStore; ++k) {
            const int row = k * kRowsPerStore + lane / kCpr;
            const int ch = lane % kCpr;
            const uint4 w = *(const uint4*)(so + row * (DV / 2) + 8 * (ch ^ ((row / kRpl) % kCpr)));
            if (wq0 + row < a.Nq) *(uint4*)(gbase + (size_t)row * DV + 8 * ch) = w;
        }
    }
    __syncthreads();  // the LDS ring and exchange area are reused by the next item
    }
}

}  // namespace
}  // namespace diffattn
