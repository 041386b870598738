// dQ and dK/dV kernels of the Differential Attention backward for head_dim
// 128 and v_dim 256 on gfx950 (CDNA4).
//
// The chain rule is that of backward.hip (the pages' operator: iloveeagents.com,
// "Mathematical Formula", lambda learnable; llmbytes.dev, "How Differential
// Attention Cancels Common-Mode Noise", step 4), with tau = 1/sqrt(d):
//   dP = dD V^T,  delta_k = rowsum(A_k * dP),
//   dS_1 = A_1 (dP - delta_1),  dS_2 = -lambda A_2 (dP - delta_2),
//   dQ_k = tau dS_k K_k,  dK_k = tau dS_k^T Q_k,  dV = (A_1 - lambda A_2)^T dD.
// A_k = exp(S_k tau - lse_k) from the training forward's log-sum-exp.
//
// Why kernels of their own.  At head_dim 128 the resident operands of a
// wave (Q or K columns over d, dD or V columns over dv) and its accumulators
// outgrow the head_dim-64 kernels' register budget.
//
//   dq    workgroup = 128 query rows of one (batch, head), 8 waves, wave w
//         rows 32 (w mod 4) .. of map w / 4, two waves per SIMD.  Sweeps the
//         key tiles twice.  Per tile, both sweeps: S^T = K Q^T (8 products)
//         and dP^T over the wave's half of the dv channels (8), the two
//         halves added through LDS; sweep 1 sums delta = rowsum(A * dP),
//         sweep 2 forms dS = A (dP - delta) in fp32 and accumulates
//         dQ^T += K^T dS^T (8).  Writes dQ_k, delta_k and the row terms of
//         the dK/dV kernel.
//   dkdv  workgroup = 128 keys, wave w keys 32 w .. of both maps, one wave
//         per SIMD: 128 registers of resident K1^T, K2^T, V^T and 256 of
//         accumulators (dV over 256 channels, both dK_k) in the AGPRs.  Per
//         query tile: S_k = Q_k K_k^T (2 x 8), dP = dD V^T (16),
//         dV^T += dD^T W with W = A_1 - lambda A_2 (16), dK_k^T += Q_k^T dS_k
//         (2 x 8).
//
// Tiles of 32 rows stream through a 3- or 4-stage LDS ring, two or three
// tiles ahead, by buffer loads with the LDS destination (no registers, no
// LDS stores).  Each
// tile is read both as rows (16-byte reads: the A operand of the score and
// dP products, rows in swap23 order so that score accumulators are the next
// product's B operands) and as columns (ds_read_b64_tr_b16: the transposed
// A operand of the dQ, dV and dK products).  One XOR swizzle of a row's
// 16-byte chunks serves both: chunk c of row r sits at position
// c ^ (4 (r mod 4) + (r / 4) mod 4), which puts the 16 rows of a row read
// and the 4 rows x 4 chunks of a transposing read on 64 distinct banks.

#include "internal.h"
#include "tile_ops.h"

#include <math.h>

// The direct-to-LDS loads set M0 in inline asm; nothing else in this file
// uses M0, so the reserved-register clobber is safe here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace diffattn {
namespace {

using namespace tile;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128, kDV = 256;
constexpr int kKRow = 2 * kD;      // bytes per Q or K row
constexpr int kVRow = 2 * kDV;     // bytes per V or dD row
constexpr int kNKB = kD / 16;      // k = 16 steps over d
constexpr int kNVB = kDV / 16;     // k = 16 steps over dv
constexpr int kNCB = kD / 32;      // 32-row blocks of d
constexpr int kNDB = kDV / 32;     // 32-row blocks of dv
constexpr int kKTile = 32 * kKRow;  // 8 KB
constexpr int kVTile = 32 * kVRow;  // 16 KB
constexpr int kStages = 4;
constexpr int kRowsWG = 128;        // rows (dq) or keys (dkdv) of a workgroup
constexpr int kTileLoads = (2 * kKTile + kVTile) / (16 * kBwdThreads);  // per wave and tile
constexpr int kStage = 2 * kKTile + kVTile;  // 32 KB: X1 | X2 | Y tiles

constexpr int kRowSlot = 1024;      // a wave's copy of a tile's row terms (dK/dV)
constexpr int kRowStage = 4 * kRowSlot;
static_assert(kStage == 32 * 1024, "stage bases must leave the in-tile address bits free");
constexpr int kBufferDword3 = 0x00020000;

static_assert(kTileLoads * 16 * kBwdThreads == 2 * kKTile + kVTile, "whole loads per wave");
static_assert(kKTile % (16 * kBwdThreads) == 0, "a load instruction stays in one tile");

__device__ __forceinline__ int rswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// The swizzle by row length: rows of 256 or 512 bytes use rswz on the low 4
// bits of the chunk index; 128-byte rows (head_dim 64 tiles of Q and K, two
// rows per pass over the banks) use c ^ (4 ((r / 2) mod 2) + (r / 4) mod 4),
// which puts the 16 rows of a row read and the 4 rows x 4 chunks of a
// transposed read on distinct banks the same way.
template <int RB>
__device__ __forceinline__ int swz(int r) {
    if constexpr (RB == 128)
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else
        return rswz(r);
}

// LDS addressing.  Every tile sits at a fixed offset in its ring stage and a
// stage's base is a multiple of 32 KB, while a read's address within a tile
// is below 16 KB, so the address of a read is
//     (lane base | stage base) ^ (bits of the k step or column block)
// plus an immediate (the tile, the k step of a transposed read): the swizzle
// is an XOR on the chunk index, and the bits a read's position adds to the
// lane's own are disjoint from the lane's row bits.  One instruction per read
// and no register per read; the per-tile base goes through an empty asm so
// that the compiler forms each address from it rather than keeping one
// register per (read, lane) across the loop.

// Row reads (A operand rows, 16 bytes at elements k0 + 8 lh of row `row`):
// lane base for RB-byte rows; the read of k step kb (k0 = 16 kb) is at
// base ^ (32 kb).
template <int RB>
__device__ __forceinline__ int row_base(int row, int lh) {
    return row * RB + 16 * (lh ^ swz<RB>(row));
}

// Transposed reads (A operand column cb + l32 over rows k0 + 8 lh .. + 7,
// two ds_read_b64_tr_b16 of rows +0..3 and +4..7): lane base of the first
// for RB-byte rows; the read of column block cbk (cb = 32 cbk) and rows
// k0 = 16 kk is at (base ^ (64 cbk)) + 16 kk RB.  Within a 16-lane group,
// lane 4e + r addresses row e at column base + 4r and receives column
// base + (lane % 16) of the 4 rows.
template <int RB>
__device__ __forceinline__ int col_base(int lane) {
    const int g = lane >> 4, e = (lane & 15) >> 2, r = lane & 3;
    const int w = 2 * (g & 1) + (r >> 1), z = 2 * (g >> 1);
    // (128-byte rows: the swizzle's bit 2 comes from (row / 2) mod 2 = e / 2)
    return (8 * (g >> 1) + e) * RB + 64 * (RB == 128 ? e >> 1 : e) + 16 * (w ^ z) + 8 * (r & 1);
}

__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int IMM>
__device__ __forceinline__ bf16x8 lds_row(const uint8_t* smem, int addr) {
    return *(const bf16x8*)(smem + addr + IMM);
}

// The half-1 base of a transposed read is the half-0 base four rows on with
// bit 4 flipped (z and hence w ^ z differ in bit 0): a1 = (a0 ^ 16) + 4 RB.
template <int RB, int IMM>
__device__ __forceinline__ bf16x8 lds_col(const uint8_t* smem, int a0) {
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_u8*)(smem + a0 + IMM));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(lds_u8*)(smem + (a0 ^ 16) + 4 * RB + IMM));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Raw buffer descriptor of `bytes` bytes from `base` (wave-uniform): loads
// past the end return zeros and touch no memory.
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

// 16 bytes per lane from global memory to LDS at m0 + 16 lane
__device__ __forceinline__ void load_lds(uint32_t m0, int voff, i32x4 rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// acc += a b with the accumulator held in AGPRs for the whole sweep.  The
// compiler's builtin may place (and move) an accumulator in either register
// file; with 256 accumulator registers per wave that costs copies and
// spills, so these products are written out.  Two hazards are the code's own
// to cover, since the compiler does not look into the statement: an operand
// written by a vector instruction needs 2 wait states before the product
// reads it (the leading s_nop 1), and the accumulators are read back only
// after settle().  Not volatile: the data dependencies order the products
// of one accumulator, and the scheduler may move LDS reads and vector work
// across them.
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// After the last mfma_acc: each accumulator passes through a statement that
// waits out the products' latency (at most 16 passes) before any other
// instruction reads it; taking the accumulator as an operand orders it after
// that accumulator's last product.
template <int N>
__device__ __forceinline__ void settle(f32x16 (&acc)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+a"(acc[i]));
}

// Work item of workgroup w in a grid of n tiles per (batch, head) times BH:
// sets the tile rank t (0 = the longest causal tile) and bh.  Workgroups are
// dispatched round-robin over the 8 XCDs (w runs on XCD w mod 8), each with
// its own L2.  When BH is a multiple of 8, XCD x takes the heads
// bh = x mod 8 one after the other (the grid's w / 8-th item of that XCD is
// tile (w / 8) mod n of its (w / 8) / n-th head): the XCD's compute units
// sweep the same head's tiles at the same time, and each tile they share comes
// from HBM into that L2 about once.  Else tile-major over all heads.
__device__ __forceinline__ void xcd_item(int w, int n, int BH, int& t, int& bh) {
    if ((BH & 7) == 0) {
        const int i = w >> 3, hl = i / n;
        t = i - hl * n;
        bh = 8 * hl + (w & 7);
    } else {
        t = w / BH;
        bh = w - t * BH;
    }
}

template <int N>
__device__ __forceinline__ void wait_loads() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 32-row tile of the two 128-wide tensors X1, X2 ([n][128] bf16) and
// the 256-wide Y ([n][256] bf16) into a ring stage laid out X1 | X2 | Y.
// Load instruction i of wave w fills chunk positions 256 i + 64 w .. + 63 of
// the stage (i < 2: X1, i < 4: X2, else Y); each lane fetches the chunk that
// the swizzle puts at its position.  Worked out, the source offsets of a
// lane are one X offset (instruction i = 1 and 3 add 16 rows, 4096 bytes)
// and one Y offset XORed with a wave-uniform 16 ((2 (i - 4) + w / 2) mod 4)
// (instruction i >= 4 starts 8 (i - 4) rows, 4096 (i - 4) bytes, further):
// two registers per lane.
struct TileFeed {
    int offx, offy;
    __device__ __forceinline__ void init(int wave, int lane) {
        const int lh = lane >> 5;
        const int xr = 4 * wave + (lane >> 4);  // row of instruction 0
        offx = xr * kKRow + 16 * ((lane & 15) ^ rswz(xr));
        const int yr = 2 * wave + lh;  // row of instruction 4
        offy = yr * kVRow + 16 * ((lane & 31) ^ (4 * (yr & 3)));
    }
    // rows row0 .. row0 + 31 of tensors with n rows
    __device__ __forceinline__ void issue(uint32_t stage, int wave, const uint8_t* x1,
                                          const uint8_t* x2, const uint8_t* y, int64_t row0,
                                          int64_t n) const {
        const int64_t left = n - row0;
        const i32x4 r1 = sgpr_rsrc(x1 + row0 * kKRow, left * kKRow);
        const i32x4 r2 = sgpr_rsrc(x2 + row0 * kKRow, left * kKRow);
        const i32x4 ry = sgpr_rsrc(y + row0 * kVRow, left * kVRow);
#pragma unroll
        for (int i = 0; i < kTileLoads; ++i) {
            const uint32_t m0 =
                __builtin_amdgcn_readfirstlane(stage + (uint32_t)(16 * (256 * i + 64 * wave)));
            // (the row steps go into the per-lane offset, which the
            // descriptor's range check covers)
            if (i < 4) {
                load_lds(m0, offx + (i & 1) * 16 * kKRow, i < 2 ? r1 : r2);
            } else {
                const int b = 16 * ((2 * (i - 4) + (wave >> 1)) & 3);
                load_lds(m0, (offy ^ b) + (i - 4) * 8 * kVRow, ry);
            }
        }
    }
    // The same with one descriptor per tensor for the whole (batch, head)
    // slice (under 2 GiB): tile t's rows start t kKTile / t kVTile bytes in,
    // added to the per-lane offset; t < 0 loads zeros (offsets past the end).
    __device__ __forceinline__ void issue_flat(uint32_t stage, int wave, const i32x4& r1,
                                               const i32x4& r2, const i32x4& ry, int t,
                                               int xend, int yend) const {
        const int xo = t >= 0 ? t * (32 * kKRow) : xend;
        const int yo = t >= 0 ? t * (32 * kVRow) : yend;
#pragma unroll
        for (int i = 0; i < kTileLoads; ++i) {
            const uint32_t m0 =
                __builtin_amdgcn_readfirstlane(stage + (uint32_t)(16 * (256 * i + 64 * wave)));
            if (i < 4) {
                load_lds(m0, offx + (i & 1) * 16 * kKRow + xo, i < 2 ? r1 : r2);
            } else {
                const int b = 16 * ((2 * (i - 4) + (wave >> 1)) & 3);
                load_lds(m0, (offy ^ b) + (i - 4) * 8 * kVRow + yo, ry);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// dQ_1, dQ_2, delta_1, delta_2 and the row terms
// ---------------------------------------------------------------------------
constexpr int kDqThreads = 512;  // 8 waves: 4 query blocks x 2 maps, two per SIMD
constexpr int kDqStages = 3;
constexpr int kXSlot = 64 * 16 * 4;  // a wave's 16 floats per lane

template <int D, int DV>
struct DqCfg {
    static constexpr int kKRow = 2 * D, kVRow = 2 * DV;  // bytes per row
    static constexpr int kKTile = 32 * kKRow, kVTile = 32 * kVRow;
    static constexpr int kStage = 2 * kKTile + kVTile;   // K1 | K2 | V
    static constexpr int kLoads = kStage / (16 * kDqThreads);
    static constexpr int kKChunks = kKTile / 16;
    static constexpr int kNKB = D / 16;                  // score products per tile
    static constexpr int kNVH = DV / 32;                 // dP products over half of dv
    static constexpr int kNCB = D / 32;                  // 32-row blocks of dQ^T
    static constexpr int kSmem = kDqStages * kStage + 8 * kXSlot;
    static_assert(kLoads * 16 * kDqThreads == kStage, "whole loads per wave");
    static_assert(kKChunks % 64 == 0, "a load instruction stays in one tile");
    static_assert((kStage & (kStage - 1)) == 0 && kStage >= 2 * kVTile,
                  "stage bases must leave the in-tile address bits free");
};

// One tile (K1 | K2 | V, 32 rows each) into a ring stage with 8 waves: load
// instruction i of wave w fills chunk positions 512 i + 64 w .. + 63, which
// lie in one of the three tiles (a wave-uniform choice of descriptor), each
// lane fetching the chunk the swizzle puts at its position.
template <int D, int DV>
struct TileFeed8 {
    using C = DqCfg<D, DV>;
    int off[C::kLoads];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const int p = 512 * i + 64 * wave + lane;
            if (p < 2 * C::kKChunks) {
                constexpr int cpr = C::kKRow / 16;
                const int q = p % C::kKChunks, row = q / cpr;
                off[i] = row * C::kKRow + 16 * ((q % cpr) ^ swz<C::kKRow>(row));
            } else {
                constexpr int cpr = C::kVRow / 16;
                const int q = p - 2 * C::kKChunks, row = q / cpr;
                off[i] = row * C::kVRow + 16 * ((q % cpr) ^ swz<C::kVRow>(row));
            }
        }
    }
    __device__ __forceinline__ void issue(uint32_t stage, int wave, const uint8_t* k1,
                                          const uint8_t* k2, const uint8_t* v, int64_t row0,
                                          int64_t n) const {
        const int64_t left = n - row0;
        const i32x4 r1 = sgpr_rsrc(k1 + row0 * C::kKRow, left * C::kKRow);
        const i32x4 r2 = sgpr_rsrc(k2 + row0 * C::kKRow, left * C::kKRow);
        const i32x4 rv = sgpr_rsrc(v + row0 * C::kVRow, left * C::kVRow);
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const int p0 = 512 * i + 64 * wave;  // wave-uniform
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + (uint32_t)(16 * p0));
            load_lds(m0, off[i], p0 < C::kKChunks ? r1 : (p0 < 2 * C::kKChunks ? r2 : rv));
        }
    }
    // one descriptor per tensor for the whole slice (see TileFeed::issue_flat)
    __device__ __forceinline__ void issue_flat(uint32_t stage, int wave, const i32x4& r1,
                                               const i32x4& r2, const i32x4& rv, int t,
                                               int kend, int vend) const {
        const int ko = t >= 0 ? t * C::kKTile : kend;
        const int vo = t >= 0 ? t * C::kVTile : vend;
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const int p0 = 512 * i + 64 * wave;  // wave-uniform
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + (uint32_t)(16 * p0));
            if (p0 < 2 * C::kKChunks)
                load_lds(m0, off[i] + ko, p0 < C::kKChunks ? r1 : r2);
            else
                load_lds(m0, off[i] + vo, rv);
        }
    }
};

// Workgroup = 128 query rows of one (batch, head); wave w owns rows
// 32 (w mod 4) .. and map w / 4.  Two sweeps over the key tiles (delta first,
// then dQ; see the file comment).  Per tile each wave forms its map's scores
// S^T = K Q^T (d/16 products) and dP^T over its map's half of the dv
// channels (dv/32), and the two waves of a query block add their halves
// through LDS: both compute own + partner, and fp32 addition commutes, so
// they hold the same dP.  Sweep 2 adds dQ^T += K^T dS^T (d/16 products).
template <int D, int DV, bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kDqThreads) void bwd_dq_pair_kernel(BackwardArgs a) {
    using C = DqCfg<D, DV>;
    constexpr int kKRow = C::kKRow, kVRow = C::kVRow, kKTile = C::kKTile, kStage = C::kStage;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int l32 = lane & 31, lh = lane >> 5;
    const int qb = wave & 3, map = wave >> 2;
    const int BH = a.B * a.H;
    const int nqt = (a.Nq + kRowsWG - 1) / kRowsWG;
    int t, bh;  // longest causal tiles first
    xcd_item(blockIdx.x, nqt, BH, t, bh);
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int h = bh % a.H;
    const int qw0 = qt * kRowsWG + 32 * qb;
    const int qrow = qw0 + l32;
    const bool qok = qrow < a.Nq;

    const uint8_t* gq = (const uint8_t*)(map ? a.q2 : a.q1) + (size_t)bh * a.Nq * kKRow;
    const uint8_t* gk1 = (const uint8_t*)a.k1 + (size_t)bh * a.Nk * kKRow;
    const uint8_t* gk2 = (const uint8_t*)a.k2 + (size_t)bh * a.Nk * kKRow;
    const uint8_t* gv = (const uint8_t*)a.v + (size_t)bh * a.Nk * kVRow;
    const uint8_t* gdd = (const uint8_t*)a.dd + (size_t)bh * a.Nq * kVRow;

    // B operands of this lane's query (column l32): Q^T of the wave's map over
    // d, dD^T over the map's half of dv (channels dv/2 map ..)
    bf16x8 qf[C::kNKB], df[C::kNVH];
#pragma unroll
    for (int kb = 0; kb < C::kNKB; ++kb)
        qf[kb] = qok ? *(const bf16x8*)(gq + (size_t)qrow * kKRow + 2 * (16 * kb + 8 * lh))
                     : bf16x8{};
#pragma unroll
    for (int c = 0; c < C::kNVH; ++c)
        df[c] = qok ? *(const bf16x8*)(gdd + (size_t)qrow * kVRow +
                                       2 * (DV / 2 * map + 16 * c + 8 * lh))
                    : bf16x8{};
    // keys visible to this lane's query: 0 .. key_end - 1
    const int key_end = qok ? (CAUSAL ? min(a.Nk, qrow + 1) : a.Nk) : 0;
    const float lse = qok ? a.lse[((size_t)map * BH + bh) * a.Nq + qrow] * kLog2e : 0.f;
    const float sl2 = a.scale_log2;
    // The compiler counts only its own loads when it waits for these, so a
    // first use inside the loop would wait for the ring's loads as well (on
    // every tile).  Used here, before the ring starts, they are complete.
#pragma unroll
    for (int kb = 0; kb < C::kNKB; ++kb) asm volatile("" ::"v"(qf[kb]));
#pragma unroll
    for (int c = 0; c < C::kNVH; ++c) asm volatile("" ::"v"(df[c]));
    asm volatile("" ::"v"(lse));

    f32x16 dq[C::kNCB];
#pragma unroll
    for (int cb = 0; cb < C::kNCB; ++cb) dq[cb] = f32x16{};
    float dsum = 0.f;

    const int nkt_all = (a.Nk + 31) / 32;
    const int nkt = CAUSAL ? min(nkt_all, (qt * kRowsWG + kRowsWG + 31) / 32) : nkt_all;
    // key tiles in which some key is visible to some row of this query block
    const int nkt_w = CAUSAL ? min(nkt, (qw0 + 31) / 32 + 1) : nkt;
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    TileFeed8<D, DV> feed;
    feed.init(wave, lane);
    // The key tiles are swept twice, as one sequence of 2 nkt ring entries:
    // entry g is key tile g mod nkt, in ring stage g mod 3.  Entries past the
    // sequence load zeros (a fixed count per iteration for the waits).
    // (FLAT: one descriptor per tensor for the (batch, head) slice)
    const int kbytes = FLAT ? a.Nk * kKRow : 0, vbytes = FLAT ? a.Nk * kVRow : 0;
    const i32x4 rk1 = sgpr_rsrc(gk1, kbytes), rk2 = sgpr_rsrc(gk2, kbytes);
    const i32x4 rv = sgpr_rsrc(gv, vbytes);
    auto issue = [&](int g, int st) {
        const int kt = g < nkt ? g : g - nkt;
        if constexpr (FLAT)
            feed.issue_flat(smem_base + (uint32_t)(st * kStage), wave, rk1, rk2, rv,
                            g < 2 * nkt ? kt : -1, kbytes, vbytes);
        else
            feed.issue(smem_base + (uint32_t)(st * kStage), wave, gk1, gk2, gv, (int64_t)kt * 32,
                       g < 2 * nkt ? (int64_t)a.Nk : 0);
    };
    issue(0, 0);
    issue(1, 1);
    int st = 0, g = 0;  // ring stage and sequence index of the next entry
    // next(): waits for entry g and returns its stage base; refill(): loads
    // entry g + 2 into the stage entry g - 1 used.  The refill comes after the
    // tile's score and dP products: its loads, which the compiler may not
    // move LDS reads across, then no longer hold back that step's operand
    // reads (measured back to back on one GPU: 11.76 -> 11.35 ms for the
    // backward with the same change in the dK/dV kernel).
    int pend_g = 0, pend_st = 0;
    auto refill = [&]() { issue(pend_g, pend_st); };
    auto next = [&]() {
        wait_loads<C::kLoads>();
        __syncthreads();
        pend_g = g + 2;
        pend_st = st == 0 ? 2 : st - 1;
        const int sb = st * kStage;
        st = st == 2 ? 0 : st + 1;
        ++g;
        return sb;
    };
    const int kr = swap23(l32);
    // the wave's map selects the K tile (K2 is kKTile on) and the half of
    // each V row (the swizzle may move a chunk across the halves: an XOR)
    const int yk = row_base<kKRow>(kr, lh) | (map * kKTile);
    const int yv = row_base<kVRow>(kr, lh) ^ (map * (kVRow / 2));
    const int yc = col_base<kKRow>(lane) | (map * kKTile);
    const int x_own = kDqStages * kStage + kXSlot * wave;
    const int x_oth = kDqStages * kStage + kXSlot * (wave ^ 4);

    // S^T = K Q^T and this map's half of dP^T = V dD^T, entry in stage sb
    auto scores = [&](int sb, f32x16& s, f32x16& dph) {
        const int ykt = opaque(yk | sb), yvt = opaque(yv | sb);
        s = dph = f32x16{};
#pragma unroll
        for (int kb = 0; kb < C::kNKB; ++kb) s = mfma(lds_row<0>(smem, ykt ^ (32 * kb)), qf[kb], s);
#pragma unroll
        for (int c = 0; c < C::kNVH; ++c)
            dph = mfma(lds_row<2 * kKTile>(smem, yvt ^ (32 * c)), df[c], dph);
    };
    // dP = own half + partner's half (the barrier between writing and reading
    // is the second of the iteration; the next iteration's first one keeps the
    // partner's read ahead of this wave's next write)
    auto exchange = [&](const f32x16& own) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(float4*)(smem + x_own + 1024 * i + 16 * lane) =
                make_float4(own[4 * i], own[4 * i + 1], own[4 * i + 2], own[4 * i + 3]);
        __syncthreads();
        f32x16 dp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 o = *(const float4*)(smem + x_oth + 1024 * i + 16 * lane);
            dp[4 * i] = own[4 * i] + o.x;
            dp[4 * i + 1] = own[4 * i + 1] + o.y;
            dp[4 * i + 2] = own[4 * i + 2] + o.z;
            dp[4 * i + 3] = own[4 * i + 3] + o.w;
        }
        return dp;
    };
    // A of register r (key kt 32 + 8 lh + 16 (r / 8) + r % 8); edge tiles
    // mask keys at offset >= lim from the lane's first key (min with -inf
    // rather than a select, formed on every lane)
    auto probs = [&](const f32x16& s, int kt, float (&p)[16]) {
        const bool full = qw0 + 31 < a.Nq && kt * 32 + 31 < a.Nk && (!CAUSAL || kt * 32 + 31 <= qw0);
        if (full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse));
        } else {
            const int lim = key_end - kt * 32 - 8 * lh;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float cap = 16 * (r >> 3) + (r & 7) < lim ? INFINITY : -INFINITY;
                p[r] = __builtin_amdgcn_exp2f(fminf(fmaf(s[r], sl2, -lse), cap));
            }
        }
    };

    // ---- sweep 1: delta = rowsum(A * dP), from the same products as sweep
    // 2's dP, so that dP - delta is formed exactly there.  (dQ as
    // tau (X - delta Y) in one sweep, X = K^T (A * dP) and Y = K^T A, loses
    // it: when A is nearly one-hot, delta is nearly the dominant key's dP and
    // X and delta Y are large and nearly equal, so the bf16 rounding of their
    // factors survives the difference.)  Tiles kt >= nkt_w mask every key of
    // the query block: its waves only keep the ring and the barriers going
    // there (loops of their own, so that the compute loops have one path).
    for (int kt = 0; kt < nkt_w; ++kt) {
        const int sb = next();
        f32x16 s, dph;
        scores(sb, s, dph);
        refill();
        float p[16];
        probs(s, kt, p);
        const f32x16 dp = exchange(dph);
#pragma unroll
        for (int r = 0; r < 16; ++r) dsum = fmaf(p[r], dp[r], dsum);
    }
    for (int kt = nkt_w; kt < nkt; ++kt) {
        next();
        refill();
        __syncthreads();
    }
    const float delta = dsum + __shfl_xor(dsum, 32);

    // ---- sweep 2: dQ^T += K^T dS^T with dS = A (dP - delta) (the factor
    // -lambda of map 2 and tau are applied at the end)
    for (int kt = 0; kt < nkt_w; ++kt) {
        const int sb = next();
        f32x16 s, dph;
        scores(sb, s, dph);
        refill();
        float p[16];
        probs(s, kt, p);
        const f32x16 dp = exchange(dph);
        float gr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) gr[r] = p[r] * (dp[r] - delta);
        bf16x8 pg[2];
        pack(gr, pg);
        const int yct = opaque(yc | sb);
#pragma unroll
        for (int cb = 0; cb < C::kNCB; ++cb) {
            const int a0 = yct ^ (64 * cb);
            dq[cb] = mfma(lds_col<kKRow, 0>(smem, a0), pg[0], dq[cb]);
            dq[cb] = mfma(lds_col<kKRow, 16 * kKRow>(smem, a0), pg[1], dq[cb]);
        }
    }
    for (int kt = nkt_w; kt < nkt; ++kt) {
        next();
        refill();
        __syncthreads();
    }
    wait_loads<0>();  // the zero-filling loads past the end land before exit

    if (!qok) return;
    const float tau = 1.f / sqrtf((float)D);
    const float sc = map ? -a.lam[h] * tau : tau;
    __bf16* o = (__bf16*)(map ? a.dq2 : a.dq1) + ((size_t)bh * a.Nq + qrow) * D;
#pragma unroll
    for (int cb = 0; cb < C::kNCB; ++cb) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(sc * dq[cb][4 * gq + e]);
            *(bf16x4*)(o + 32 * cb + 8 * gq + 4 * lh) = v;
        }
    }
    if (lh == 0) {
        a.delta[((size_t)map * BH + bh) * a.Nq + qrow] = delta;
        // row terms (lse_1, delta_1, lse_2, delta_2): this map's pair
        *(float2*)(a.rows + 4 * ((size_t)bh * a.Nq + qrow) + 2 * map) = make_float2(lse, delta);
    }
}

// ---------------------------------------------------------------------------
// dK_1, dK_2, dV
// ---------------------------------------------------------------------------
template <bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_ring_kernel(BackwardArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * (kStage + kRowStage)];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int BH = a.B * a.H;
    // key tile kt = blockIdx / BH: under the causal mask the first key tiles
    // see the most queries, so the longest workgroups start first
    int kt, bh;
    xcd_item(blockIdx.x, (a.Nk + kRowsWG - 1) / kRowsWG, BH, kt, bh);
    const int h = bh % a.H;
    const int kw0 = __builtin_amdgcn_readfirstlane(kt * kRowsWG + 32 * wave_u);
    const int key = kw0 + l32;
    const bool kok = key < a.Nk;

    const uint8_t* gk1 = (const uint8_t*)a.k1 + (size_t)bh * a.Nk * kKRow;
    const uint8_t* gk2 = (const uint8_t*)a.k2 + (size_t)bh * a.Nk * kKRow;
    const uint8_t* gv = (const uint8_t*)a.v + (size_t)bh * a.Nk * kVRow;
    const uint8_t* gq1 = (const uint8_t*)a.q1 + (size_t)bh * a.Nq * kKRow;
    const uint8_t* gq2 = (const uint8_t*)a.q2 + (size_t)bh * a.Nq * kKRow;
    const uint8_t* gdd = (const uint8_t*)a.dd + (size_t)bh * a.Nq * kVRow;
    const uint8_t* grows = (const uint8_t*)a.rows + (size_t)bh * a.Nq * 16;

    // B operands of this lane's key (column l32): K_k^T over d, V^T over dv
    bf16x8 k1f[kNKB], k2f[kNKB], vf[kNVB];
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) {
        const size_t o = (size_t)key * kKRow + 2 * (16 * kb + 8 * lh);
        k1f[kb] = kok ? *(const bf16x8*)(gk1 + o) : bf16x8{};
        k2f[kb] = kok ? *(const bf16x8*)(gk2 + o) : bf16x8{};
    }
#pragma unroll
    for (int c = 0; c < kNVB; ++c)
        vf[c] = kok ? *(const bf16x8*)(gv + (size_t)key * kVRow + 2 * (16 * c + 8 * lh))
                    : bf16x8{};
    const float sl2 = a.scale_log2;
    const float lam = a.lam[h];
    // waited for here, before the ring starts (see the dQ kernel)
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) asm volatile("" ::"v"(k1f[kb]), "v"(k2f[kb]));
#pragma unroll
    for (int c = 0; c < kNVB; ++c) asm volatile("" ::"v"(vf[c]));
    // queries that see this lane's key: q_begin .. q_end - 1
    const int q_begin = CAUSAL ? key : 0;
    const int q_end = kok ? a.Nq : q_begin;

    f32x16 dvt[kNDB], dk1t[kNCB], dk2t[kNCB];
#pragma unroll
    for (int i = 0; i < kNDB; ++i) dvt[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < kNCB; ++i) dk1t[i] = dk2t[i] = f32x16{};

    const int nqt = (a.Nq + 31) / 32;
    const int qt0 = CAUSAL ? (kt * kRowsWG) / 32 : 0;
    // first query tile that sees a key of this wave
    const int qt_w = CAUSAL ? kw0 / 32 : 0;
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    TileFeed feed;
    feed.init(wave_u, lane);
    // row terms of the tile's 32 queries: each wave loads its own copy (lanes
    // 32..63 repeat lanes 0..31), so every wave issues the same number of loads
    const int row_off = 16 * l32;
    // (FLAT: one descriptor per tensor for the (batch, head) slice)
    const int qbytes = FLAT ? a.Nq * kKRow : 0, dbytes = FLAT ? a.Nq * kVRow : 0;
    const i32x4 rq1 = sgpr_rsrc(gq1, qbytes), rq2 = sgpr_rsrc(gq2, qbytes);
    const i32x4 rd = sgpr_rsrc(gdd, dbytes), rr = sgpr_rsrc(grows, FLAT ? a.Nq * 16 : 0);
    auto issue = [&](int qt) {
        const uint32_t sti = (uint32_t)(qt & (kStages - 1));
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(
            smem_base + kStages * kStage + sti * kRowStage + (uint32_t)(kRowSlot * wave_u));
        if constexpr (FLAT) {
            const bool real = qt < nqt;
            feed.issue_flat(smem_base + sti * kStage, wave_u, rq1, rq2, rd, real ? qt : -1, qbytes,
                            dbytes);
            load_lds(m0, row_off + (real ? qt * 32 * 16 : a.Nq * 16), rr);
        } else {
            const int64_t n = qt < nqt ? (int64_t)a.Nq : 0;
            feed.issue(smem_base + sti * kStage, wave_u, gq1, gq2, gdd, (int64_t)qt * 32, n);
            load_lds(m0, row_off,
                     sgpr_rsrc(grows + (int64_t)qt * 32 * 16, (n - (int64_t)qt * 32) * 16));
        }
    };
    issue(qt0);
    issue(qt0 + 1);
    issue(qt0 + 2);
    const int qr = swap23(l32);
    const int yq = row_base<kKRow>(qr, lh), yd = row_base<kVRow>(qr, lh);
    const int ycq = col_base<kKRow>(lane), ycd = col_base<kVRow>(lane);

    // tiles qt < qt_w mask every query for this wave: it only keeps the ring
    // going there (a loop of its own, so that the compute loop has one path)
    const int qt_c = min(qt_w, nqt);
    for (int qt = qt0; qt < qt_c; ++qt) {
        wait_loads<2 * (kTileLoads + 1)>();
        __syncthreads();
        issue(qt + 3);
    }
    for (int qt = qt_c; qt < nqt; ++qt) {
        wait_loads<2 * (kTileLoads + 1)>();
        __syncthreads();  // tile qt is in; stage (qt - 1) mod 4 is free
        // stage layout Q1 | Q2 | dD; the row terms in a ring of their own
        const int sb = (qt & (kStages - 1)) * kStage;
        const int yqt = opaque(yq | sb), ydt = opaque(yd | sb);
        const int ycqt = opaque(ycq | sb), ycdt = opaque(ycd | sb);
        const float4* srow = (const float4*)(smem + kStages * kStage +
                                             (qt & (kStages - 1)) * kRowStage + kRowSlot * wave_u);
        f32x16 s1 = f32x16{}, s2 = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb) {
            s1 = mfma(lds_row<0>(smem, yqt ^ (32 * kb)), k1f[kb], s1);
            s2 = mfma(lds_row<kKTile>(smem, yqt ^ (32 * kb)), k2f[kb], s2);
        }
#pragma unroll
        for (int c = 0; c < kNVB; ++c) dp = mfma(lds_row<2 * kKTile>(smem, ydt ^ (32 * c)), vf[c], dp);
        // the next loads after this step's operand reads (see the dQ kernel)
        issue(qt + 3);

        bf16x8 pwd[2], pd1[2], pd2[2];
        const bool full = kw0 + 31 < a.Nk && qt * 32 + 31 < a.Nq && (!CAUSAL || kw0 + 31 <= qt * 32);
        // register r holds query qt 32 + 8 lh + (16 (r / 8) + r % 8), visible
        // while that offset minus lo is below span (unsigned).  Full tiles skip
        // the mask; each path packs its own operands (the paths then merge 24
        // packed registers rather than 48 floats).
        const int lo = q_begin - qt * 32 - 8 * lh;
        const unsigned span = (unsigned)(q_end - q_begin);
        auto probs = [&](auto masked) {
            float wd[16], d1[16], d2[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = 16 * (r >> 3) + 8 * lh + (r & 7);
                const float4 tr = srow[qi];
                float e1 = fmaf(s1[r], sl2, -tr.x), e2 = fmaf(s2[r], sl2, -tr.z);
                if constexpr (decltype(masked)::value) {
                    // min with +inf or -inf: formed on every lane (a select lets
                    // the compiler put the row-term read under a branch)
                    const float cap =
                        (unsigned)(16 * (r >> 3) + (r & 7) - lo) < span ? INFINITY : -INFINITY;
                    e1 = fminf(e1, cap);
                    e2 = fminf(e2, cap);
                }
                const float p1 = __builtin_amdgcn_exp2f(e1);
                const float p2 = __builtin_amdgcn_exp2f(e2);
                wd[r] = p1 - lam * p2;
                d1[r] = p1 * (dp[r] - tr.y);
                d2[r] = -lam * p2 * (dp[r] - tr.w);
            }
            pack(wd, pwd);
            pack(d1, pd1);
            pack(d2, pd2);
        };
        if (full)
            probs(std::false_type{});
        else
            probs(std::true_type{});
        // dV^T += dD^T W,  dK_k^T += Q_k^T dS_k  (k = queries)
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
            const int a0 = ycdt ^ (64 * db);
            mfma_acc(dvt[db], lds_col<kVRow, 2 * kKTile>(smem, a0), pwd[0]);
            mfma_acc(dvt[db], lds_col<kVRow, 2 * kKTile + 16 * kVRow>(smem, a0), pwd[1]);
        }
#pragma unroll
        for (int cb = 0; cb < kNCB; ++cb) {
            const int a0 = ycqt ^ (64 * cb);
            mfma_acc(dk1t[cb], lds_col<kKRow, 0>(smem, a0), pd1[0]);
            mfma_acc(dk1t[cb], lds_col<kKRow, 16 * kKRow>(smem, a0), pd1[1]);
            mfma_acc(dk2t[cb], lds_col<kKRow, kKTile>(smem, a0), pd2[0]);
            mfma_acc(dk2t[cb], lds_col<kKRow, kKTile + 16 * kKRow>(smem, a0), pd2[1]);
        }
    }
    wait_loads<0>();  // the zero-filling loads past the end land before exit
    settle(dvt);
    settle(dk1t);
    settle(dk2t);

    if (!kok) return;
    const float tau = 1.f / sqrtf((float)kD);
    __bf16* o1 = (__bf16*)a.dk1 + ((size_t)bh * a.Nk + key) * kD;
    __bf16* o2 = (__bf16*)a.dk2 + ((size_t)bh * a.Nk + key) * kD;
    __bf16* ov = (__bf16*)a.dv + ((size_t)bh * a.Nk + key) * kDV;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int cb = 0; cb < kNCB; ++cb) {
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
        for (int db = 0; db < kNDB; ++db) {
            bf16x4 wv;
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[e] = (__bf16)dvt[db][4 * g + e];
            *(bf16x4*)(ov + 32 * db + 8 * g + 4 * lh) = wv;
        }
    }
}

}  // namespace

namespace {
// the dQ kernel with paired map waves (it is written for any (d, dv) whose
// tiles fit its ring; at head_dim 64 the one-sweep kernel of backward.hip
// is faster, so only (128, 256) is instantiated)
hipError_t launch_bwd_dq_pair(const BackwardArgs& a, int d, int dv, bool causal,
                              hipStream_t stream) {
    BackwardArgs copy = a;
    void* args[] = {&copy};
    const int64_t g_dq = (int64_t)((a.Nq + kRowsWG - 1) / kRowsWG) * a.B * a.H;
    if (g_dq > 0x7fffffff) return hipErrorInvalidValue;
    if (d != 128 || dv != 256) return hipErrorInvalidValue;
    // one descriptor per tensor when each (batch, head) slice spans < 2 GiB
    const bool flat = one_descriptor(a.flags, (int64_t)a.Nk * 2 * dv);
    const void* fn = causal ? (flat ? (const void*)bwd_dq_pair_kernel<128, 256, true, true>
                                    : (const void*)bwd_dq_pair_kernel<128, 256, true, false>)
                            : (flat ? (const void*)bwd_dq_pair_kernel<128, 256, false, true>
                                    : (const void*)bwd_dq_pair_kernel<128, 256, false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)g_dq), dim3(kDqThreads), args, 0, stream);
}
}  // namespace

hipError_t launch_backward_ring(const BackwardArgs& a, bool causal, hipStream_t stream) {
    BackwardArgs copy = a;
    void* args[] = {&copy};
    const int64_t BH = (int64_t)a.B * a.H;
    const int64_t g_kv = (int64_t)((a.Nk + kRowsWG - 1) / kRowsWG) * BH;
    if (g_kv > 0x7fffffff) return hipErrorInvalidValue;
    hipError_t e = launch_bwd_dq_pair(a, kD, kDV, causal, stream);
    if (e != hipSuccess) return e;
    const bool flat = one_descriptor(a.flags, (int64_t)a.Nq * kVRow);
    const void* fn = causal ? (flat ? (const void*)bwd_dkdv_ring_kernel<true, true>
                                    : (const void*)bwd_dkdv_ring_kernel<true, false>)
                            : (flat ? (const void*)bwd_dkdv_ring_kernel<false, true>
                                    : (const void*)bwd_dkdv_ring_kernel<false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)g_kv), dim3(kBwdThreads), args, 0, stream);
}

}  // namespace diffattn
