// The projections in front of Differential Attention, fused with the head
// split: Y = X W^T on the bf16 MFMA, each output written straight into the
// head-major Q1, Q2, K1, K2 [B][H][N][d] and V [B][H][N][dv] that the
// attention kernels read (step 1 on llmbytes.dev, "How Differential Attention
// Cancels Common-Mode Noise": per head two queries, two keys and one value
// projected from the input).
//
// Weight layout: W [H (4 d + dv)][d_model], a linear layer's (output feature,
// input feature); output feature f is head h = f / S (S = 4 d + dv), offset
// o = f - h S: Q1 at [0, d), Q2 [d, 2d), K1 [2d, 3d), K2 [3d, 4d), V [4d, S).
//
// Workgroup = 256 output features x 256 tokens, 8 waves (4 feature quarters
// x 2 token halves), each 64 x 128 as 2 x 4 blocks of 32 x 32.  The
// contraction runs in steps of 64: both tiles of a step (W and X rows, 128
// bytes each: whole cache lines) go from global memory straight into a
// 2-stage LDS ring by buffer loads with the LDS destination, one step ahead.
// Rows are 128 bytes, two per 256-byte bank line; chunk c of row r sits at
// c ^ ((r >> 1) & 7), so the 16 rows a 16-byte operand read touches at once
// hit distinct banks.  (Steps of 32 in a 4-stage ring, half cache lines per
// row and step, measured 5% slower.)

#include "internal.h"

// The direct-to-LDS loads set M0 in inline asm; nothing else in this file
// uses M0, so the reserved-register clobber is safe here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kTileF = 256;   // output features per workgroup
constexpr int kTileT = 256;   // tokens per workgroup
constexpr int kStepK = 64;    // contraction elements per stage
constexpr int kStages = 2;
constexpr int kAhead = kStages - 1;
constexpr int kRowBytes = kStepK * 2;                       // 64
constexpr int kRegionBytes = kTileF * kRowBytes;           // one operand's tile: 16 KB
constexpr int kStageBytes = 2 * kRegionBytes;               // W tile, then X tile
constexpr int kLoads = kStageBytes / 16 / 64 / (kThreads / 64);  // per wave and stage
constexpr int kGroupT = 4;    // token tiles per group of the tile order
constexpr int kBufferWord3 = 0x00020000;
static_assert(kTileF == kTileT, "the two regions share one load layout");
static_assert(kLoads == 8, "four loads of each region per wave");
constexpr int kCpr = kRowBytes / 16;

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ i32x4 rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
    const uint64_t p = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = kBufferWord3;
    return r;
}

template <int D, int DV>
__global__ __launch_bounds__(kThreads) void qkv_proj_kernel(ProjArgs a) {
    constexpr int S = 4 * D + DV;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wf = wave_u & 3, wt = wave_u >> 2;

    // tile order: block b runs on XCD b % 8; each XCD takes a contiguous run
    // of the order, which goes through groups of kGroupT token tiles, all
    // feature tiles of a group before the next (X and W tiles reused in L2)
    const int n_f = (a.n_out + kTileF - 1) / kTileF;
    const int n_t = (a.T + kTileT - 1) / kTileT;
    const int total = n_f * n_t;
    const int b = blockIdx.x;
    const int L = (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
    const int gsize = kGroupT * n_f;
    const int g = L / gsize, gi = L - g * gsize;
    const int first_t = g * kGroupT;
    const int gt = min(n_t - first_t, kGroupT);
    const int tile_t = first_t + gi % gt;
    const int tile_f = gi / gt;
    const int f0 = tile_f * kTileF, t0 = tile_t * kTileT;

    const int64_t row_bytes = (int64_t)a.d_model * 2;
    // d_model is a multiple of 32: a last step of 32 uses its first half
    // only (its second half reads past the row: the next row, or zeros)
    const int nst = (a.d_model + kStepK - 1) / kStepK;
    const int half_last = (a.d_model % kStepK) != 0 ? nst - 1 : -1;

    // loads: instruction i of wave w fills LDS chunk positions 64 j .. of its
    // region (W for i < 4, X for i >= 4; j = w + 8 (i % 4)); lane l takes
    // row (64 j + l) / 8 of the region, chunk position (64 j + l) % 8
    i32x4 rs[2];
    uint32_t region[2];
    {
        const int64_t nf = min(kTileF, a.n_out - f0), nt = min(kTileT, a.T - t0);
        rs[0] = rsrc((const char*)a.w + (int64_t)f0 * row_bytes, nf * row_bytes);
        rs[1] = rsrc((const char*)a.x + (int64_t)t0 * row_bytes, nt * row_bytes);
        region[0] = (uint32_t)min<int64_t>(nf * row_bytes, 0x7fffffff);
        region[1] = (uint32_t)min<int64_t>(nt * row_bytes, 0x7fffffff);
    }
    uint32_t ld_off[kLoads], m0_off[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int j = wave_u + (kThreads / 64) * (i & 3);  // instruction within the region
        const int pos = 64 * j + lane;
        const int row = pos / kCpr, cp = pos % kCpr;
        ld_off[i] = (uint32_t)(row * row_bytes) + 16u * (uint32_t)(cp ^ swz(row));
        m0_off[i] = (uint32_t)((i >> 2) * kRegionBytes + 16 * 64 * j);
    }
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    // stages past the last one read out of range (zeros, no memory touched),
    // so every wave issues the same loads for every stage it counts on
    auto issue = [&](int s) {
        const uint32_t stage = smem_base + (uint32_t)((s & (kStages - 1)) * kStageBytes);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = i >> 2;
            const uint32_t toff = s < nst ? (uint32_t)s * kRowBytes : region[r];
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + m0_off[i]);
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :
                         : "s"(m0), "v"(ld_off[i] + toff), "s"(rs[r])
                         : "memory", "m0");
        }
    };

    // operand reads: A = W rows wf*64 + 32 fb + l32, B = X rows wt*128 + 32 tb
    // + l32; k-step ks (of 4) of a stage is chunk 2 ks + lh
    int a_off[2][4], b_off[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
            const int row = wf * 64 + 32 * fb + l32;
            a_off[fb][ks] = row * kRowBytes + 16 * ((2 * ks + lh) ^ swz(row));
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int row = wt * 128 + 32 * tb + l32;
            b_off[tb][ks] = kRegionBytes + row * kRowBytes + 16 * ((2 * ks + lh) ^ swz(row));
        }
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[fb][tb] = f32x16{};

#pragma unroll
    for (int s = 0; s < kAhead; ++s) issue(s);
    for (int s = 0; s < nst; ++s) {
        // this wave's loads of stage s have landed
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 1) * kLoads) : "memory");
        __syncthreads();  // everyone's loads of s landed; everyone is done with s-1
        issue(s + kAhead);  // into the slot of s-1
        const uint8_t* st = smem + (s & (kStages - 1)) * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks == 2 && s == half_last) break;
            bf16x8 av[2], bv[4];
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) av[fb] = *(const bf16x8*)(st + a_off[fb][ks]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) bv[tb] = *(const bf16x8*)(st + b_off[tb][ks]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int fb = 0; fb < 2; ++fb)
                    acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[fb], bv[tb],
                                                                         acc[fb][tb], 0, 0, 0);
        }
    }
    // the trailing out-of-range loads still write the ring: let them land
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // epilogue: accumulator (fb, tb) holds features fbase + 8 (r/4) + 4 lh +
    // r%4 of token t0 + wt*128 + 32 tb + l32; the 32 features of a block lie
    // in one of the five outputs (every boundary is a multiple of 32)
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
        const int fbase = f0 + wf * 64 + 32 * fb;
        if (fbase >= a.n_out) continue;
        const int h = fbase / S, o = fbase - h * S;
        const int seg = o < 4 * D ? o / D : 4;
        const int ch0 = o < 4 * D ? o - seg * D : o - 4 * D;
        const int width = seg == 4 ? DV : D;
        __bf16* dst = (__bf16*)(seg == 0 ? a.q1 : seg == 1 ? a.q2 : seg == 2 ? a.k1
                                : seg == 3 ? a.k2 : a.v);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int t = t0 + wt * 128 + 32 * tb + l32;
            if (t >= a.T) continue;
            const int bb = t / a.N, n = t - bb * a.N;
            __bf16* row = dst + (((int64_t)bb * a.H + h) * a.N + n) * width + ch0 + 4 * lh;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (__bf16)acc[fb][tb][4 * q + e];
                *(bf16x4*)(row + 8 * q) = v4;
            }
        }
    }
}

template <int D, int DV>
hipError_t launch_d(const ProjArgs& a, hipStream_t stream) {
    const int64_t n_f = (a.n_out + kTileF - 1) / kTileF;
    const int64_t n_t = (a.T + kTileT - 1) / kTileT;
    if (n_f * n_t > 0x7fffffff) return hipErrorInvalidValue;
    ProjArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel((const void*)qkv_proj_kernel<D, DV>, dim3((unsigned)(n_f * n_t)),
                           dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_qkv_proj_bf16(const ProjArgs& a, hipStream_t stream) {
    if (a.d == 32 && a.dv == 64) return launch_d<32, 64>(a, stream);
    if (a.d == 64 && a.dv == 128) return launch_d<64, 128>(a, stream);
    if (a.d == 128 && a.dv == 256) return launch_d<128, 256>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
