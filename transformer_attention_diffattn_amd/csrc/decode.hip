// Differential Attention decode against a KV cache (gfx950).
//
// One query token per (batch, head) attends every cached key: the DiffAttn
// formula (iloveeagents.com, "Mathematical Formula") with a single query row,
// then the per-head GroupNorm and (1 - lambda_init) scale of step 4 on
// llmbytes.dev.  With one query the operator does 1.5 flops per byte of cache,
// so it is bound by HBM bandwidth, not by arithmetic: the kernels run on the
// vector ALUs and are built to keep many coalesced 16-byte loads in flight.
//
// Split-K: each sequence's cache is cut into `splits` chunks.  Kernel 1 runs
// one workgroup per (batch, head, chunk); its 4 waves stream blocks of the
// chunk independently, each keeping two online-softmax states (running max m,
// sum l and weighted value sum O for each map), and merge them through LDS at
// the end.  The merge of two states rescales by 2^(m_a - m_max) before adding,
// so the result does not depend on how the keys were split.  With one split
// kernel 1 also applies the epilogue; otherwise it writes the merged state to
// the workspace and kernel 2 merges the chunks of each (batch, head) in a fixed
// order (deterministic) and applies the epilogue.
//
// Per block of KB keys a wave
//   1. loads the K1 and K2 rows with d/8 lanes per key (16 bytes per lane,
//      whole rows per instruction) and the V rows with dv/8 lanes per key;
//   2. forms each key's two scores from in-lane dot products and a DPP sum
//      over the lanes of the key, and moves them through a wave-private LDS
//      slot so that lane j holds key j;
//   3. updates both online softmaxes (wave max, exp2, lane-partial sums);
//   4. accumulates p1 * V and p2 * V into per-lane channel accumulators.

#include "../../include/diffattn.h"
#include "internal.h"

#include <mutex>

#include <math.h>

namespace diffattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// 8 consecutive channels of one row, as loaded (16 bytes for bf16, 32 for fp32)
template <typename T>
struct Chunk8;

template <>
struct Chunk8<uint16_t> {
    u32x4 w;
    __device__ __forceinline__ void load(const uint16_t* p) { w = *(const u32x4*)p; }
    // a cache row, read once per launch: streamed past the caches
    __device__ __forceinline__ void stream(const uint16_t* p) {
        w = __builtin_nontemporal_load((const u32x4*)p);
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t x = w[e >> 1];
        return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    }
};

template <>
struct Chunk8<float> {
    u32x4 w0, w1;
    __device__ __forceinline__ void load(const float* p) {
        w0 = *(const u32x4*)p;
        w1 = *(const u32x4*)(p + 4);
    }
    __device__ __forceinline__ void stream(const float* p) {
        w0 = __builtin_nontemporal_load((const u32x4*)p);
        w1 = __builtin_nontemporal_load((const u32x4*)(p + 4));
    }
    __device__ __forceinline__ float get(int e) const {
        return __uint_as_float(e < 4 ? w0[e] : w1[e - 4]);
    }
};

// Partial dot product of 8 channels of q (kept as a loaded chunk) with a key
// chunk.  bf16 values unpack exactly to fp32; the products accumulate in fp32.
template <typename T>
__device__ __forceinline__ float dot8(const Chunk8<T>& q, const Chunk8<T>& k) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(q.get(e), k.get(e), s);
    return s;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 4, 8 or 16); every lane gets its group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (G >= 16) x += dpp<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// a*b - c*d with both products rounded before the subtraction (no fused
// multiply-add), so equal operands cancel to exactly zero
__device__ __forceinline__ float diff_of_products(float a, float b, float c, float d) {
#pragma clang fp contract(off)
    return a * b - c * d;
}

// Orders this wave's LDS accesses around a cross-lane exchange.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int D, int DV>
struct Cfg {
    static constexpr int kLpk = D / 8;              // lanes per K row
    static constexpr int kKpi = 64 / kLpk;          // keys per K load
    static constexpr int kLpr = DV / 8;             // lanes per V row
    static constexpr int kRpi = 64 / kLpr;          // V rows per load
    // keys per wave block, sized to keep 128 VGPRs of loads in flight
    static constexpr int kKb0 = (sizeof(T) == 2 ? 16384 : 8192) / (2 * D + DV);
    static constexpr int kKb = kKb0 > 64 ? 64 : kKb0;
    static constexpr int kKLoads = kKb / kKpi;
    static constexpr int kVLoads = kKb / kRpi;
    static constexpr int kEl = DV / 64;             // channels per lane in the epilogue
    static_assert(kKb % kKpi == 0 && kKb % kRpi == 0, "block must split into loads");
};

// Applies the epilogue to a merged state held by one wave, kEl channels per
// lane (channel c = lane + 64 * i), and stores the output row.
template <typename T, int DV>
__device__ void finish_row(const float (&o1)[DV / 64], const float (&o2)[DV / 64], float l1,
                           float l2, float lam, const DecodeArgs& a, T* out_row, int lane) {
    constexpr int E = DV / 64;
    float dv_[E];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        // an empty sequence (l = 0) gives D = 0
        const float x = diff_of_products(o1[i], l1 > 0.f ? 1.f / l1 : 0.f,
                                         o2[i], l2 > 0.f ? lam / l2 : 0.f);
        dv_[i] = x;
        s += x;
    }
    if (!(a.flags & 1u)) {
        const float mean = wave_sum(s) * (1.f / DV);
        float vs = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float c = dv_[i] - mean;
            vs = fmaf(c, c, vs);
        }
        const float var = wave_sum(vs) * (1.f / DV);
        const float scale = (1.f - a.lambda_init) / sqrtf(var + a.eps);
#pragma unroll
        for (int i = 0; i < E; ++i) dv_[i] = (dv_[i] - mean) * scale;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
        if constexpr (sizeof(T) == 2)
            ((__bf16*)out_row)[lane + 64 * i] = (__bf16)dv_[i];
        else
            ((float*)out_row)[lane + 64 * i] = dv_[i];
    }
}

template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeArgs a) {
    using C = Cfg<T, D, DV>;
    __shared__ float sc[kWaves][2][C::kKb];                  // scores, then probabilities
    __shared__ float st[kWaves][4];                          // m1, l1, m2, l2 per wave
    __shared__ __attribute__((aligned(16))) float so[kWaves][2][DV];  // O1, O2 per wave

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int split = blockIdx.x % a.splits;
    const int bh = blockIdx.x / a.splits;
    const int b = bh / a.H;
    const int h = bh - b * a.H;

    int len = a.L;
    if (a.kv_lens) len = min(max(a.kv_lens[b], 0), a.L);
    const int start = split * a.chunk;
    const int end = min(start + a.chunk, len);

    const T* gk1 = (const T*)a.k1 + (size_t)bh * a.cap * D;
    const T* gk2 = (const T*)a.k2 + (size_t)bh * a.cap * D;
    const T* gv = (const T*)a.v + (size_t)bh * a.cap * DV;

    // this lane's 8 channels of both queries (the K lane layout repeats them)
    Chunk8<T> q1c, q2c;
    const int kch = lane % C::kLpk;
    q1c.load((const T*)a.q1 + (size_t)bh * D + 8 * kch);
    q2c.load((const T*)a.q2 + (size_t)bh * D + 8 * kch);

    const float NEG_INF = -INFINITY;
    const float sl2 = a.scale_log2;
    float m1 = NEG_INF, m2 = NEG_INF, l1 = 0.f, l2 = 0.f;
    float o1[8], o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o1[e] = 0.f;
        o2[e] = 0.f;
    }
    const int vch = lane % C::kLpr;  // this lane's 8 V channels: 8*vch ..
    const int vrow = lane / C::kLpr;

    const int nblk = end > start ? (end - start + C::kKb - 1) / C::kKb : 0;
    for (int blk = wave; blk < nblk; blk += kWaves) {
        const int kbase = start + blk * C::kKb;
        const int last = end - 1;  // clamp target: a valid row of this sequence
        Chunk8<T> kc1[C::kKLoads], kc2[C::kKLoads], vc[C::kVLoads];
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
            const int key = min(kbase + i * C::kKpi + lane / C::kLpk, last);
            kc1[i].stream(gk1 + (size_t)key * D + 8 * kch);
            kc2[i].stream(gk2 + (size_t)key * D + 8 * kch);
        }
#pragma unroll
        for (int i = 0; i < C::kVLoads; ++i) {
            const int key = min(kbase + i * C::kRpi + vrow, last);
            vc[i].stream(gv + (size_t)key * DV + 8 * vch);
        }

        // scores: in-lane partial dot products, summed over the key's lanes
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
            const float s1 = group_sum<C::kLpk>(dot8(q1c, kc1[i]));
            const float s2 = group_sum<C::kLpk>(dot8(q2c, kc2[i]));
            if (kch == 0) {
                sc[wave][0][i * C::kKpi + lane / C::kLpk] = s1;
                sc[wave][1][i * C::kKpi + lane / C::kLpk] = s2;
            }
        }
        wave_lds_sync();

        // online softmax update with lane j holding key kbase + j
        const bool valid = lane < C::kKb && kbase + lane < end;
        const float x1 = valid ? sc[wave][0][lane] * sl2 : NEG_INF;
        const float x2 = valid ? sc[wave][1][lane] * sl2 : NEG_INF;
        const float mn1 = fmaxf(m1, wave_max(x1));
        const float mn2 = fmaxf(m2, wave_max(x2));
        const float base1 = mn1 == NEG_INF ? 0.f : mn1;
        const float base2 = mn2 == NEG_INF ? 0.f : mn2;
        const float al1 = __builtin_amdgcn_exp2f(m1 - base1);
        const float al2 = __builtin_amdgcn_exp2f(m2 - base2);
        const float p1 = __builtin_amdgcn_exp2f(x1 - base1);
        const float p2 = __builtin_amdgcn_exp2f(x2 - base2);
        m1 = mn1;
        m2 = mn2;
        l1 = fmaf(l1, al1, p1);
        l2 = fmaf(l2, al2, p2);
        wave_lds_sync();
        if (lane < C::kKb) {
            sc[wave][0][lane] = p1;
            sc[wave][1][lane] = p2;
        }
        wave_lds_sync();

#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o1[e] *= al1;
            o2[e] *= al2;
        }
#pragma unroll
        for (int i = 0; i < C::kVLoads; ++i) {
            const int kl = i * C::kRpi + vrow;
            const float w1 = sc[wave][0][kl];
            const float w2 = sc[wave][1][kl];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = vc[i].get(e);
                o1[e] = fmaf(w1, x, o1[e]);
                o2[e] = fmaf(w2, x, o2[e]);
            }
        }
        wave_lds_sync();
    }

    // wave totals: sum l over lanes, O over the lanes that share channels
    l1 = wave_sum(l1);
    l2 = wave_sum(l2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int m = C::kLpr; m < 64; m <<= 1) {
            o1[e] += __shfl_xor(o1[e], m);
            o2[e] += __shfl_xor(o2[e], m);
        }
    }
    if (lane == 0) {
        st[wave][0] = m1;
        st[wave][1] = l1;
        st[wave][2] = m2;
        st[wave][3] = l2;
    }
    if (lane < C::kLpr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            so[wave][0][8 * lane + e] = o1[e];
            so[wave][1][8 * lane + e] = o2[e];
        }
    }
    __syncthreads();
    if (wave != 0) return;

    // merge the 4 wave states (wave 0); lane holds channels lane + 64 i
    float mm1 = NEG_INF, mm2 = NEG_INF;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        mm1 = fmaxf(mm1, st[w][0]);
        mm2 = fmaxf(mm2, st[w][2]);
    }
    float L1 = 0.f, L2 = 0.f;
    float O1[C::kEl], O2[C::kEl];
#pragma unroll
    for (int i = 0; i < C::kEl; ++i) {
        O1[i] = 0.f;
        O2[i] = 0.f;
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float f1 = st[w][0] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(st[w][0] - mm1);
        const float f2 = st[w][2] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(st[w][2] - mm2);
        L1 = fmaf(f1, st[w][1], L1);
        L2 = fmaf(f2, st[w][3], L2);
#pragma unroll
        for (int i = 0; i < C::kEl; ++i) {
            O1[i] = fmaf(f1, so[w][0][lane + 64 * i], O1[i]);
            O2[i] = fmaf(f2, so[w][1][lane + 64 * i], O2[i]);
        }
    }

    if (a.splits == 1) {
        T* out_row = (T*)a.out + (size_t)bh * DV;
        finish_row<T, DV>(O1, O2, L1, L2, a.lam[h], a, out_row, lane);
    } else {
        float* rec = a.partials + ((size_t)bh * a.splits + split) * decode_record_floats(DV);
        if (lane == 0) {
            rec[0] = mm1;
            rec[1] = L1;
            rec[2] = mm2;
            rec[3] = L2;
        }
#pragma unroll
        for (int i = 0; i < C::kEl; ++i) {
            rec[4 + lane + 64 * i] = O1[i];
            rec[4 + DV + lane + 64 * i] = O2[i];
        }
    }
}

// One wave per (batch, head): merges the split records in order, then the epilogue.
template <typename T, int DV>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
    constexpr int E = DV / 64;
    const int lane = threadIdx.x;
    const int bh = blockIdx.x;
    const int h = bh % a.H;
    const int64_t rs = decode_record_floats(DV);
    const float* recs = a.partials + (size_t)bh * a.splits * rs;

    float mm1 = -INFINITY, mm2 = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
        mm1 = fmaxf(mm1, recs[s * rs + 0]);
        mm2 = fmaxf(mm2, recs[s * rs + 2]);
    }
    float L1 = 0.f, L2 = 0.f, O1[E], O2[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        O1[i] = 0.f;
        O2[i] = 0.f;
    }
    for (int s = 0; s < a.splits; ++s) {
        const float* r = recs + s * rs;
        const float f1 = r[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(r[0] - mm1);
        const float f2 = r[2] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(r[2] - mm2);
        L1 = fmaf(f1, r[1], L1);
        L2 = fmaf(f2, r[3], L2);
#pragma unroll
        for (int i = 0; i < E; ++i) {
            O1[i] = fmaf(f1, r[4 + lane + 64 * i], O1[i]);
            O2[i] = fmaf(f2, r[4 + DV + lane + 64 * i], O2[i]);
        }
    }
    T* out_row = (T*)a.out + (size_t)bh * DV;
    finish_row<T, DV>(O1, O2, L1, L2, a.lam[h], a, out_row, lane);
}

template <typename T, int D, int DV>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    DecodeArgs copy = a;
    void* args[] = {&copy};
    const dim3 grid1((unsigned)((int64_t)a.B * a.H * a.splits));
    hipError_t e = hipLaunchKernel((const void*)decode_partial_kernel<T, D, DV>, grid1,
                                   dim3(kThreads), args, 0, stream);
    if (e != hipSuccess || a.splits == 1) return e;
    const dim3 grid2((unsigned)((int64_t)a.B * a.H));
    return hipLaunchKernel((const void*)decode_merge_kernel<T, DV>, grid2, dim3(64), args, 0,
                           stream);
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, int d, int dv, hipStream_t stream) {
    if (d == 32 && dv == 64) return launch_typed<T, 32, 64>(a, stream);
    if (d == 64 && dv == 128) return launch_typed<T, 64, 128>(a, stream);
    if (d == 128 && dv == 256) return launch_typed<T, 128, 256>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

// Partial records of diffattn_decode_noalloc: a fixed device array instead of
// a caller workspace.  Host code must not pass the array's name to a kernel
// (on the host it is a stand-in, not a device address): decode_scratch looks
// up each device's own copy once, with that device current, and the kernels
// get that address.
static __device__ __align__(256) uint8_t scratch[DIFFATTN_NOALLOC_SCRATCH_BYTES];

hipError_t decode_scratch(void** ptr, size_t* bytes) {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int d, int dv, bool bf16, hipStream_t stream) {
    return bf16 ? launch_t<uint16_t>(a, d, dv, stream) : launch_t<float>(a, d, dv, stream);
}

}  // namespace diffattn
