// Internal declarations shared by the library's translation units: kernel
// argument blocks and the host-side launchers the C ABI dispatches to.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

// PrefillArgs / BackwardArgs flags bit of DIFFATTN_FLAG_TILE_DESCRIPTORS:
// per-tile buffer descriptors at any size
constexpr uint32_t kFlagTileDescriptors = 2u;

// One buffer descriptor per tensor when the largest (batch, head) slice a
// kernel loads through one spans less than 2 GiB (its tile offsets, and the
// past-the-end offset of up to 64 KB, then stay in the 31-bit range), unless
// the caller asked for per-tile descriptors.
inline bool one_descriptor(uint32_t flags, int64_t slice_bytes) {
    return !(flags & kFlagTileDescriptors) && slice_bytes + 64 * 1024 < (int64_t)0x7fffffff;
}

// Arguments of every prefill kernel.  Pointers are device memory, layouts as in
// diffattn.h.  Element pointers are untyped; each kernel reinterprets them.
struct PrefillArgs {
    const void* q1;
    const void* q2;
    const void* k1;
    const void* k2;
    const void* v;
    const float* lam;
    void* out;
    int32_t B, H, Nq, Nk;
    float lambda_init;
    float eps;
    float scale_log2;  // log2(e) / sqrt(d): folds the score scale into exp2
    uint32_t flags;
    // training forward only (NULL otherwise): D before the GroupNorm
    // [B][H][Nq][dv] fp32 and the natural-log log-sum-exp of each score row
    // [2][B][H][Nq] fp32 (map 1, then map 2)
    float* d_save;
    float* lse;
    // e4m3 Q/K variant only: per map, the product of the Q and K
    // dequantisation scales (score = qk_scale[map] * sum of e4m3 products)
    float qk_scale[2];
};

// Arguments of the fused Q/K/V projection.  x [T][d_model] (T = B N tokens),
// w [n_out][d_model] with n_out = H (4 d + dv); outputs head-major.
struct ProjArgs {
    const void* x;
    const void* w;
    void* q1;
    void* q2;
    void* k1;
    void* k2;
    void* v;
    int32_t T, N, H, d, dv, d_model, n_out;
};

// Arguments of the backward kernels.  Pointers are device memory; layouts as
// in diffattn.h.
struct BackwardArgs {
    const void* q1;
    const void* q2;
    const void* k1;
    const void* k2;
    const void* v;
    const float* lam;
    const void* dout;    // [B][H][Nq][dv]
    const float* d_save; // [B][H][Nq][dv]
    const float* lse;    // [2][B][H][Nq]
    void* dq1;
    void* dq2;
    void* dk1;
    void* dk2;
    void* dv;
    float* dlam;         // [H]
    void* dd;            // workspace: dD [B][H][Nq][dv] bf16
    float* delta;        // workspace: [2][B][H][Nq] row terms sum_j P_k dP
    float* rows;         // workspace: [B][H][Nq][4] lse_1, delta_1, lse_2, delta_2 (lse in log2 units)
    int32_t B, H, Nq, Nk;
    float lambda_init;
    float eps;
    float scale_log2;
    uint32_t flags;
};

// Arguments of the diagnostics kernels.
struct DiagArgs {
    const void* q1;
    const void* q2;
    const void* k1;
    const void* k2;
    const float* lse;         // [2][B][H][Nq] from the training forward (needles only)
    const int32_t* needle_q;  // [B][H][n]
    const int32_t* needle_k;  // [B][H][n]
    float* row_max;           // [2][B][H][Nq] or NULL
    float* needles;           // [B][H][n][4] or NULL
    int32_t n_needles;
    int32_t B, H, Nq, Nk;
};

// Arguments of the decode kernels.
struct DecodeArgs {
    const void* q1;
    const void* q2;
    const void* k1;
    const void* k2;
    const void* v;
    const int32_t* kv_lens;  // NULL or [B]
    const float* lam;
    void* out;
    float* partials;  // [B*H*splits][4 + 2*dv] when splits > 1
    int32_t B, H, L, cap;
    int32_t splits;
    int32_t chunk;  // keys per split, a multiple of 64
    float lambda_init;
    float eps;
    float scale_log2;
    uint32_t flags;
};

// Each launcher returns hipSuccess or the launch error.  d and dv are one of
// the supported pairs; the callers have checked that.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, int dv, bool causal,
                               hipStream_t stream);
// Q1, Q2, K1, K2 as OCP e4m3 bytes, V and the output bf16 (d, dv = 64, 128 or
// 128, 256)
hipError_t launch_prefill_fp8qk(const PrefillArgs& a, int d, int dv, bool causal,
                                hipStream_t stream);
hipError_t launch_qkv_proj_bf16(const ProjArgs& a, hipStream_t stream);
// head_dim 128, v_dim 256: the two-sweep kernel (also the training forward);
// fp8qk: scores from e4m3 queries and keys
hipError_t launch_prefill_twopass(const PrefillArgs& a, int d, int dv, bool causal, bool fp8qk,
                                  hipStream_t stream);
// dQ and dK/dV kernels of the head_dim-128, v_dim-256 backward (after the dD
// prep, before the dlambda sum)
hipError_t launch_backward_ring(const BackwardArgs& a, bool causal, hipStream_t stream);

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, int dv, bool causal,
                              hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, int dv, bool bf16, hipStream_t stream);
// Device address and size of the current device's decode scratch array (the
// partials of diffattn_decode_noalloc), looked up once per device.
hipError_t decode_scratch(void** ptr, size_t* bytes);
hipError_t launch_backward_bf16(const BackwardArgs& a, int d, int dv, bool causal,
                                hipStream_t stream);
hipError_t launch_diag_bf16(const DiagArgs& a, int d, bool causal, hipStream_t stream);
// Workspace bytes of the backward: dD in bf16, then the row terms (256-byte
// aligned sections).
size_t backward_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int dv);

// Compute units of the current device (cached per device); 0 if unknown.
int device_cus();

// Size in floats of one split's partial record: m1, l1, m2, l2, O1[dv], O2[dv].
__host__ __device__ inline int64_t decode_record_floats(int dv) { return 4 + 2 * (int64_t)dv; }

}  // namespace diffattn
