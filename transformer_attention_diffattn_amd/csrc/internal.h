// Internal declarations shared by the library's translation units: kernel
// argument blocks and the host-side launchers the C ABI dispatches to.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

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
hipError_t launch_prefill_bf16_wide(const PrefillArgs& a, int d, int dv, bool causal,
                                    hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, int d, int dv, bool causal,
                              hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, int dv, bool bf16, hipStream_t stream);

// Compute units of the current device (cached per device); 0 if unknown.
int device_cus();

// Size in floats of one split's partial record: m1, l1, m2, l2, O1[dv], O2[dv].
__host__ __device__ inline int64_t decode_record_floats(int dv) { return 4 + 2 * (int64_t)dv; }

}  // namespace diffattn
