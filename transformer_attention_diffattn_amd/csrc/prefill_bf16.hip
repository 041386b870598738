// Fused Differential Attention prefill for bf16 inputs on gfx950 (CDNA4):
// the kernels for head_dim 32 and 64, the training forward, and the variant
// with e4m3 queries and keys (head_dim 128, in both forms, is in
// prefill_twopass.hip).  The kernel body is prefill_items in
// prefill_core.h; this file is compiled with the MFMA accumulators in
// ordinary VGPRs, where the softmax reads the scores without a copy.

#include "prefill_core.h"

namespace diffattn {
namespace {

template <int D, int DV, bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
    prefill_items<D, DV, CAUSAL, FLAT, false, false>(a);
}

// The training forward: the same, plus a.d_save and a.lse.
template <int D, int DV, bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kThreads) void prefill_train_kernel(PrefillArgs a) {
    prefill_items<D, DV, CAUSAL, FLAT, false, true>(a);
}

// Scores from e4m3 queries and keys (per-tensor scales in a.qk_scale).
template <bool CAUSAL, bool FLAT>
__global__ __launch_bounds__(kThreads) void prefill_fp8qk_kernel(PrefillArgs a) {
    prefill_items<64, 128, CAUSAL, FLAT, true, false>(a);
}

template <int D, int DV, bool F8>
hipError_t launch_dims(const PrefillArgs& a, bool causal, hipStream_t stream) {
    const int nqt = (a.Nq + Cfg<D, DV, F8>::kBr - 1) / Cfg<D, DV, F8>::kBr;
    const int64_t items = (int64_t)nqt * a.B * a.H;
    // item indices (and the snake's r * G + w) stay in int range
    if (items > (int64_t)0x7fffffff - 4096) return hipErrorInvalidValue;
    const int cus = device_cus();
    const dim3 grid((unsigned)(cus > 0 && items > cus ? cus : items));
    PrefillArgs copy = a;
    void* args[] = {&copy};
    // one descriptor per tensor when each (batch, head) slice spans < 2 GiB
    const bool flat = one_descriptor(a.flags, (int64_t)a.Nk * DV * 2);
    const void* fn;
    if constexpr (F8)
        fn = causal ? (flat ? (const void*)prefill_fp8qk_kernel<true, true>
                            : (const void*)prefill_fp8qk_kernel<true, false>)
                    : (flat ? (const void*)prefill_fp8qk_kernel<false, true>
                            : (const void*)prefill_fp8qk_kernel<false, false>);
    else if (a.lse)
        fn = causal ? (flat ? (const void*)prefill_train_kernel<D, DV, true, true>
                            : (const void*)prefill_train_kernel<D, DV, true, false>)
                    : (flat ? (const void*)prefill_train_kernel<D, DV, false, true>
                            : (const void*)prefill_train_kernel<D, DV, false, false>);
    else
        fn = causal ? (flat ? (const void*)prefill_bf16_kernel<D, DV, true, true>
                            : (const void*)prefill_bf16_kernel<D, DV, true, false>)
                    : (flat ? (const void*)prefill_bf16_kernel<D, DV, false, true>
                            : (const void*)prefill_bf16_kernel<D, DV, false, false>);
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, int dv, bool causal,
                               hipStream_t stream) {
    if (d == 32 && dv == 64) return launch_dims<32, 64, false>(a, causal, stream);
    if (d == 64 && dv == 128) return launch_dims<64, 128, false>(a, causal, stream);
    if (d == 128 && dv == 256) return launch_prefill_twopass(a, d, dv, causal, false, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_fp8qk(const PrefillArgs& a, int d, int dv, bool causal,
                                hipStream_t stream) {
    if (d == 64 && dv == 128) return launch_dims<64, 128, true>(a, causal, stream);
    if (d == 128 && dv == 256) return launch_prefill_twopass(a, d, dv, causal, true, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
