// C ABI of the Differential Attention library: argument checks, the decode
// split plan, and dispatch to the kernel launchers.  Every check runs before
// the first HIP call, so a rejected call launches nothing and writes nothing.

#include "../../include/diffattn.h"
#include "internal.h"

#include <math.h>
#include <mutex>

namespace diffattn {

// Compute units of the current device, cached per device.
int device_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> g(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = cus;
    }
    return cache[dev];
}

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_dims(int d, int dv) {
    return (d == 32 && dv == 64) || (d == 64 && dv == 128) || (d == 128 && dv == 256);
}

// Checks shared by prefill and decode.  Returns DIFFATTN_OK or an error.
int check_dims(const diffattn_dims* dm) {
    if (!dm) return DIFFATTN_ERR_INVALID;
    if (dm->batch < 1 || dm->heads < 1 || dm->seq_q < 1 || dm->seq_k < 1 || dm->head_dim < 1 ||
        dm->v_dim < 1)
        return DIFFATTN_ERR_INVALID;
    if (!(dm->eps >= 0.f) || !isfinite(dm->eps)) return DIFFATTN_ERR_INVALID;
    if (dm->flags & ~(DIFFATTN_FLAG_PRE_NORM | DIFFATTN_FLAG_TILE_DESCRIPTORS))
        return DIFFATTN_ERR_INVALID;
    if (dm->dtype != DIFFATTN_F32 && dm->dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
    if (!supported_dims(dm->head_dim, dm->v_dim)) return DIFFATTN_ERR_UNSUPPORTED;
    if ((int64_t)dm->batch * dm->heads > 0x7fffffff) return DIFFATTN_ERR_UNSUPPORTED;
    if (dm->seq_q > (1 << 30) || dm->seq_k > (1 << 30)) return DIFFATTN_ERR_UNSUPPORTED;
    return DIFFATTN_OK;
}

float scale_log2(int d) { return (float)(1.4426950408889634 / sqrt((double)d)); }

// Keys per split, rounded to whole 128-key blocks.
int32_t split_chunk(int32_t L, int32_t splits) {
    int64_t c = ((int64_t)L + splits - 1) / splits;
    c = (c + 127) / 128 * 128;
    return (int32_t)c;
}

// Splits actually used once the chunk is rounded up (never more than asked).
int32_t splits_used(int32_t L, int32_t splits) {
    const int32_t c = split_chunk(L, splits);
    return (int32_t)(((int64_t)L + c - 1) / c);
}

// Enough workgroups to fill the chip about twice over, but chunks of at least
// 512 keys so the per-split fixed cost stays small.
int32_t default_splits(const diffattn_dims* dm, int cus) {
    const int64_t bh = (int64_t)dm->batch * dm->heads;
    const int64_t want = 4 * (int64_t)cus;
    int64_t s = (want + bh - 1) / bh;
    const int64_t max_s = dm->seq_k / 512 > 1 ? dm->seq_k / 512 : 1;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    return (int32_t)s;
}

int check_decode_dims(const diffattn_dims* dm) {
    const int st = check_dims(dm);
    if (st != DIFFATTN_OK) return st;
    if (dm->seq_q != 1) return DIFFATTN_ERR_UNSUPPORTED;
    return DIFFATTN_OK;
}

// Resolves num_splits (0 = default) to the count the kernels run with; 0 on error.
int32_t resolve_splits(const diffattn_dims* dm, int32_t num_splits) {
    if (num_splits < 0) return 0;
    if (num_splits == 0) {
        const int cus = device_cus();
        if (cus <= 0) return 0;
        num_splits = default_splits(dm, cus);
    }
    if (num_splits > dm->seq_k) num_splits = dm->seq_k;
    return splits_used(dm->seq_k, num_splits);
}

}  // namespace
}  // namespace diffattn

using namespace diffattn;

namespace {

// diffattn_decode and diffattn_decode_noalloc: noalloc takes the partials'
// memory from the library's scratch array instead of `workspace`.
int decode_common(const void* q1, const void* q2, const void* k1_cache, const void* k2_cache,
                  const void* v_cache, int32_t kv_capacity, const int32_t* kv_lens,
                  const float* lambda, float lambda_init, void* out, void* workspace,
                  size_t workspace_bytes, bool noalloc, int32_t num_splits,
                  const diffattn_dims* dims, void* stream) {
    using namespace diffattn;
    int st = check_decode_dims(dims);
    if (st != DIFFATTN_OK) return st;
    const void* ptrs[] = {q1, q2, k1_cache, k2_cache, v_cache, lambda, out};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (kv_lens && ((uintptr_t)kv_lens & 3u)) return DIFFATTN_ERR_INVALID;
    if (!isfinite(lambda_init) || num_splits < 0) return DIFFATTN_ERR_INVALID;
    if (kv_capacity < dims->seq_k) return DIFFATTN_ERR_INVALID;

    const int32_t splits = resolve_splits(dims, num_splits);
    if (splits < 1) return DIFFATTN_ERR_HIP;  // device query failed
    if (splits > 1) {
        const size_t need = (size_t)dims->batch * dims->heads * splits *
                            decode_record_floats(dims->v_dim) * sizeof(float);
        if (noalloc) {
            if (need > DIFFATTN_NOALLOC_SCRATCH_BYTES) return DIFFATTN_ERR_WORKSPACE;
            size_t have = 0;
            if (decode_scratch(&workspace, &have) != hipSuccess) return DIFFATTN_ERR_HIP;
            if (need > have) return DIFFATTN_ERR_WORKSPACE;
        } else if (!workspace || !aligned16(workspace) || workspace_bytes < need) {
            return DIFFATTN_ERR_WORKSPACE;
        }
    }

    DecodeArgs a;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1_cache;
    a.k2 = k2_cache;
    a.v = v_cache;
    a.kv_lens = kv_lens;
    a.lam = lambda;
    a.out = out;
    a.partials = (float*)workspace;
    a.B = dims->batch;
    a.H = dims->heads;
    a.L = dims->seq_k;
    a.cap = kv_capacity;
    a.splits = splits;
    a.chunk = split_chunk(dims->seq_k, splits);
    a.lambda_init = lambda_init;
    a.eps = dims->eps;
    a.scale_log2 = scale_log2(dims->head_dim);
    a.flags = dims->flags;
    const hipError_t e = launch_decode(a, dims->head_dim, dims->v_dim,
                                       dims->dtype == DIFFATTN_BF16, (hipStream_t)stream);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int diffattn_abi_version(void) { return DIFFATTN_ABI_VERSION; }

const char* diffattn_status_string(int status) {
    switch (status) {
        case DIFFATTN_OK: return "ok";
        case DIFFATTN_ERR_INVALID: return "invalid argument";
        case DIFFATTN_ERR_UNSUPPORTED: return "unsupported problem";
        case DIFFATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case DIFFATTN_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

const char* diffattn_status_str(int status) { return diffattn_status_string(status); }

int diffattn_fwd(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                 const float* lambda, float lambda_init, int causal, void* out,
                 const diffattn_dims* dims, void* stream) {
    int st = check_dims(dims);
    if (st != DIFFATTN_OK) return st;
    const void* ptrs[] = {q1, q2, k1, k2, v, lambda, out};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (!isfinite(lambda_init)) return DIFFATTN_ERR_INVALID;
    if (causal && dims->seq_q != dims->seq_k) return DIFFATTN_ERR_UNSUPPORTED;

    PrefillArgs a;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1;
    a.k2 = k2;
    a.v = v;
    a.lam = lambda;
    a.out = out;
    a.B = dims->batch;
    a.H = dims->heads;
    a.Nq = dims->seq_q;
    a.Nk = dims->seq_k;
    a.lambda_init = lambda_init;
    a.eps = dims->eps;
    a.scale_log2 = scale_log2(dims->head_dim);
    a.flags = dims->flags;
    a.d_save = nullptr;
    a.lse = nullptr;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = dims->dtype == DIFFATTN_BF16
                             ? launch_prefill_bf16(a, dims->head_dim, dims->v_dim, causal != 0, s)
                             : launch_prefill_f32(a, dims->head_dim, dims->v_dim, causal != 0, s);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

int diffattn_fwd_fp8(const void* q1, const void* q2, const void* k1, const void* k2,
                     const void* v, const float* qk_scales, const float* lambda,
                     float lambda_init, int causal, void* out, const diffattn_dims* dims,
                     void* stream) {
    int st = check_dims(dims);
    if (st != DIFFATTN_OK) return st;
    const void* ptrs[] = {q1, q2, k1, k2, v, lambda, out};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (!qk_scales || !isfinite(lambda_init)) return DIFFATTN_ERR_INVALID;
    for (int i = 0; i < 4; ++i)
        if (!(qk_scales[i] > 0.f) || !isfinite(qk_scales[i])) return DIFFATTN_ERR_INVALID;
    const float s1 = qk_scales[0] * qk_scales[2], s2 = qk_scales[1] * qk_scales[3];
    if (!(s1 > 0.f) || !isfinite(s1) || !(s2 > 0.f) || !isfinite(s2)) return DIFFATTN_ERR_INVALID;
    if (dims->dtype != DIFFATTN_BF16 || !((dims->head_dim == 64 && dims->v_dim == 128) ||
                                          (dims->head_dim == 128 && dims->v_dim == 256)))
        return DIFFATTN_ERR_UNSUPPORTED;
    if (causal && dims->seq_q != dims->seq_k) return DIFFATTN_ERR_UNSUPPORTED;

    PrefillArgs a;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1;
    a.k2 = k2;
    a.v = v;
    a.lam = lambda;
    a.out = out;
    a.B = dims->batch;
    a.H = dims->heads;
    a.Nq = dims->seq_q;
    a.Nk = dims->seq_k;
    a.lambda_init = lambda_init;
    a.eps = dims->eps;
    a.scale_log2 = scale_log2(dims->head_dim);
    a.flags = dims->flags;
    a.d_save = nullptr;
    a.lse = nullptr;
    a.qk_scale[0] = s1;
    a.qk_scale[1] = s2;
    const hipError_t e = launch_prefill_fp8qk(a, dims->head_dim, dims->v_dim, causal != 0,
                                              (hipStream_t)stream);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

int diffattn_qkv_proj(const void* x, const void* w, int32_t batch, int32_t seq, int32_t heads,
                      int32_t head_dim, int32_t v_dim, int32_t model_dim, void* q1, void* q2,
                      void* k1, void* k2, void* v, void* stream) {
    const void* ptrs[] = {x, w, q1, q2, k1, k2, v};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (batch < 1 || seq < 1 || heads < 1 || head_dim < 1 || v_dim < 1 || model_dim < 1)
        return DIFFATTN_ERR_INVALID;
    if (!supported_dims(head_dim, v_dim)) return DIFFATTN_ERR_UNSUPPORTED;
    if (model_dim % 32 != 0 || model_dim > (1 << 20)) return DIFFATTN_ERR_UNSUPPORTED;
    const int64_t T = (int64_t)batch * seq;
    const int64_t n_out = (int64_t)heads * (4 * head_dim + v_dim);
    if (T > 0x7fffffff - 256 || n_out > 0x7fffffff - 256) return DIFFATTN_ERR_UNSUPPORTED;
    ProjArgs a;
    a.x = x;
    a.w = w;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1;
    a.k2 = k2;
    a.v = v;
    a.T = (int32_t)T;
    a.N = seq;
    a.H = heads;
    a.d = head_dim;
    a.dv = v_dim;
    a.d_model = model_dim;
    a.n_out = (int32_t)n_out;
    const hipError_t e = launch_qkv_proj_bf16(a, (hipStream_t)stream);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

// The training pair (forward that saves D and the log-sum-exp, backward):
// bf16 with (d, dv) = (32, 64) or (64, 128).
static int check_train_dims(const diffattn_dims* dims, int causal) {
    int st = check_dims(dims);
    if (st != DIFFATTN_OK) return st;
    if (dims->dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
    if (!((dims->head_dim == 32 && dims->v_dim == 64) || (dims->head_dim == 64 && dims->v_dim == 128) ||
          (dims->head_dim == 128 && dims->v_dim == 256)))
        return DIFFATTN_ERR_UNSUPPORTED;
    if (causal && dims->seq_q != dims->seq_k) return DIFFATTN_ERR_UNSUPPORTED;
    return DIFFATTN_OK;
}

int diffattn_fwd_train(const void* q1, const void* q2, const void* k1, const void* k2,
                       const void* v, const float* lambda, float lambda_init, int causal,
                       void* out, float* d_save, float* lse, const diffattn_dims* dims,
                       void* stream) {
    int st = check_train_dims(dims, causal);
    if (st != DIFFATTN_OK) return st;
    const void* ptrs[] = {q1, q2, k1, k2, v, lambda, out, d_save, lse};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (!isfinite(lambda_init)) return DIFFATTN_ERR_INVALID;

    PrefillArgs a;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1;
    a.k2 = k2;
    a.v = v;
    a.lam = lambda;
    a.out = out;
    a.B = dims->batch;
    a.H = dims->heads;
    a.Nq = dims->seq_q;
    a.Nk = dims->seq_k;
    a.lambda_init = lambda_init;
    a.eps = dims->eps;
    a.scale_log2 = scale_log2(dims->head_dim);
    a.flags = dims->flags;
    a.d_save = d_save;
    a.lse = lse;
    const hipError_t e = launch_prefill_bf16(a, dims->head_dim, dims->v_dim, causal != 0,
                                             (hipStream_t)stream);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

size_t diffattn_bwd_workspace_size(const diffattn_dims* dims) {
    if (check_train_dims(dims, 0) != DIFFATTN_OK) return 0;
    return backward_workspace_bytes(dims->batch, dims->heads, dims->seq_q, dims->v_dim);
}

int diffattn_bwd(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                 const float* lambda, float lambda_init, int causal, const void* dout,
                 const float* d_save, const float* lse, void* dq1, void* dq2, void* dk1,
                 void* dk2, void* dv, float* dlambda, void* workspace, size_t workspace_bytes,
                 const diffattn_dims* dims, void* stream) {
    int st = check_train_dims(dims, causal);
    if (st != DIFFATTN_OK) return st;
    const void* ptrs[] = {q1, q2, k1, k2, v, lambda, dout, d_save, lse,
                          dq1, dq2, dk1, dk2, dv, dlambda, workspace};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (!isfinite(lambda_init)) return DIFFATTN_ERR_INVALID;
    const size_t need =
        backward_workspace_bytes(dims->batch, dims->heads, dims->seq_q, dims->v_dim);
    if (workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;

    BackwardArgs a;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1;
    a.k2 = k2;
    a.v = v;
    a.lam = lambda;
    a.dout = dout;
    a.d_save = d_save;
    a.lse = lse;
    a.dq1 = dq1;
    a.dq2 = dq2;
    a.dk1 = dk1;
    a.dk2 = dk2;
    a.dv = dv;
    a.dlam = dlambda;
    const size_t rows = (size_t)dims->batch * dims->heads * dims->seq_q;
    a.dd = workspace;
    a.delta = (float*)((char*)workspace + (rows * dims->v_dim * 2 + 255) / 256 * 256);
    a.rows = (float*)((char*)a.delta + (2 * rows * sizeof(float) + 255) / 256 * 256);
    a.B = dims->batch;
    a.H = dims->heads;
    a.Nq = dims->seq_q;
    a.Nk = dims->seq_k;
    a.lambda_init = lambda_init;
    a.eps = dims->eps;
    a.scale_log2 = scale_log2(dims->head_dim);
    a.flags = dims->flags;
    const hipError_t e = launch_backward_bf16(a, dims->head_dim, dims->v_dim, causal != 0,
                                              (hipStream_t)stream);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

int diffattn_diag(const void* q1, const void* q2, const void* k1, const void* k2,
                  const float* lse, int causal, const int32_t* needle_q,
                  const int32_t* needle_k, int32_t n_needles, float* row_max, float* needles,
                  const diffattn_dims* dims, void* stream) {
    int st = check_dims(dims);
    if (st != DIFFATTN_OK) return st;
    if (dims->dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
    if (causal && dims->seq_q != dims->seq_k) return DIFFATTN_ERR_UNSUPPORTED;
    const void* ptrs[] = {q1, q2, k1, k2};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return DIFFATTN_ERR_INVALID;
    if (n_needles < 0 || n_needles > 4096) return DIFFATTN_ERR_INVALID;
    if (!row_max && !needles) return DIFFATTN_ERR_INVALID;
    if (row_max && ((uintptr_t)row_max & 3u)) return DIFFATTN_ERR_INVALID;
    if (needles) {
        if (n_needles < 1 || !lse || !needle_q || !needle_k) return DIFFATTN_ERR_INVALID;
        if (((uintptr_t)lse | (uintptr_t)needle_q | (uintptr_t)needle_k | (uintptr_t)needles) & 3u)
            return DIFFATTN_ERR_INVALID;
    }
    DiagArgs a;
    a.q1 = q1;
    a.q2 = q2;
    a.k1 = k1;
    a.k2 = k2;
    a.lse = lse;
    a.needle_q = needle_q;
    a.needle_k = needle_k;
    a.row_max = row_max;
    a.needles = needles;
    a.n_needles = needles ? n_needles : 0;
    a.B = dims->batch;
    a.H = dims->heads;
    a.Nq = dims->seq_q;
    a.Nk = dims->seq_k;
    const hipError_t e = launch_diag_bf16(a, dims->head_dim, causal != 0, (hipStream_t)stream);
    return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP;
}

int32_t diffattn_decode_default_splits(const diffattn_dims* dims) {
    if (check_decode_dims(dims) != DIFFATTN_OK) return 0;
    return resolve_splits(dims, 0);
}

size_t diffattn_decode_workspace_size(const diffattn_dims* dims, int32_t num_splits) {
    if (check_decode_dims(dims) != DIFFATTN_OK) return 0;
    const int32_t s = resolve_splits(dims, num_splits);
    if (s <= 1) return 0;
    return (size_t)dims->batch * dims->heads * s * decode_record_floats(dims->v_dim) * sizeof(float);
}

int diffattn_decode(const void* q1, const void* q2, const void* k1_cache, const void* k2_cache,
                    const void* v_cache, int32_t kv_capacity, const int32_t* kv_lens,
                    const float* lambda, float lambda_init, void* out, void* workspace,
                    size_t workspace_bytes, int32_t num_splits, const diffattn_dims* dims,
                    void* stream) {
    return decode_common(q1, q2, k1_cache, k2_cache, v_cache, kv_capacity, kv_lens, lambda,
                         lambda_init, out, workspace, workspace_bytes, false, num_splits, dims,
                         stream);
}

int diffattn_decode_noalloc(const void* q1, const void* q2, const void* k1_cache,
                            const void* k2_cache, const void* v_cache, int32_t kv_capacity,
                            const int32_t* kv_lens, const float* lambda, float lambda_init,
                            void* out, int32_t num_splits, const diffattn_dims* dims,
                            void* stream) {
    return decode_common(q1, q2, k1_cache, k2_cache, v_cache, kv_capacity, kv_lens, lambda,
                         lambda_init, out, nullptr, 0, true, num_splits, dims, stream);
}

}  // extern "C"
