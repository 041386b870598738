/*
 * diffattn.h -- C ABI of the MI355X (gfx950) Differential Attention forward
 * operator.
 *
 * The operator (iloveeagents.com, "Mathematical Formula"; llmbytes.dev, "How
 * Differential Attention Cancels Common-Mode Noise", steps 1-4), per batch
 * entry b, head h and query row i:
 *
 *   A1 = softmax(Q1 K1^T / sqrt(d)),  A2 = softmax(Q2 K2^T / sqrt(d))
 *   D  = (A1 - lambda[h] * A2) V                                 (dv channels)
 *   out = (1 - lambda_init) * (D - mean(D)) / sqrt(var(D) + eps)
 *
 * where d is the query/key head dimension, mean and var are the population
 * moments of the head's dv channels of that row (GroupNorm with one group per
 * head, no affine parameters), and a causal mask, when asked for, lets query i
 * see keys 0..i in both maps.
 *
 * Conventions shared by every entry point:
 *   - Tensors are device memory owned by the caller, contiguous, row-major,
 *     [batch][heads][seq][channels] with the channel dimension unit-stride.
 *     Base pointers must be 16-byte aligned.  The library keeps no pointer
 *     after a call returns and never frees caller memory.
 *   - q1, q2, k1, k2, v and out share one element type (DIFFATTN_F32 or
 *     DIFFATTN_BF16).  All arithmetic is fp32; the output is rounded once
 *     (round-to-nearest-even) to the element type.
 *   - lambda is a device array of `heads` fp32 values.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; faults during execution surface at the caller's next
 *     synchronisation.
 *   - Every argument is checked before any HIP call.  On an error status
 *     nothing is launched and no memory is written.  Nothing is printed and
 *     nothing aborts.
 *   - out must not overlap any input.
 *   - Calls are thread-safe; the library holds no state besides a per-device
 *     cache of the compute-unit count.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIFFATTN_ABI_VERSION 2

/* element types */
#define DIFFATTN_F32 0
#define DIFFATTN_BF16 1

/* status codes */
#define DIFFATTN_OK 0
#define DIFFATTN_ERR_INVALID 1     /* NULL pointer, size < 1, misaligned pointer,
                                      non-finite scalar, eps < 0 */
#define DIFFATTN_ERR_UNSUPPORTED 2 /* well formed but outside the support matrix */
#define DIFFATTN_ERR_WORKSPACE 3   /* decode workspace missing or too small */
#define DIFFATTN_ERR_HIP 4         /* the HIP runtime refused the launch */

/* flags */
#define DIFFATTN_FLAG_PRE_NORM 1u  /* write D itself: skip the GroupNorm and the
                                      (1 - lambda_init) scale (for checks) */
#define DIFFATTN_FLAG_TILE_DESCRIPTORS 2u
/* Prefill, training forward and backward kernels address each K/V (or Q/dD)
 * tile through a buffer descriptor of its own when a (batch, head) slice of a
 * tensor spans 2 GiB or more, and through one descriptor per tensor below
 * that.  This flag selects the per-tile form at any size; the results are
 * bitwise the same (for checks of the large-tensor path at small sizes).
 * Decode, diagnostics and the projection ignore it. */

/*
 * Problem sizes.  Supported (head_dim, v_dim) pairs: (32, 64), (64, 128),
 * (128, 256), for both element types.  Sizes are limited to
 * batch * heads <= 2^31 - 1 and seq_q, seq_k <= 2^30.
 */
typedef struct {
    int32_t batch;    /* B >= 1 */
    int32_t heads;    /* H >= 1 */
    int32_t seq_q;    /* query rows per head (decode: must be 1) */
    int32_t seq_k;    /* keys per head; decode: the longest valid cache length */
    int32_t head_dim; /* d: channels of Q1, Q2, K1, K2 */
    int32_t v_dim;    /* dv: channels of V and of the output */
    int32_t dtype;    /* DIFFATTN_F32 or DIFFATTN_BF16 */
    float eps;        /* GroupNorm epsilon, >= 0 (added to the variance) */
    uint32_t flags;   /* DIFFATTN_FLAG_* */
} diffattn_dims;

/* The version this library was built with (DIFFATTN_ABI_VERSION). */
int diffattn_abi_version(void);

/* A static, human-readable name for a status code. */
const char* diffattn_status_string(int status);
/* The same function under a shorter name. */
const char* diffattn_status_str(int status);

/*
 * Prefill (fused forward over all query rows).
 *   q1, q2 [B][H][seq_q][d]; k1, k2 [B][H][seq_k][d]; v [B][H][seq_k][dv];
 *   out [B][H][seq_q][dv]; lambda [H] fp32 (device).
 *   causal != 0 applies the mask j <= i to both maps and needs seq_q == seq_k.
 * Allocates nothing.  Returns a DIFFATTN_* status.
 */
int diffattn_fwd(const void* q1, const void* q2, const void* k1, const void* k2,
                 const void* v, const float* lambda, float lambda_init, int causal,
                 void* out, const diffattn_dims* dims, void* stream);

/*
 * Prefill with FP8 query and key operands.  Among the low-bit formats that
 * the smaller attention-logit outliers of differential attention make usable,
 * the pages name FP8 (llmbytes.dev, "Solving the Quantization Crisis").
 *   q1, q2 [B][H][seq_q][d], k1, k2 [B][H][seq_k][d]: one byte per element,
 *     OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *     subnormals; no infinities; codes 0x7f and 0xff are NaN), each tensor
 *     with one scale: element = qk_scales[t] * decoded code;
 *   qk_scales: HOST array of 4 fp32 scales (q1, q2, k1, k2), finite and > 0;
 *   v [B][H][seq_k][dv] and out [B][H][seq_q][dv] bf16; lambda, lambda_init,
 *     causal, dims->eps and dims->flags as diffattn_fwd.
 * Each score is the exact sum of products of the codes (fp32 accumulation)
 * times qk_scales[q] * qk_scales[k] / sqrt(d); the rest of the operator runs
 * as in the bf16 prefill.  Supported: dims->dtype == DIFFATTN_BF16 (the type
 * of v and out) with (head_dim, v_dim) = (64, 128) or (128, 256); anything
 * else returns DIFFATTN_ERR_UNSUPPORTED.  Quantising Q and K (choosing the scales,
 * rounding to E4M3) is the caller's.
 * Allocates nothing.  Returns a DIFFATTN_* status.
 */
int diffattn_fwd_fp8(const void* q1, const void* q2, const void* k1, const void* k2,
                     const void* v, const float* qk_scales, const float* lambda,
                     float lambda_init, int causal, void* out, const diffattn_dims* dims,
                     void* stream);

/*
 * The projections in front of the operator, fused with the split into heads
 * (step 1 on llmbytes.dev, "How Differential Attention Cancels Common-Mode
 * Noise": per head, two queries, two keys and one value projected from the
 * input): Y = X W^T in one pass, written straight into the layout the other
 * entry points read.
 *   x [batch][seq][model_dim] bf16 (hidden states, tokens in order);
 *   w [heads * (4 head_dim + v_dim)][model_dim] bf16, a linear layer's
 *     (output feature, input feature) layout; output feature f belongs to
 *     head h = f / S, S = 4 head_dim + v_dim, at offset o = f - h S, with
 *     Q1 at o in [0, d), Q2 [d, 2d), K1 [2d, 3d), K2 [3d, 4d), V [4d, S);
 *   q1, q2, k1, k2 [batch][heads][seq][head_dim], v [batch][heads][seq][v_dim]
 *     bf16 (fp32 accumulation, one rounding to nearest even).
 * Supported: (head_dim, v_dim) as diffattn_fwd; model_dim a multiple of 32,
 * at most 2^20; batch * seq and the output feature count below 2^31 - 256.
 * Outputs must not overlap the inputs or each other.  All pointers device
 * memory, 16-byte aligned.  Allocates nothing.  Returns a DIFFATTN_* status.
 */
int diffattn_qkv_proj(const void* x, const void* w, int32_t batch, int32_t seq, int32_t heads,
                      int32_t head_dim, int32_t v_dim, int32_t model_dim, void* q1, void* q2,
                      void* k1, void* k2, void* v, void* stream);

/*
 * Training forward: diffattn_fwd plus what diffattn_bwd needs, for bf16 with
 * (head_dim, v_dim) = (32, 64), (64, 128) or (128, 256) (else
 * DIFFATTN_ERR_UNSUPPORTED).
 * The backward differentiates the same operator: lambda is a learnable scalar
 * (iloveeagents.com, "Mathematical Formula") and the GroupNorm of step 4 on
 * llmbytes.dev ("How Differential Attention Cancels Common-Mode Noise") is
 * there for stable gradients.
 *   out as diffattn_fwd (same flags);
 *   d_save [B][H][seq_q][dv] fp32: D = O1/l1 - lambda O2/l2 before the
 *     GroupNorm (head_dim 128: D = (A1 - lambda A2) V, the same value);
 *   lse [2][B][H][seq_q] fp32: natural-log log-sum-exp of each row of the
 *     scaled scores, map 1 then map 2.
 * All pointers device memory, 16-byte aligned, owned by the caller.
 * Allocates nothing.  Returns a DIFFATTN_* status.
 */
int diffattn_fwd_train(const void* q1, const void* q2, const void* k1, const void* k2,
                       const void* v, const float* lambda, float lambda_init, int causal,
                       void* out, float* d_save, float* lse, const diffattn_dims* dims,
                       void* stream);

/*
 * Workspace bytes diffattn_bwd needs (dD in bf16 and six fp32 row terms per
 * query row); 0 when the sizes are invalid or unsupported.
 */
size_t diffattn_bwd_workspace_size(const diffattn_dims* dims);

/*
 * Backward: gradients of sum(dout * out) with out as written by
 * diffattn_fwd_train with the same arguments (the flags, PRE_NORM included,
 * must match), from its d_save and lse.
 *   dout [B][H][seq_q][dv] bf16;
 *   dq1, dq2 [B][H][seq_q][d], dk1, dk2 [B][H][seq_k][d], dv [B][H][seq_k][dv]
 *     bf16 (fp32 accumulation, one rounding);
 *   dlambda [H] fp32: summed over the batch and the query rows;
 *   workspace: >= diffattn_bwd_workspace_size(dims) bytes, 16-byte aligned,
 *     contents on entry ignored (DIFFATTN_ERR_WORKSPACE if too small).
 * Same support matrix as diffattn_fwd_train.  Deterministic: no atomics.
 * Allocates nothing.  Returns a DIFFATTN_* status.
 */
int diffattn_bwd(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                 const float* lambda, float lambda_init, int causal, const void* dout,
                 const float* d_save, const float* lse, void* dq1, void* dq2, void* dk1,
                 void* dk2, void* dv, float* dlambda, void* workspace, size_t workspace_bytes,
                 const diffattn_dims* dims, void* stream);

/*
 * Diagnostics of the two softmax maps (bf16; any supported head_dim), the
 * quantities the pages report for trained models (llmbytes.dev, "Benchmark
 * Performance": attention share on needles; "Solving the Quantization
 * Crisis": top attention logit):
 *   row_max [2][B][H][seq_q] fp32 (or NULL): each query row's largest scaled
 *     score q.k/sqrt(d) over the keys it sees, map 1 then map 2;
 *   needles [B][H][n_needles][4] fp32 (or NULL): for planted pair r of a head
 *     (query needle_q[b][h][r], key needle_k[b][h][r], int32 device arrays),
 *     the weight of the pair in A1 and in A2, and the query row's total A1
 *     and A2 weight on all of the head's needle keys it sees; needs lse from
 *     diffattn_fwd_train with the same inputs.  A pair with an index out of
 *     range gets NaNs.  1 <= n_needles <= 4096.
 * At least one of row_max and needles must be given.  Allocates nothing.
 */
int diffattn_diag(const void* q1, const void* q2, const void* k1, const void* k2,
                  const float* lse, int causal, const int32_t* needle_q,
                  const int32_t* needle_k, int32_t n_needles, float* row_max, float* needles,
                  const diffattn_dims* dims, void* stream);

/*
 * Decode: one new query token per (b, h) against a KV cache.  Every cached
 * position of the sequence is visible (the cache already holds the current
 * token), so no mask applies.
 *   q1, q2 [B][H][d]; k1_cache, k2_cache [B][H][kv_capacity][d];
 *   v_cache [B][H][kv_capacity][dv]; out [B][H][dv]; lambda [H] (device).
 *   dims->seq_q must be 1; dims->seq_k = L is the cache length used, with
 *   1 <= L <= kv_capacity.
 *   kv_lens: NULL (every sequence has length L) or a device int32 array [B]
 *   of per-sequence lengths; each is clamped to [0, L], and a sequence of
 *   length 0 gets an all-zero output row.
 *   num_splits: how many pieces each sequence's cache is cut into (split-K);
 *   0 lets the library choose.  With more than one piece, partial results go
 *   to `workspace` (device memory of at least
 *   diffattn_decode_workspace_size(dims, num_splits) bytes, 16-byte aligned,
 *   owned by the caller, contents on entry ignored) and a second kernel merges
 *   them.  workspace may be NULL when that size is 0.
 * Allocates nothing.  Returns a DIFFATTN_* status.
 */
int diffattn_decode(const void* q1, const void* q2, const void* k1_cache,
                    const void* k2_cache, const void* v_cache, int32_t kv_capacity,
                    const int32_t* kv_lens, const float* lambda, float lambda_init,
                    void* out, void* workspace, size_t workspace_bytes,
                    int32_t num_splits, const diffattn_dims* dims, void* stream);

/*
 * Decode that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, results and errors as
 * diffattn_decode, without workspace and workspace_bytes: with more than one
 * split the partial results go to a scratch array the library holds in
 * device memory, DIFFATTN_NOALLOC_SCRATCH_BYTES per GPU, kept until the
 * process ends.  A call whose partials would not fit returns
 * DIFFATTN_ERR_WORKSPACE and launches nothing (ask for fewer splits).  All
 * calls on one GPU share that array, so calls that overlap in time on one
 * GPU (different streams, or threads) race; calls on one stream are
 * ordered.  Nothing in the array needs to start at zero: every record a call
 * reads it has written first.  Calls no allocating routine.
 */
#define DIFFATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int diffattn_decode_noalloc(const void* q1, const void* q2, const void* k1_cache,
                            const void* k2_cache, const void* v_cache, int32_t kv_capacity,
                            const int32_t* kv_lens, const float* lambda, float lambda_init,
                            void* out, int32_t num_splits, const diffattn_dims* dims,
                            void* stream);

/*
 * The split count diffattn_decode uses for num_splits = 0 on the current
 * device (queries the device's compute-unit count once).  Returns a value
 * >= 1, or 0 if dims is invalid or the device cannot be queried.
 */
int32_t diffattn_decode_default_splits(const diffattn_dims* dims);

/*
 * Workspace bytes diffattn_decode needs for these sizes and num_splits
 * (0 = the default count).  0 when no workspace is needed (one split) or
 * when the arguments are invalid.
 */
size_t diffattn_decode_workspace_size(const diffattn_dims* dims, int32_t num_splits);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
