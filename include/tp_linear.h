/*
 * tp_linear.h -- one GPU's shard of a Megatron-style tensor-parallel layer on MI355X (gfx950).
 *
 * The operations follow these pages:
 *   [P3] "Understanding Tensor Parallelism for Multi-GPU LLM Serving" (DevBytes):
 *        section "How Tensor Parallelism Works Under the Hood" (Y = XW; column
 *        parallelism splits W's output dimension, row parallelism its input
 *        dimension and sums the partials) and the ColumnParallelLinear /
 *        RowParallelLinear listing (per-partition sizes = size / world_size,
 *        asserted divisible; the row layer's bias is added once after the sum).
 *   [P4] "What is tensor parallelism?" (tecyfy), section "How a layer is split":
 *        attention heads go to different GPUs; the TP size divides the heads.
 *   [P5] "Tensor parallel serving" (Learn AI): the simulation script (column
 *        shards are W[:split] / W[split:], combined by torch.cat on the last
 *        axis), "Common mistakes" (row shards combine by summing), and the
 *        researcher section (column then row: the intermediate is never
 *        communicated).
 *
 * Conventions for every call:
 *   - A weight is stored [out_features, in_features], row-major (the listing's
 *     layout), so Y = X W of the pages is computed as Y = X * W^T (+ b).
 *   - p = tp_size. Shard r owns the contiguous block [r*n/p, (r+1)*n/p) of the
 *     split dimension.
 *   - Every data pointer is a DEVICE pointer unless marked (host). The caller owns
 *     every buffer; outputs must not alias inputs.
 *   - Tensors are row-major and contiguous unless a leading dimension (ld*) is given.
 *   - dtype TP_DTYPE_BF16: bf16 storage, fp32 accumulation, each output rounded
 *     once to bf16 (round to nearest even). TP_DTYPE_F32: fp32 throughout.
 *   - stream is a hipStream_t (NULL = the null stream). Each call validates its
 *     arguments on the host, enqueues its kernels on `stream` and returns without
 *     synchronising. On any validation error nothing is enqueued and no device
 *     memory is touched.
 *   - Alignment: every base pointer and every row stride in bytes must be a
 *     multiple of 16 (TP_ERR_ALIGN otherwise). For bf16 this means K % 8 == 0,
 *     for fp32 K % 4 == 0, for every row length that is read or written.
 *   - Work space: kernels that split a reduction across workgroups keep fp32
 *     partial sums and arrival counters in a device work space, one per (device,
 *     stream), which the caller reserves once at setup with tp_workspace_reserve
 *     (the only call that allocates; it may synchronise the stream when it
 *     replaces a smaller space). A dry run between tp_plan_begin and tp_plan_end
 *     reports the size a sequence of calls needs. The compute calls never
 *     allocate, free or synchronise: a call whose launches need more work space
 *     than is reserved for its device and stream returns TP_ERR_WORKSPACE having
 *     enqueued nothing. Calls that split no reduction need no reservation. Calls
 *     on one stream are ordered by the stream and share its space; calls on
 *     different streams use different spaces. tp_release_workspaces() frees them.
 *   - Every call checks all of its launches (including their work space) before it
 *     enqueues the first one, so any error leaves the stream untouched.
 *   - Results are deterministic: every reduction runs in a fixed order.
 *   - Errors are returned, never raised; TP_ERR_HIP reports a failed launch or
 *     allocation (hipGetLastError after the launch).
 */
#ifndef TP_LINEAR_H
#define TP_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_DTYPE_F32 = 0,
    TP_DTYPE_BF16 = 1
} tp_dtype_t;

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = 1,        /* a required pointer is NULL */
    TP_ERR_SHAPE = 2,       /* a size <= 0 (M may be 0: nothing is done), ld < width,
                               tp_size outside [1, 64], rank outside [0, tp_size) */
    TP_ERR_INDIVISIBLE = 3, /* a size that is split by tp_size is not divisible by it */
    TP_ERR_DTYPE = 4,       /* unknown dtype, or an fp32 input with bf16 partials */
    TP_ERR_ALIGN = 5,       /* a pointer or row stride is not a multiple of 16 bytes */
    TP_ERR_HIP = 6,         /* the HIP runtime reported an error */
    TP_ERR_WORKSPACE = 7    /* the reserved work space of this device and stream is too small */
} tp_status_t;

/* Column-parallel linear, shard r ([P3] "How ... Under the Hood", column parallelism;
 * [P3] ColumnParallelLinear.forward; [P5] simulation script: each GPU's output is its
 * own weight rows applied to the full input, plus its bias slice).
 *   Y_r[M, out_features/p] = X[M, in_features] * W_r^T + b_r
 *   X   : [M, in_features], the full input, replicated on every shard.
 *   W_r : [out_features/p, in_features], the shard's contiguous block of output rows.
 *   b_r : [out_features/p] or NULL (no bias).
 *   Y_r : [M, out_features/p] output.
 * TP_ERR_INDIVISIBLE if out_features % tp_size != 0 (the listing's assertion). */
tp_status_t tp_linear_col(const void* X, const void* W_r, const void* b_r, void* Y_r,
                          int64_t M, int64_t in_features, int64_t out_features,
                          int32_t tp_size, tp_dtype_t dtype, void* stream);

/* Row-parallel partial, shard r ([P3] row parallelism, RowParallelLinear.forward up to the
 * all-reduce; the bias is NOT applied here -- see tp_combine_sum).
 *   P_r[M, out_features] = X_r[M, in_features/p] * W_r^T
 *   X_r : rows of in_features/p values with row stride ldx (elements, >= in_features/p).
 *         Pass the previous column layer's local output with ldx = in_features/p, or
 *         X + r*in_features/p with ldx = in_features to take the rank's slice of a full X
 *         (the listing's x[..., r*k:(r+1)*k]).
 *   W_r : [out_features, in_features/p], the shard's block of input columns, contiguous.
 *   P_r : [M, out_features] partial, in partial_dtype (bf16 inputs allow bf16 or fp32
 *         partials; fp32 inputs need fp32 partials).
 * TP_ERR_INDIVISIBLE if in_features % tp_size != 0. */
tp_status_t tp_linear_row_partial(const void* X_r, int64_t ldx, const void* W_r, void* P_r,
                                  int64_t M, int64_t in_features, int64_t out_features,
                                  int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype,
                                  void* stream);

/* Paired column -> row MLP shard with SwiGLU ([P3] FFN: column then row; [P5] researcher
 * section "Column-parallel and row-parallel layers, paired": the intermediate stays local).
 *   H_r[M, I/p] = silu(X * Wg_r^T + bg_r) * (X * Wu_r^T + bu_r),  silu(z) = z / (1 + e^-z)
 *   P_r[M, hidden] = H_r * Wd_r^T   (partial, no bias; skipped when P_r is NULL)
 *   X : [M, hidden]; Wg_r, Wu_r : [I/p, hidden]; bg_r, bu_r : [I/p] or NULL (both or neither);
 *   Wd_r : [hidden, I/p] (may be NULL when P_r is NULL); H_r : [M, I/p] output (always
 *   written: it is the row layer's input and the concat check's operand).
 * TP_ERR_INDIVISIBLE if intermediate % tp_size != 0. */
tp_status_t tp_mlp_shard(const void* X, const void* Wg_r, const void* Wu_r,
                         const void* bg_r, const void* bu_r, const void* Wd_r,
                         void* H_r, void* P_r, int64_t M, int64_t hidden, int64_t intermediate,
                         int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype,
                         void* stream);

/* tp_mlp_shard for callers that cannot allocate device memory or reserve a work space
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, validation and results (bitwise) as tp_mlp_shard. Its split reductions
 * take their partial sums and arrival counters from a fixed scratch array inside the
 * library instead of the reserved work space: 16 MiB of partials and 65536 counters, one
 * copy per GPU, held until the process ends (its address is looked up on the first call on
 * each device). It calls no hipMalloc, hipFree or other allocating routine and needs no
 * tp_workspace_reserve. It clears the counters it uses with a small kernel on `stream`
 * before its launches. A call whose launches need more scratch than that (large prefill
 * products split across workgroups) returns TP_ERR_WORKSPACE with nothing enqueued; on a
 * 256-CU MI355X every decode size (M <= 64, up to 2^20 intermediate features per shard)
 * fits. All calls on one GPU share the array: calls that overlap on
 * one GPU (different streams, or several host threads) race and give wrong results. */
tp_status_t tp_mlp_shard_noalloc(const void* X, const void* Wg_r, const void* Wu_r,
                                 const void* bg_r, const void* bu_r, const void* Wd_r,
                                 void* H_r, void* P_r, int64_t M, int64_t hidden, int64_t intermediate,
                                 int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype,
                                 void* stream);

/* The pages' own FFN, shard r ([P3] "Implementing Tensor Parallelism with Hugging Face
 * Accelerate": a ColumnParallelLinear hidden -> intermediate, GELU, a RowParallelLinear
 * intermediate -> hidden; its example is 4096 -> 11008 -> 4096 at batch 4):
 *   H_r[M, I/p]    = gelu(X * W1_r^T + b1_r),  gelu(z) = z * (1 + erf(z / sqrt(2))) / 2
 *   P_r[M, hidden] = H_r * W2_r^T   (partial, no bias; skipped when P_r is NULL)
 *   X : [M, hidden]; W1_r : [I/p, hidden]; b1_r : [I/p] or NULL; W2_r : [hidden, I/p]
 *   (may be NULL when P_r is NULL); H_r is always written. The listing slices the row
 *   layer's input by rank a second time; here the row layer takes the shard's own H_r.
 * TP_ERR_INDIVISIBLE if intermediate % tp_size != 0. Errors as for tp_mlp_shard. */
tp_status_t tp_ffn_gelu_shard(const void* X, const void* W1_r, const void* b1_r, const void* W2_r,
                              void* H_r, void* P_r, int64_t M, int64_t hidden, int64_t intermediate,
                              int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype,
                              void* stream);

/* Head-split attention projections, shard r ([P4] "How a layer is split": heads go to
 * different GPUs and the TP size divides the heads; [P5] one sum per attention block).
 *   QKV_r[M, (Hq/p + 2*G/p)*d] = X * Wqkv_r^T + bqkv_r   (skipped when QKV_r is NULL)
 *       Wqkv_r rows are [Q heads r*Hq/p .. | K heads r*G/p .. | V heads r*G/p ..], each head
 *       head_dim rows, i.e. the output segments are (Hq/p*d, G/p*d, G/p*d).
 *   P_r[M, hidden] = A_r * Wo_r^T   (partial, no bias; skipped when P_r is NULL)
 *       A_r : [M, Hq/p*d], the shard's attention output (its own heads).
 *       Wo_r : [hidden, Hq/p*d], the O projection's input-column block of those heads.
 *   Hq = n_heads, G = n_kv_heads, d = head_dim; bqkv_r may be NULL.
 * TP_ERR_INDIVISIBLE if n_heads % tp_size != 0, or tp_size neither divides n_kv_heads nor is a
 * multiple of it (then each KV head is replicated, as for tp_shard_qkv). */
tp_status_t tp_attn_proj_shard(const void* X, const void* Wqkv_r, const void* bqkv_r, void* QKV_r,
                               const void* A_r, const void* Wo_r, void* P_r,
                               int64_t M, int64_t hidden, int32_t n_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t tp_size, tp_dtype_t dtype,
                               tp_dtype_t partial_dtype, void* stream);

/* Head-local attention core of shard r, between its QKV projection and its O partial
 * (heads go to different GPUs, so no exchange: [P4] "How a layer is split"). The core is
 * not on the pages; this is scaled dot-product attention over the M tokens of one
 * sequence, grouped-query, causal when `causal` != 0:
 *   A_r[:, h*d:(h+1)*d] = softmax(Q_h K_g^T / sqrt(d) (+ mask)) V_g,  g = h / (hq/hk)
 * with Q_h, K_g, V_g the column blocks of QKV_r [M, (hq + 2hk)*d] (segments Q | K | V as
 * tp_attn_proj_shard writes them; hq = n_heads/p, hk = KV heads per shard, replicated as
 * for tp_shard_qkv). A_r : [M, hq*d], the input tp_attn_proj_shard's O half expects.
 * bf16 only (TP_ERR_DTYPE otherwise); head_dim 64 or 128 (TP_ERR_SHAPE otherwise);
 * TP_ERR_INDIVISIBLE if the heads do not split or group evenly. Scores, the softmax and the
 * accumulation are fp32; each softmax weight is rounded to bf16 where it enters the P*V
 * product on the matrix cores (whose operands are bf16), the normaliser sums the fp32
 * weights, and each output is rounded once to bf16. */
tp_status_t tp_attn_core_shard(const void* QKV_r, void* A_r, int64_t M, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t tp_size,
                               int32_t causal, tp_dtype_t dtype, void* stream);

/* One decode step of the head-local attention core over shard r's KV cache (each GPU keeps
 * the keys and values of its own KV heads: [P4] "How a layer is split"; "Why it helps when
 * serving" on the memory that splitting frees for the cache). The new tokens' projections
 * QKV_r [M, (hq + 2hk)*d] (as tp_attn_proj_shard writes them) sit at positions
 * cache_len .. cache_len + M - 1. The call first appends their K and V rows to the caches
 *   K_cache_r, V_cache_r : [capacity, hk*d] token-major (row t = the shard's KV heads at
 *   position t; caller-owned, rows 0 .. cache_len - 1 already filled),
 * then computes, with n = cache_len + M keys and the core's definition (tp_attn_core_shard),
 *   A_r[i, h*d:(h+1)*d] = softmax(Q_h[i] K_g[0 .. cache_len + i]^T / sqrt(d)) V_g[0 .. cache_len + i]
 * i.e. every new token sees the whole cache and the new tokens up to itself. A_r : [M, hq*d].
 * The caller advances cache_len by M afterwards. TP_ERR_SHAPE if cache_len + M > capacity or
 * a K/V cache exceeds 2 GiB; bf16 only; head_dim 64 or 128; the head rules of
 * tp_attn_core_shard. */
tp_status_t tp_attn_decode_shard(const void* QKV_r, void* K_cache_r, void* V_cache_r, int64_t cache_len,
                                 int64_t capacity, void* A_r, int64_t M, int32_t n_heads,
                                 int32_t n_kv_heads, int32_t head_dim, int32_t tp_size,
                                 tp_dtype_t dtype, void* stream);

/* Concat of column-parallel outputs, on one device ([P5] torch.cat([...], dim=-1) and its
 * walkthrough). shards (host array of tp_size device pointers) each hold [M, S] with
 * S = sum(seg_widths) (host array of nseg widths). Segment j of shard r goes to output
 * columns p*(w_0+..+w_{j-1}) + r*w_j .. +w_j, so nseg = 1 is a plain concat in rank order
 * and seg_widths = (Hq/p*d, G/p*d, G/p*d) rebuilds the unsharded [Q | K | V].
 *   Y : [M, p*S]. Pure copy, exact. */
tp_status_t tp_combine_concat(const void* const* shards, int32_t tp_size,
                              const int64_t* seg_widths, int32_t nseg, void* Y, int64_t M,
                              tp_dtype_t dtype, void* stream);

/* Sum of row-parallel partials plus the bias, once ([P3] all_reduce(SUM) then + bias;
 * [P5] "Common mistakes": summing, not concatenating). Computed on one device by reading
 * every shard's partial: Y = sum_{r=0}^{p-1} P_r + b, fp32 accumulation with ranks in
 * ascending order and one rounding to out_dtype.
 *   partials : host array of tp_size device pointers, each [M, N] in partial_dtype.
 *   b : [N] in out_dtype, or NULL.  Y : [M, N] in out_dtype. */
tp_status_t tp_combine_sum(const void* const* partials, int32_t tp_size, tp_dtype_t partial_dtype,
                           const void* b, void* Y, int64_t M, int64_t N, tp_dtype_t out_dtype,
                           void* stream);

/* Take shard `rank` of an unsharded weight into a contiguous buffer ([P3] listing: each GPU
 * stores only its shard; [P5] W[:split], W[split:]).
 *   axis 0 (column-parallel): W_r = W[r*out/p:(r+1)*out/p, :] -> [out/p, in]
 *   axis 1 (row-parallel):    W_r = W[:, r*in/p:(r+1)*in/p]   -> [out, in/p]
 *   A bias is sharded with axis 0 and in_features = 1 (no 16-byte row rule then).
 * TP_ERR_INDIVISIBLE if the split size is not divisible by tp_size; TP_ERR_SHAPE for a bad
 * axis or rank. Exact copy. */
tp_status_t tp_shard_weight(const void* W, int64_t out_features, int64_t in_features,
                            int32_t tp_size, int32_t rank, int32_t axis, void* W_r,
                            tp_dtype_t dtype, void* stream);

/* An uneven split ([P5] "Try it yourself": 9 outputs split 5 + 4 still match exactly): take
 * the block [start, start + width) of W along axis 0 (output rows -> [width, in]) or axis 1
 * (input columns -> [out, width]) into a contiguous buffer. The linear entry points then run
 * the shard with tp_size = 1 and its own width (a row shard reads X + start with ldx = in).
 * TP_ERR_SHAPE if the block leaves W or width <= 0. Exact copy. */
tp_status_t tp_shard_weight_block(const void* W, int64_t out_features, int64_t in_features,
                                  int32_t axis, int64_t start, int64_t width, void* W_r,
                                  tp_dtype_t dtype, void* stream);

/* Concat of an uneven column split: Y[M, sum(widths)] = [shard_0 | shard_1 | ...] with
 * shard r of width widths[r] (host array of n_shards widths; shards: host array of device
 * pointers, each [M, widths[r]]). Pure copy, exact. */
tp_status_t tp_combine_concat_v(const void* const* shards, int32_t n_shards, const int64_t* widths,
                                void* Y, int64_t M, tp_dtype_t dtype, void* stream);

/* Take shard `rank` of a fused [Wq; Wk; Wv] weight ([(Hq + 2G)*d, in_features]) or, with
 * in_features = 1, of its bias ([P4] "How a layer is split": heads go to different GPUs):
 * the rows of Q heads r*Hq/p.., K heads r*G/p.., V heads r*G/p.., in that order ->
 * [(Hq/p + 2G/p)*d, in_features]. With more shards than KV heads (tp_size a multiple of G)
 * each KV head is replicated on p/G consecutive shards: shard r holds KV head floor(r*G/p)
 * and its shard is [(Hq/p + 2)*d, in_features]; the same rule holds for tp_attn_proj_shard.
 * TP_ERR_INDIVISIBLE if p does not divide Hq, or neither divides G nor is a multiple of it.
 * Exact copy. */
tp_status_t tp_shard_qkv(const void* Wqkv, int64_t in_features, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, int32_t tp_size, int32_t rank, void* Wqkv_r,
                         tp_dtype_t dtype, void* stream);

/* Reserves the work space of the current device and `stream` (see the conventions above):
 * at least partial_bytes of fp32 partial sums and n_counters arrival counters. Allocates
 * with hipMalloc and zeroes the counters with a kernel on `stream`; keeps a space that is
 * already large enough; otherwise synchronises `stream`, frees the old space and takes
 * one covering both sizes. Setup only: not to be called while the stream is captured.
 * TP_ERR_HIP if the allocation fails. Inside a dry run it does nothing. */
tp_status_t tp_workspace_reserve(void* stream, size_t partial_bytes, size_t n_counters);

/* Sizes reserved for the current device and `stream` (0, 0 if none). */
tp_status_t tp_workspace_reserved(void* stream, size_t* partial_bytes, size_t* n_counters);

/* Dry run of this host thread: after tp_plan_begin, every call validates its arguments and
 * plans its launches as usual but enqueues nothing and needs no work space; tp_plan_end
 * returns the largest work space any of those calls needs (partial bytes, counters; either
 * pointer may be NULL) and ends the dry run. */
tp_status_t tp_plan_begin(void);
tp_status_t tp_plan_end(size_t* partial_bytes, size_t* n_counters);

/* Frees every work space the library holds (synchronising each space's stream). No call may
 * be in flight on any stream. */
tp_status_t tp_release_workspaces(void);

/* Static, human-readable name of a status code. */
const char* tp_status_string(tp_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* TP_LINEAR_H */
