/*
 * attn_block.h -- C ABI of libattnblock.so: forward pass of a non-causal
 * multi-head self-attention block on AMD Instinct MI355X (gfx950), and the
 * one-GPU share of context-parallel attention (partial results over K/V
 * blocks, merged by log-sum-exp).
 *
 * What is computed (the definitions the library follows):
 *   - The block: Q = X W_Q, K = X W_K, V = X W_V; split into heads; scaled
 *     dot-product attention per head; concatenate the heads and multiply by
 *     W_O. ["Tensor Parallelism: Sharding Weights for Parallel Layer
 *     Execution", section 3 "Parallelizing the Multi-Head Attention Block";
 *     Y = X A for a linear layer, section 1.]
 *   - The query is pre-scaled before the QK^T product (the tensor named
 *     q_scaled), here by 1/sqrt(head_dim); the block has hidden 4096 with 32
 *     heads of 128 and an activation of shape (sequence, batch, hidden) in
 *     fp16. ["Multi-Device Attention Inference with TensorRT", "What is
 *     hint.json?" and "Generating the ONNX Models", Step 1.]
 *   - Attention is bidirectional (no causal mask). A context-parallel rank
 *     keeps its own Q slice and attends either to the gathered full K/V
 *     (AllGather KV) or to K/V streamed in blocks whose results are combined
 *     by online softmax (Ring Attention). [News summary of "Scaling AI
 *     Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device
 *     Inference Support", section on the three context-parallel
 *     implementations.]
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, borrowed: the caller owns them
 *     and keeps them valid until the work enqueued on `stream` completes.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream); nothing blocks the host except attn_block_create and
 *     attn_block_destroy, as stated there.
 *   - Arguments are validated before any HIP call. A non-OK status means
 *     nothing was enqueued (ATTN_E_HIP: a launch was rejected; earlier
 *     launches of the same call may have been enqueued). attn_last_error()
 *     returns a thread-local description of the last non-OK status.
 *   - Faults while the kernels run surface at the caller's next
 *     synchronisation. NaN/Inf inputs are not errors; they propagate.
 *   - Strides and sizes are in ELEMENTS of the tensor's dtype. Floating point
 *     arithmetic accumulates in fp32; ATTN_F16 tensors are IEEE binary16.
 *   - LSE values are natural-log, fp32: lse = m + ln(sum_j exp(s_j - m)).
 *   - No exception, abort or exit crosses this interface.
 */
#ifndef ATTN_BLOCK_H
#define ATTN_BLOCK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_E_INVALID_ARG = 1, /* null pointer, bad size, stride or alignment */
    ATTN_E_UNSUPPORTED = 2, /* valid but not implemented (head_dim, batch, dtype) */
    ATTN_E_OOM = 3,         /* device allocation failed (create calls, attn_partial_forward's staging) */
    ATTN_E_HIP = 4          /* a HIP runtime call or kernel launch failed */
} attn_status_t;

typedef enum {
    ATTN_F16 = 0, /* IEEE binary16; head_dim 128 */
    ATTN_F32 = 1  /* IEEE binary32; head_dim 64 or 128 */
} attn_dtype_t;

/* Opaque block: packed weights plus the workspace of one forward pass. */
typedef struct attn_block attn_block_t;

/* Leading dimension (row stride) of a head-major V^T tensor for `seq` keys:
 * seq rounded up to a multiple of 8, so every row starts 16-byte aligned. */
#define ATTN_VT_LD(seq) ((((int64_t)(seq)) + 7) / 8 * 8)

/*
 * Optional taps of attn_block_forward: caller-owned device buffers that
 * receive the block's intermediates. k, v_t, attn_out and lse replace the
 * block's internal buffers (tapping them costs no copy); taps never change y.
 * Every field may be NULL. Layouts, with S = seq, H = heads, d = head_dim,
 * h = H*d, elements of the block's dtype unless noted:
 *   q_scaled  [H][S][d]   q_scaled = (X W_Q)/sqrt(d), head j = columns j*d..
 *             (fp16 blocks keep their own Q with an extra factor log2(e), the
 *             base change of the softmax's exponential, so this tap costs one
 *             more write of S*h elements from the projection's epilogue)
 *   k         [H][S][d]   K = X W_K, head-major
 *   v_t       [H][d][ATTN_VT_LD(S)]  V = X W_V transposed per head (keys
 *             contiguous); columns S..ld-1 of each row are padding
 *   attn_out  [S][h]      concatenated head outputs before W_O
 *   lse       [H][S]      fp32 natural-log LSE of every query row
 *   qkv_only  non-zero: stop after the QKV projection (q_scaled, k, v_t are
 *             written; attention and the output projection are skipped and
 *             y is not written). This is how the rank share gets its inputs.
 *   events    NULL, or 4 caller-created hipEvent_t recorded on `stream`
 *             before the QKV projection, after it, after attention and after
 *             the output projection (kernel timing in the real launch
 *             configuration). With qkv_only only the first two are recorded.
 *   v         [H][S][d]   V = X W_V head-major, row-major like q_scaled and k
 *             (the layout attn_partial_forward takes). Written by a transpose
 *             of the V^T the projection produces, so it costs one extra pass
 *             over V (read + write of S*h elements) when requested.
 * [Taps of the projection's outputs: "Multi-Device Attention Inference with
 * TensorRT", "What is hint.json?" (the q_scaled tensor feeds QK^T; Q stays
 * local while K/V are gathered, so a rank's inputs are these tensors).]
 */
typedef struct {
    void *q_scaled;
    void *k;
    void *v_t;
    void *attn_out;
    float *lse;
    int qkv_only;
    hipEvent_t *events;
    void *v;
} attn_taps_t;

/*
 * attn_block_create -- pack the four projection weights into library-owned
 * device memory and allocate the workspace for up to max_tokens rows.
 * [The block's weights W_Q, W_K, W_V, W_O applied as Y = X W: "Tensor
 * Parallelism: Sharding Weights for Parallel Layer Execution", section 1 and
 * section 3, steps 1 and 4; hidden 4096 = 32 heads of 128 in fp16:
 * "Multi-Device Attention Inference with TensorRT", "Generating the ONNX
 * Models", Step 1.]
 *   out        receives the block (set to NULL on failure).
 *   hidden     h = num_heads * head_dim; head_dim 128 for ATTN_F16,
 *              64 or 128 for ATTN_F32.
 *   wq,wk,wv,wo device [h][h] row-major in `dt`, applied as Y = X W (input
 *              features along rows). Copied; the caller may free them once
 *              this returns.
 *   max_tokens largest seq*batch any forward will use (>= 1).
 *   stream     used for the packing kernels; synchronised before return.
 * Workspace: about 4 * max_tokens * h elements of `dt`.
 * Errors: ATTN_E_INVALID_ARG (null, h != H*d, max_tokens < 1),
 * ATTN_E_UNSUPPORTED (head_dim, dtype), ATTN_E_OOM, ATTN_E_HIP.
 */
attn_status_t attn_block_create(attn_block_t **out, int hidden, int num_heads, attn_dtype_t dt,
                                const void *wq, const void *wk, const void *wv, const void *wo,
                                int64_t max_tokens, hipStream_t stream);

/*
 * attn_block_create_shard -- like attn_block_create, for one rank's share of
 * tensor parallelism over n_ranks GPUs: W_Q, W_K, W_V are split by columns
 * and W_O by rows, so the rank owns heads [rank*H/N, (rank+1)*H/N) and its
 * forward returns the PARTIAL output y_r = O_r W_O[rows of its heads], the
 * term the all-reduce sums (sum over ranks = the unsharded block's y).
 * ["Tensor Parallelism: Sharding Weights for Parallel Layer Execution",
 * section 1 (column- and row-wise splits of Y = X A) and section 3, steps
 * 1-4 (heads split across GPUs, local attention, row-split W_O, all-reduce).]
 *   hidden, num_heads, dt, max_tokens   as for attn_block_create (the full
 *            block's sizes);
 *   n_ranks  >= 1, divides num_heads;  rank  0 <= rank < n_ranks;
 *   wq,wk,wv,wo  the FULL device [h][h] weights; only the rank's columns of
 *            W_Q/W_K/W_V and rows of W_O are copied (the caller may free them
 *            after the call, which synchronises `stream`).
 * attn_block_forward then takes x [seq][h] (replicated) and writes the
 * partial y [seq][h]; its taps hold the rank's heads only (H/N heads,
 * attn_out [seq][(H/N)*d]). attn_block_set_prenorm applies as for a full block.
 * Errors: those of attn_block_create, plus ATTN_E_INVALID_ARG for n_ranks,
 * rank or num_heads % n_ranks.
 */
attn_status_t attn_block_create_shard(attn_block_t **out, int hidden, int num_heads, int n_ranks, int rank,
                                      attn_dtype_t dt, const void *wq, const void *wk, const void *wv,
                                      const void *wo, int64_t max_tokens, hipStream_t stream);

/*
 * attn_block_set_prenorm -- from now on, every attn_block_forward of `blk`
 * first normalises each token row of x by RMSNorm (pre-norm):
 *   x_i <- x_i / sqrt(mean_j x_ij^2 + eps) * gain.
 * The sample's self-attention model lists RMSNorm among its operations
 * ["Multi-Device Attention Inference with TensorRT", "Generating the ONNX
 * Models", Step 1], and each GPU normalises its own tokens [same page,
 * introduction]; the pages give neither its placement nor eps nor gain, so
 * pre-norm on the block input is this library's reading and eps and gain
 * are arguments (1e-6 and unit gain are the defaults of the reading).
 *   gain  NULL (unit gain) or device [h] in the block's dtype, 4-byte
 *         aligned. Folded once into the packed Q/K/V weights (rounded to the
 *         block's dtype); the call synchronises `stream` before returning and
 *         the caller may then free gain.
 *   eps   finite and >= 0 (rows of zeros with eps = 0 give NaN, which
 *         propagates).
 * The per-row factor 1/sqrt(mean x^2 + eps) is computed by a row-reduction
 * kernel and applied in the projection's epilogue; the normalised x is not
 * written to memory. Allocates max_tokens floats of workspace on first use.
 * Errors: ATTN_E_INVALID_ARG (NULL blk, eps not finite or < 0, pre-norm
 * already enabled on blk), ATTN_E_OOM, ATTN_E_HIP.
 */
attn_status_t attn_block_set_prenorm(attn_block_t *blk, const void *gain, float eps, hipStream_t stream);

/*
 * attn_block_forward -- y = Block(x) for an activation [seq][batch][hidden].
 * [Project to Q, K, V, split heads, scaled dot-product attention per head,
 * concatenate and multiply by W_O: "Tensor Parallelism: Sharding Weights for
 * Parallel Layer Execution", section 3, steps 1-4; q_scaled and the
 * (sequence, batch, hidden) activation: "Multi-Device Attention Inference with
 * TensorRT", "What is hint.json?"; no causal mask: news summary of "Scaling AI
 * Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device
 * Inference Support", context parallelism.]
 *   x, y   device [seq][batch][h] in the block's dtype, 16-byte aligned; x and
 *          y must not overlap. y is not written when taps->qkv_only is set.
 *   seq    0 <= seq*batch <= max_tokens; seq = 0 enqueues nothing.
 *   batch  must be 1 (ATTN_E_UNSUPPORTED otherwise).
 *   taps   NULL, or caller buffers for intermediates (attn_taps_t).
 * Steps on `stream`: (RMSNorm row factors, when pre-norm is enabled); QKV
 * projection with the head split, the 1/sqrt(d) pre-scale (and the RMSNorm
 * row factors) fused into its epilogue; attention of every query row over
 * all seq keys; output projection. Not safe to run concurrently with another
 * forward of the same block (the workspace is shared).
 */
attn_status_t attn_block_forward(attn_block_t *blk, const void *x, void *y, int64_t seq,
                                 int64_t batch, const attn_taps_t *taps, hipStream_t stream);

/*
 * attn_partial_forward -- attention of a query chunk against one block of
 * keys/values, all heads: o_part = softmax(q_scaled K^T) V normalised within
 * the block, and its LSE. With the block being all keys this is the
 * AllGather-KV share; with K/V streamed in blocks it is one Ring step.
 * [A rank keeps its own Q slice and attends to the gathered K/V, or to K/V
 * streamed in blocks combined by online softmax: news summary of "Scaling AI
 * Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device
 * Inference Support", the three context-parallel implementations; q_scaled
 * stays local and K/V are gathered: "Multi-Device Attention Inference with
 * TensorRT", "What is hint.json?".]
 *   num_heads, head_dim, dt  as for the block (d = 128 for ATTN_F16).
 *   q_scaled  element (j,i,c) at q_scaled[j*q_head_stride + i*head_dim + c],
 *             i < sq; already multiplied by 1/sqrt(head_dim).
 *   k, v      element (j,t,c) at k[j*kv_head_stride + t*head_dim + c] and
 *             v[j*kv_head_stride + t*head_dim + c], t < skv (head-major, rows
 *             of head_dim contiguous elements; both use the one head stride).
 *   o_part    fp32 [H][sq][d] (contiguous), normalised within the block.
 *   lse_part  fp32 [H][sq] (contiguous), natural-log.
 * The attention kernel reads V with keys contiguous, so this call first
 * transposes V into a V^T staging buffer taken from a library-owned,
 * stream-ordered device pool (H*d*ATTN_VT_LD(skv) elements, allocated on
 * `stream` and released on it after the kernels; the pool keeps the memory
 * for reuse). That pass reads and writes H*skv*d elements more than
 * attn_partial_forward_vt, which takes V^T directly. Calls on different
 * streams may overlap. In fp16, a call whose grid would leave a last round
 * of workgroups partly idle runs the last query rows of each head as a tail
 * of smaller workgroups, over all keys or split over key ranges and merged by
 * LSE (the same plan for the same num_heads, sq and skv, in every partial
 * entry point and in attn_ring_forward); split partials, at most 64 MiB, come
 * from the same pool.
 * Pointers 16-byte aligned; head strides multiples of 8 (ATTN_F16) or 4
 * (ATTN_F32), q_head_stride >= sq*d and kv_head_stride >= skv*d when
 * num_heads > 1. sq = 0 enqueues nothing. skv = 0 writes o_part = 0 and
 * lse_part = -inf (a block with no keys, which carries zero weight in
 * attn_merge_lse). Errors: ATTN_E_INVALID_ARG, ATTN_E_UNSUPPORTED, ATTN_E_OOM
 * (the staging buffer), ATTN_E_HIP.
 */
attn_status_t attn_partial_forward(int num_heads, int head_dim, attn_dtype_t dt,
                                   const void *q_scaled, int64_t sq, int64_t q_head_stride,
                                   const void *k, const void *v, int64_t skv, int64_t kv_head_stride,
                                   float *o_part, float *lse_part, hipStream_t stream);

/*
 * attn_partial_forward_vt -- attn_partial_forward with V given transposed per
 * head (keys contiguous), the layout the block's projection writes (the v_t
 * tap) and the attention kernel reads, so no staging pass.
 * [Same definition and sources as attn_partial_forward.]
 *   k         element (j,t,c) at k[j*k_head_stride + t*head_dim + c], t < skv.
 *   v_t       element (j,c,t) at v_t[j*v_head_stride + c*v_row_stride + t]
 *             (V transposed per head: keys contiguous).
 * Other arguments, outputs and errors as for attn_partial_forward
 * (ATTN_E_OOM only from the split partials of the fp16 plan). v_row_stride >=
 * skv and a multiple of 8 (ATTN_F16) or 4 (ATTN_F32).
 */
attn_status_t attn_partial_forward_vt(int num_heads, int head_dim, attn_dtype_t dt,
                                      const void *q_scaled, int64_t sq, int64_t q_head_stride,
                                      const void *k, int64_t skv, int64_t k_head_stride,
                                      const void *v_t, int64_t v_head_stride, int64_t v_row_stride,
                                      float *o_part, float *lse_part, hipStream_t stream);

/*
 * attn_partial_forward_noalloc -- attn_partial_forward for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the V^T staging (up to 64 MiB)
 * and the split partials of the fp16 plan (up to 64.5 MiB) live in a fixed
 * 128.5 MiB device array of the library instead of the stream-ordered pool,
 * and the call makes no allocation of any kind.
 *   Arguments, layouts and results: as attn_partial_forward (bit-identical
 *   output).
 *   Limit: num_heads * head_dim * ATTN_VT_LD(skv) * element size <= 64 MiB
 *   (e.g. 32 heads of 128 in fp16: skv <= 8192); larger calls return
 *   ATTN_E_UNSUPPORTED, enqueue nothing, and should use attn_partial_forward.
 *   Each GPU the library runs on holds its own copy of the array until the
 *   process ends; its device address is looked up once per device, on the
 *   first call made with that device current.
 *   All calls on one GPU share that GPU's array: calls that overlap in time
 *   on one GPU (two streams, or two host threads) race on it. Calls ordered on
 *   one stream do not.
 * Errors: those of attn_partial_forward except ATTN_E_OOM.
 */
attn_status_t attn_partial_forward_noalloc(int num_heads, int head_dim, attn_dtype_t dt,
                                           const void *q_scaled, int64_t sq, int64_t q_head_stride,
                                           const void *k, const void *v, int64_t skv, int64_t kv_head_stride,
                                           float *o_part, float *lse_part, hipStream_t stream);

/*
 * attn_heads_forward -- attention of num_heads heads over the full sequence,
 * output token-major: o[i][j*d + c] for row i, head j. This is the block's
 * attention step on its own; under Ulysses context parallelism a rank runs it
 * on its subset of heads for every row of the sequence. [Scaled dot-product
 * attention per head, "Tensor Parallelism: Sharding Weights for Parallel
 * Layer Execution", section 3, step 3; Ulysses: news summary of "Scaling AI
 * Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device
 * Inference Support", the three context-parallel implementations.]
 *   q_scaled, k  [H][seq][d] contiguous (q already times 1/sqrt(d));
 *   v_t          [H][d][ATTN_VT_LD(seq)] (V transposed per head);
 *   o            [seq][o_ld] in dt, o_ld >= H*d and a multiple of 8 (fp16)
 *                or 4 (fp32);
 *   lse          NULL or fp32 [H][seq], natural-log.
 * head_dim 128 (ATTN_F16) or 64/128 (ATTN_F32); pointers 16-byte aligned.
 * seq = 0 enqueues nothing. In fp16, when the grid would leave a last round
 * of workgroups partly idle, the last query rows of each head run as a tail of
 * smaller workgroups, over all keys or split over key ranges and merged by LSE;
 * split partials (at most 256 MiB) come from the library's stream-ordered
 * pool, allocated and released on `stream`.
 * Errors: ATTN_E_INVALID_ARG, ATTN_E_UNSUPPORTED, ATTN_E_OOM (the split
 * partials), ATTN_E_HIP.
 */
attn_status_t attn_heads_forward(int num_heads, int head_dim, attn_dtype_t dt, const void *q_scaled,
                                 const void *k, const void *v_t, int64_t seq, void *o, int64_t o_ld,
                                 float *lse, hipStream_t stream);

/*
 * attn_ulysses_gather -- receive side of Ulysses' first all-to-all. Rank p
 * holds rows [p*S/N, (p+1)*S/N) and projects them head-major; the slice of
 * its heads that belongs to rank r is contiguous, and the all-to-all delivers
 * it to r as block p. This call lays rank r's N blocks out as the full
 * sequence of its H/N heads, ready for attn_heads_forward. [News summary of
 * "Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
 * Multi-Device Inference Support", the three context-parallel
 * implementations (DeepSpeed Ulysses: all-to-all on Q, K, V; every GPU gets
 * the whole sequence for a subset of heads).]
 *   n_ranks N >= 1; num_heads_local Hl = H/N; seq S with S/N a multiple of 8.
 *   recv_q, recv_k  [N][Hl][S/N][d];   recv_vt  [N][Hl][d][S/N]
 *   q_scaled, k     [Hl][S][d];        v_t      [Hl][d][ATTN_VT_LD(S)] (= S)
 * Pure data movement (bit-exact). Buffers 16-byte aligned, not overlapping.
 */
attn_status_t attn_ulysses_gather(int n_ranks, int num_heads_local, int head_dim, attn_dtype_t dt, int64_t seq,
                                  const void *recv_q, const void *recv_k, const void *recv_vt,
                                  void *q_scaled, void *k, void *v_t, hipStream_t stream);

/*
 * attn_ulysses_unpack_o -- receive side of Ulysses' second all-to-all. Rank r
 * writes its heads' output token-major [S][Hl*d]; rows [p*S/N, (p+1)*S/N) of
 * it go back to rank p, which receives N such blocks, one per r. This call
 * puts rank p's blocks in the concatenated-heads layout [S/N][H*d] that the
 * output projection reads (block r fills columns [r*Hl*d, (r+1)*Hl*d)).
 * [Same source: a second all-to-all restores the head and sequence layout.]
 *   n_ranks N; num_heads H (a multiple of N); rows = S/N.
 *   recv_o  [N][rows][(H/N)*d];  o  [rows][H*d].  Bit-exact data movement.
 */
attn_status_t attn_ulysses_unpack_o(int n_ranks, int num_heads, int head_dim, attn_dtype_t dt, int64_t rows,
                                    const void *recv_o, void *o, hipStream_t stream);

/*
 * attn_merge_lse -- combine n_parts partial results of the same query rows
 * by log-sum-exp: with M = max_b lse_b, lse = M + ln sum_b exp(lse_b - M)
 * and o = sum_b exp(lse_b - lse) o_b (online softmax across blocks).
 * [Blocks of K/V combined by online softmax (Ring Attention): news summary
 * of "Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
 * Multi-Device Inference Support", the three context-parallel
 * implementations; the output is the concatenation of the heads that W_O
 * multiplies: "Tensor Parallelism: Sharding Weights for Parallel Layer
 * Execution", section 3, step 4.]
 * Parts are summed in index order 0..n_parts-1 (deterministic).
 *   o_parts   fp32 [n_parts][H][sq][d] contiguous, each normalised in its block.
 *   lse_parts fp32 [n_parts][H][sq] contiguous.
 *   o_out     [sq][H*d] token-major in out_dt (the concatenated-heads layout
 *             the output projection consumes).
 *   lse_out   NULL or fp32 [H][sq].
 * Rows whose parts all have lse = -inf get o = 0 and lse = -inf.
 * Pointers 16-byte aligned (o_out 8-byte aligned for ATTN_F16).
 */
attn_status_t attn_merge_lse(int n_parts, int num_heads, int head_dim, int64_t sq,
                             const float *o_parts, const float *lse_parts,
                             void *o_out, attn_dtype_t out_dt, float *lse_out,
                             hipStream_t stream);

/*
 * attn_ring_t -- Ring-style streaming of K/V blocks on one GPU. K/V blocks
 * arrive by asynchronous copy on the ring's own copy stream while the
 * attention of the blocks already in place runs on the caller's stream; the
 * per-block partial results are merged by log-sum-exp. [Ring Attention:
 * K/V streamed around the GPUs, local Q computation overlapped with the
 * transfer, blocks combined by online softmax, the full K/V never resident --
 * news summary of "Scaling AI Inference Across Multiple GPUs Using NVIDIA
 * TensorRT with Multi-Device Inference Support", the three context-parallel
 * implementations.]
 *
 * attn_ring_create -- allocate two staging slots (K [H][max_block_len][d] and
 * V^T [H][d][ATTN_VT_LD(max_block_len)]), n_blocks partial results for up to
 * max_sq query rows (fp32, about n_blocks*H*max_sq*d*4 bytes), a copy stream
 * (default priority) and its events. Errors: ATTN_E_INVALID_ARG,
 * ATTN_E_UNSUPPORTED (head_dim, dtype, sizes), ATTN_E_OOM, ATTN_E_HIP.
 */
typedef struct attn_ring attn_ring_t;
attn_status_t attn_ring_create(attn_ring_t **out, int num_heads, int head_dim, attn_dtype_t dt, int n_blocks,
                               int64_t max_sq, int64_t max_block_len);

/*
 * attn_ring_forward -- o = softmax(q_scaled K^T) V over the keys of all
 * n_blocks blocks, for sq query rows, all heads.
 *   q_scaled    device [H][sq][d] (times 1/sqrt(d)), 16-byte aligned.
 *   k_blocks[b] [H][len_b][d] and vt_blocks[b] [H][d][ATTN_VT_LD(len_b)]:
 *               block b as its owner holds it (e.g. the taps of its
 *               projection); device memory or pinned host memory (a
 *               stand-in for a peer's link). Host arrays of n_blocks entries.
 *   block_lens  host array, 0 <= len_b <= max_block_len (0: an empty block).
 *   o_out       device [sq][H*d] token-major in dt; lse_out NULL or fp32 [H][sq].
 * A block whose K and V^T are both in this device's memory is read in place.
 * Any other block is copied into slot b % 2 on the copy stream once the
 * partial of the block that used the slot before has finished on `stream`, so
 * the copy of block b+1 overlaps the partial of block b; `stream` waits for
 * each copied block's arrival. The copies of
 * a call start after the work already enqueued on `stream`; calls on one ring
 * must use one stream (or be ordered by the caller). The result equals
 * attn_partial_forward over each block followed by attn_merge_lse, bit for bit
 * when some block must be copied. When every block already sits in this
 * device's memory (fp16, n_blocks <= 16) one launch does the work: blocks of
 * one power-of-two length (>= 64) are read as a single key sequence (the
 * result equals attn_partial_forward_vt over the concatenated K/V, rounded to
 * fp16, bit for bit); other blocks get one partial each, each over its whole
 * key range, then the merge (equal to the per-block calls bit for bit below
 * 1024 keys per block). Either way the result meets the split-merge gate
 * against the per-block calls, whose plans may split a block's last query
 * rows over key ranges.
 */
attn_status_t attn_ring_forward(attn_ring_t *ring, const void *q_scaled, int64_t sq,
                                const void *const *k_blocks, const void *const *vt_blocks,
                                const int64_t *block_lens, void *o_out, float *lse_out, hipStream_t stream);

/* attn_ring_destroy -- synchronise the ring's device and free it. NULL is a no-op. */
void attn_ring_destroy(attn_ring_t *ring);

/* attn_block_destroy -- synchronise the block's device and free everything
 * the block owns. NULL is a no-op. [Borrowed resources outlive their user,
 * as an execution context's communicator must stay valid while the context
 * lives: news summary of "Scaling AI Inference Across Multiple GPUs Using
 * NVIDIA TensorRT with Multi-Device Inference Support", the paragraph on
 * running the engine; the block owns only what create made.] */
void attn_block_destroy(attn_block_t *blk);

/* attn_last_error -- thread-local, NUL-terminated text for the last non-OK
 * status returned on this thread ("" if none). Valid until the next call.
 * [Library convention: the pages define no error interface.] */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BLOCK_H */
