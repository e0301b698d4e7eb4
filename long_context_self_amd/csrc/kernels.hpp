// Launch interfaces of the library's kernels (internal; the public C ABI is
// include/attn_block.h). Every launcher assumes its arguments were validated
// by the caller (api.hip) and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"
#include "launch_plan.hpp"

namespace attnblk {

// Most K/V blocks one fp16 attention launch takes (FlashArgs::n_kv_blocks).
constexpr int kMaxKvBlocks = 16;

// Attention over one key range for every head (fp16 path: head_dim 128;
// fp32 path: head_dim 64 or 128). Elements are of the path's dtype.
//   q   (j,i,c) at q[j*q_head_stride + i*D + c], i < sq
//   k   (j,t,c) at k[j*k_head_stride + t*D + c], t < skv
//   vt  (j,c,t) at vt[j*v_head_stride + c*v_row_stride + t]
// Outputs (any may be null): o16/otok token-major [sq][o16_ld] in the path's
// dtype at column head*D; o32 fp32 head-major, row (j, i) at
// o32 + j*o32_head_stride + i*D; lse fp32 at lse[j*lse_head_stride + i]. A
// head stride of 0 means the packed layout ([H][sq][D], [H][sq]).
struct FlashArgs {
    const _Float16 *q;
    const _Float16 *k;
    const _Float16 *vt;
    int64_t q_head_stride, k_head_stride, v_head_stride, v_row_stride;
    int sq, skv, num_heads;
    _Float16 *o16;
    int64_t o16_ld;
    float *o32;
    float *lse;
    int64_t o32_head_stride, lse_head_stride;
    // Key split (0 or 1: none): workgroup item w covers split w / (H * query
    // blocks), keys [split * split_len, min(skv, (split + 1) * split_len)),
    // and writes its partial o32 / lse at split * H * sq * d / split * H * sq
    // (packed layout; the head strides must be 0).
    int n_split, split_len;
    // Non-zero: q holds q_scaled * log2(e) (the block's internal Q), so the
    // softmax works in base 2 with no per-score multiply.
    int q_log2e;
    // Separate K/V blocks (n_kv_blocks > 0; n_split must be 0): workgroup item w
    // covers block b = w / (H * query blocks), whose K and V^T are given by the
    // b-th entries below (k/vt and their strides above are then unused), and
    // writes its partial o32 / lse at b * H * sq * d / b * H * sq (packed).
    int n_kv_blocks;
    const _Float16 *kv_k[kMaxKvBlocks];
    const _Float16 *kv_vt[kMaxKvBlocks];
    int64_t kv_k_head_stride[kMaxKvBlocks], kv_v_head_stride[kMaxKvBlocks], kv_v_row_stride[kMaxKvBlocks];
    int kv_len[kMaxKvBlocks];
    // Non-zero (with n_kv_blocks > 0, q_log2e 0): the blocks are one key
    // sequence of skv keys, block b holding keys [b << kv_lg_len, ...); every
    // block but the last has 2^kv_lg_len >= 64 keys, and all share one V^T row
    // stride. The launch is then an ordinary attention over those keys
    // (outputs as without blocks; n_split splits that sequence).
    int kv_concat, kv_lg_len;
    // 16-row query blocks per wave: 3 (384-row workgroups; also 0) or 2 (256).
    int nq;
};

struct FlashArgsF32 {
    const float *q;
    const float *k;
    const float *vt;
    int64_t q_head_stride, k_head_stride, v_head_stride, v_row_stride;
    int sq, skv, num_heads, head_dim;
    float *otok;
    int64_t otok_ld;
    float *o32;
    float *lse;
};

// C[M][N] = A[M][K] * B^T with B stored [N][K] (fp16, fp32 accumulation).
// mode kPlain: C row-major with ldc. mode kQkv: columns [0,h) are Q (scaled
// by q_scale) -> q [H][seq][d]; [h,2h) are K -> k [H][seq][d]; [2h,3h) are V
// -> vt [H][d][vt_ld] (transposed per head). With q_tap set, Q is also
// written there scaled by q_tap_scale (same layout as q).
enum GemmMode { kPlain = 0, kQkv = 1 };

struct GemmArgs {
    const _Float16 *a;
    int64_t lda;
    const _Float16 *b;
    int64_t ldb;
    int M, N, K;
    int mode;
    _Float16 *c;
    int64_t ldc;
    _Float16 *q;
    _Float16 *k;
    _Float16 *vt;
    int64_t vt_ld;
    int hidden, head_dim;
    float q_scale;
    const float *row_scale;  // nullable: output row m is multiplied by row_scale[m] (RMSNorm pre-norm)
    _Float16 *q_tap;         // nullable
    float q_tap_scale;
};

// fp32 path: C[M][N] = A[M][K] * W[K][N] with W row-major (as given).
struct GemmArgsF32 {
    const float *a;
    int64_t lda;
    const float *w;
    int64_t ldw;
    int M, N, K;
    int mode;
    float *c;
    int64_t ldc;
    float *q;
    float *k;
    float *vt;
    int64_t vt_ld;
    int hidden, head_dim;
    float q_scale;
    const float *row_scale;  // nullable, as in GemmArgs
};

// Batch of equal contiguous segments: segment (o, i), o < n_outer, i < n_inner,
// of chunks_per_seg 16-byte chunks, from src + o*src_so + i*src_si to
// dst + o*dst_so + i*dst_si (byte strides).
struct SegCopyArgs {
    const char *src;
    char *dst;
    uint32_t n_outer, n_inner;
    int64_t src_so, src_si, dst_so, dst_si;
    uint32_t chunks_per_seg;
    // set by the launcher: the 16-byte chunks of all segments form one index
    // space, split evenly over the workgroups
    uint32_t total_chunks;
    FastDiv div_cps, div_inner;
};

struct MergeArgs {
    int n_parts, num_heads, head_dim;
    int64_t sq;
    const float *o_parts;
    const float *lse_parts;
    void *o_out;
    int64_t o_ld;  // row stride of o_out (elements); 0 means num_heads * head_dim
    int64_t o_hs;  // head stride of o_out (elements); 0 means head_dim (heads side by side)
    int out_f16;
    float *lse_out;
    int64_t lse_hs;  // head stride of lse_out; 0 means sq
};

// Workspace budgets of a key-split attention tail (floats of partial rows):
// the block's own workspace, and the one every rank-share partial entry point
// plans with (pool, fixed array or ring alike, so that they all choose the
// same plan and give the same bits).
constexpr int64_t kSplitWsFloats = int64_t(64) << 20;
constexpr int64_t kPartialWsFloats = int64_t(16) << 20;

// The library's stream-ordered memory pool on the current device
// (partial.hip): memory freed on a stream stays in the pool for later calls.
hipError_t staging_pool(hipMemPool_t *out);

hipError_t launch_flash_fwd_f16(const FlashArgs &a, hipStream_t stream);
// Plan for num_heads heads, sq query rows and skv keys whose split workspace
// holds at most max_o_elems floats of partial rows.
AttnPlan plan_attention_f16(int num_heads, int sq, int skv, int64_t max_o_elems);
// The attention of `a` (n_split 0; outputs o16 or o32, and lse) by plan p,
// with ws_o / ws_lse holding p.o_elems / p.lse_elems floats when p splits.
hipError_t launch_attention_f16(const FlashArgs &a, const AttnPlan &p, float *ws_o, float *ws_lse,
                                hipStream_t stream);
hipError_t launch_flash_fwd_f32(const FlashArgsF32 &a, hipStream_t stream);
hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t stream);
hipError_t launch_gemm_f32(const GemmArgsF32 &a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs &a, hipStream_t stream);
// RMSNorm pre-norm: rs[r] = 1 / sqrt(mean_j x[r][j]^2 + eps) for rows x [rows][h]
// (fp16 when f16, else fp32); and w_qkv's input-feature rows scaled by gain.
hipError_t launch_rms_rowscale(const void *x, bool f16, int64_t rows, int h, float eps, float *rs,
                               hipStream_t stream);
hipError_t launch_fold_gain(void *w_qkv, bool f16, int h, int64_t n_out, const void *gain, hipStream_t stream);
hipError_t launch_seg_copy(SegCopyArgs a, hipStream_t stream);
// Batched transpose of 2- or 4-byte elements: for every head b < heads,
// row r < rows and column c < cols, dst[b][c][r] = src[b][r][c], with
//   src element (b, r, c) at src + b*src_hs + r*src_rs + c,
//   dst element (b, c, r) at dst + b*dst_hs + c*dst_rs + r (strides in elements).
// E = 16 / elem_bytes. Each src row must be readable up to round_up(cols, E)
// elements; each dst row is written for r < rows_out (a multiple of E, >= rows),
// zeros past rows. Pointers 16-byte aligned and strides multiples of E.
hipError_t launch_transpose_heads(const void *src, int64_t src_hs, int64_t src_rs, void *dst, int64_t dst_hs,
                                  int64_t dst_rs, int heads, int64_t rows, int64_t rows_out, int64_t cols,
                                  int elem_bytes, hipStream_t stream);
// dst[n][k] = src[k][n] for an [rows][cols] fp16 matrix (dst is [cols][rows]).
hipError_t launch_transpose_f16(const _Float16 *src, int rows, int cols, int64_t ld_src, _Float16 *dst,
                                int64_t ld_dst, hipStream_t stream);

}  // namespace attnblk
