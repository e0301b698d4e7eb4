// Launch interfaces of the library's kernels (internal; the public C ABI is
// include/attn_block.h). Every launcher assumes its arguments were validated
// by the caller (api.hip) and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace attnblk {

// Attention over one key range for every head (fp16 path: head_dim 128;
// fp32 path: head_dim 64 or 128). Elements are of the path's dtype.
//   q   (j,i,c) at q[j*q_head_stride + i*D + c], i < sq
//   k   (j,t,c) at k[j*k_head_stride + t*D + c], t < skv
//   vt  (j,c,t) at vt[j*v_head_stride + c*v_row_stride + t]
// Outputs (any may be null): o16/otok token-major [sq][o16_ld] in the path's
// dtype at column head*D; o32 fp32 [H][sq][D]; lse fp32 [H][sq].
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
    // Key split (0 or 1: none): workgroup item w covers split w / (H * query
    // blocks), keys [split * split_len, min(skv, (split + 1) * split_len)),
    // and writes its partial o32 / lse at split * H * sq * d / split * H * sq.
    int n_split, split_len;
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
// -> vt [H][d][vt_ld] (transposed per head).
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
    int out_f16;
    float *lse_out;
};

hipError_t launch_flash_fwd_f16(const FlashArgs &a, hipStream_t stream);
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
// dst[n][k] = src[k][n] for an [rows][cols] fp16 matrix (dst is [cols][rows]).
hipError_t launch_transpose_f16(const _Float16 *src, int rows, int cols, int64_t ld_src, _Float16 *dst,
                                int64_t ld_dst, hipStream_t stream);

}  // namespace attnblk
