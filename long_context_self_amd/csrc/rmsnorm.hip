// RMSNorm of the block input, applied as a per-row scale in the Q/K/V
// projection's epilogue (pre-norm): y = x / sqrt(mean_j x_j^2 + eps) * gain.
// The sample's self-attention model lists RMSNorm among its operations
// ("Multi-Device Attention Inference with TensorRT", "Generating the ONNX
// Models", Step 1), and normalisation is local to a token (same page,
// introduction). Since (r_i x_i diag(g)) W = r_i (x_i (diag(g) W)), the gain is
// folded into the packed projection weights once, and the projection scales
// its output row i by r_i = 1 / sqrt(mean_j x_ij^2 + eps): the normalised X is
// never written to memory.
//
// rms_rowscale: HBM-bound row reduction, one wave per token row, 16-byte
// loads, fp32 sum of squares, cross-lane sum by shuffles.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// One wave per row; h is a multiple of 8 (fp16) or 4 (fp32).
__global__ __launch_bounds__(256) void rms_rowscale_f16(const half_t *x, int64_t rows, int h, float eps,
                                                        float *rs) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const half_t *xr = x + row * h;
    float acc = 0.0f;
    for (int c = lane * 8; c < h; c += 64 * 8) {
        const half8 v = as_half8(ldg16(xr + c));
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf((float)v[j], (float)v[j], acc);
    }
    const float ms = wave_sum(acc) / (float)h;
    if (lane == 0) rs[row] = 1.0f / sqrtf(ms + eps);
}

__global__ __launch_bounds__(256) void rms_rowscale_f32(const float *x, int64_t rows, int h, float eps, float *rs) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float *xr = x + row * h;
    float acc = 0.0f;
    for (int c = lane * 4; c < h; c += 64 * 4) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(xr + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = fmaf(v[j], v[j], acc);
    }
    const float ms = wave_sum(acc) / (float)h;
    if (lane == 0) rs[row] = 1.0f / sqrtf(ms + eps);
}

// Packed fp16 Q/K/V weights [n_out][h] (row n = output feature, column k =
// input feature): w[n][k] *= g[k], rounded to fp16 once.
__global__ __launch_bounds__(256) void fold_gain_f16(half_t *w, int64_t n_rows, int h, const half_t *g) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_rows * h) return;
    const int k = (int)(i % h);
    w[i] = (half_t)((float)w[i] * (float)g[k]);
}

// fp32 weights [h][n_out] (row k = input feature): w[k][n] *= g[k].
__global__ __launch_bounds__(256) void fold_gain_f32(float *w, int h, int64_t n_cols, const float *g) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)h * n_cols) return;
    w[i] *= g[i / n_cols];
}

}  // namespace

hipError_t launch_rms_rowscale(const void *x, bool f16, int64_t rows, int h, float eps, float *rs,
                               hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (f16)
        hipLaunchKernelGGL(rms_rowscale_f16, grid, dim3(256), 0, stream, static_cast<const half_t *>(x), rows, h,
                           eps, rs);
    else
        hipLaunchKernelGGL(rms_rowscale_f32, grid, dim3(256), 0, stream, static_cast<const float *>(x), rows, h,
                           eps, rs);
    return hipGetLastError();
}

hipError_t launch_fold_gain(void *w_qkv, bool f16, int h, int64_t n_out, const void *gain, hipStream_t stream) {
    const int64_t n = n_out * h;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (f16)
        hipLaunchKernelGGL(fold_gain_f16, grid, dim3(256), 0, stream, static_cast<half_t *>(w_qkv), n_out, h,
                           static_cast<const half_t *>(gain));
    else
        hipLaunchKernelGGL(fold_gain_f32, grid, dim3(256), 0, stream, static_cast<float *>(w_qkv), h, n_out,
                           static_cast<const float *>(gain));
    return hipGetLastError();
}

}  // namespace attnblk
