// Log-sum-exp merge of per-block partial attention results (the combine step
// of the online softmax that Ring Attention streams K/V with; news summary of
// "Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
// Multi-Device Inference Support", three context-parallel implementations):
//   M = max_b lse_b, w_b = exp(lse_b - M), lse = M + ln sum_b w_b,
//   o = (sum_b w_b o_b) / sum_b w_b.
// Output rows are written token-major [sq][H*d] by default -- the
// concatenated-heads layout the output projection reads ("Tensor Parallelism:
// Sharding Weights for Parallel Layer Execution", section 3) -- or with any
// row and head strides.
//
// HBM-bound: each thread owns four consecutive head dimensions of one
// (head, query) row, so every part is read in 16-byte coalesced chunks (four
// parts in flight per thread) and each part's LSE is read once per row from
// cache. Parts are summed in index order, so the result is deterministic.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int kBatch = 4;  // parts whose loads are in flight together

__global__ __launch_bounds__(256) void lse_merge(MergeArgs a) {
    const int tpr = a.head_dim / 4;  // threads per row
    const int rows_per_block = 256 / tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / tpr;
    const int t = threadIdx.x % tpr;
    const int64_t nrows = (int64_t)a.num_heads * a.sq;
    if (row >= nrows) return;
    const int head = (int)(row / a.sq);
    const int64_t q = row % a.sq;
    const int64_t part_stride_o = nrows * a.head_dim;

    float m = -INFINITY;
    for (int b = 0; b < a.n_parts; ++b) m = fmaxf(m, a.lse_parts[b * nrows + row]);

    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float lse;
    if (m == -INFINITY) {
        lse = -INFINITY;
    } else {
        // Parts go kBatch at a time: their loads are all issued before the
        // first is used, so each thread keeps kBatch 16-byte reads in flight.
        // The sums still run in part order.
        float total = 0.0f;
        for (int b0 = 0; b0 < a.n_parts; b0 += kBatch) {
            float l[kBatch];
            floatx4 v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j < a.n_parts) {
                    l[j] = a.lse_parts[(b0 + j) * nrows + row];
                    v[j] = *reinterpret_cast<const floatx4 *>(a.o_parts + (b0 + j) * part_stride_o + row * a.head_dim +
                                                             4 * t);
                }
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j < a.n_parts) {
                    const float w = expf(l[j] - m);
                    total += w;
                    acc += w * v[j];
                }
            }
        }
        acc *= 1.0f / total;
        lse = m + logf(total);
    }
    const int64_t ocol = (int64_t)head * (a.o_hs ? a.o_hs : a.head_dim) + 4 * t;
    const int64_t ld = a.o_ld ? a.o_ld : (int64_t)a.num_heads * a.head_dim;
    if (a.out_f16) {
        half4 hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (half_t)acc[r];
        *reinterpret_cast<half4 *>(reinterpret_cast<half_t *>(a.o_out) + q * ld + ocol) = hv;
    } else {
        *reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(a.o_out) + q * ld + ocol) = acc;
    }
    if (a.lse_out && t == 0) a.lse_out[(int64_t)head * (a.lse_hs ? a.lse_hs : a.sq) + q] = lse;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs &a, hipStream_t stream) {
    const int64_t nrows = (int64_t)a.num_heads * a.sq;
    if (nrows <= 0) return hipSuccess;
    const int rows_per_block = 256 / (a.head_dim / 4);
    const int64_t blocks = (nrows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(lse_merge, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attnblk
