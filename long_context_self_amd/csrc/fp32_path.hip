// fp32 instantiation of the block for small configurations (hidden 256,
// 4 heads of 64 in the tiny case): the same steps as the fp16 path -- QKV
// projection with the q_scaled pre-scale, head split and V transpose in the
// epilogue; attention with a streaming (online) softmax over the keys;
// output projection -- in plain fp32 FMA arithmetic.
// Definitions: "Tensor Parallelism: Sharding Weights for Parallel Layer
// Execution", sections 1 and 3; q_scaled: "Multi-Device Attention Inference
// with TensorRT", "What is hint.json?"; online softmax over streamed K/V:
// news summary of "Scaling AI Inference Across Multiple GPUs Using NVIDIA
// TensorRT with Multi-Device Inference Support", three context-parallel
// implementations.
//
// These shapes are launch-bound, so the kernels favour simplicity: a 64x64
// LDS-tiled SIMT GEMM and an attention kernel with four lanes per query row.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;

__global__ __launch_bounds__(256) void gemm_f32_nn(GemmArgsF32 g) {
    __shared__ float as[TK][TM + 4];
    __shared__ float ws[TK][TN + 4];
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += TK) {
        for (int i = threadIdx.x; i < TM * TK; i += 256) {
            int r = i / TK, c = i % TK;
            int m = m0 + r, k = k0 + c;
            as[c][r] = (m < g.M && k < g.K) ? g.a[(int64_t)m * g.lda + k] : 0.0f;
        }
        for (int i = threadIdx.x; i < TK * TN; i += 256) {
            int r = i / TN, c = i % TN;
            int k = k0 + r, n = n0 + c;
            ws[r][c] = (k < g.K && n < g.N) ? g.w[(int64_t)k * g.ldw + n] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float av[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m >= g.M || n >= g.N) continue;
            const float v = g.row_scale ? acc[i][j] * g.row_scale[m] : acc[i][j];
            if (g.mode == kPlain) {
                g.c[(int64_t)m * g.ldc + n] = v;
            } else {
                const int region = n / g.hidden;
                const int nn = n - region * g.hidden;
                const int head = nn / g.head_dim, dd = nn % g.head_dim;
                if (region == 0)
                    g.q[((int64_t)head * g.M + m) * g.head_dim + dd] = v * g.q_scale;
                else if (region == 1)
                    g.k[((int64_t)head * g.M + m) * g.head_dim + dd] = v;
                else
                    g.vt[((int64_t)head * g.head_dim + dd) * g.vt_ld + m] = v;
            }
        }
}

// Four lanes per query row, each owning D/4 of the head dimensions. Keys are
// staged 64 at a time in LDS; every key updates the running max m, the
// running sum l and the output o of the row (the textbook streaming form).
template <int D>
__global__ __launch_bounds__(256) void flash_fwd_f32(FlashArgsF32 a) {
    constexpr int QPB = 64;  // queries per block
    constexpr int KT = 64;   // keys per LDS tile
    constexpr int DQ = D / 4;
    __shared__ float ks[KT][D + 1];
    __shared__ float vs[KT][D + 1];
    const int nqb = (a.sq + QPB - 1) / QPB;
    const int head = blockIdx.x / nqb, qb = blockIdx.x % nqb;
    const int qi = qb * QPB + threadIdx.x / 4;
    const int part = threadIdx.x % 4;
    const int qc = min(qi, a.sq - 1);
    const float *qrow = a.q + (int64_t)head * a.q_head_stride + (int64_t)qc * D + part * DQ;
    float q[DQ], o[DQ];
#pragma unroll
    for (int c = 0; c < DQ; ++c) {
        q[c] = qrow[c];
        o[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const float *kh = a.k + (int64_t)head * a.k_head_stride;
    const float *vh = a.vt + (int64_t)head * a.v_head_stride;
    for (int t0 = 0; t0 < a.skv; t0 += KT) {
        const int nt = min(KT, a.skv - t0);
        __syncthreads();
        for (int i = threadIdx.x; i < KT * D; i += 256) {
            int t = i / D, c = i % D;
            ks[t][c] = t < nt ? kh[(int64_t)(t0 + t) * D + c] : 0.0f;
        }
        for (int i = threadIdx.x; i < KT * D; i += 256) {
            int c = i / KT, t = i % KT;
            vs[t][c] = t < nt ? vh[(int64_t)c * a.v_row_stride + t0 + t] : 0.0f;
        }
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < DQ; ++c) s = fmaf(q[c], ks[t][part * DQ + c], s);
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            if (s > m) {
                const float alpha = expf(m - s);
                l *= alpha;
#pragma unroll
                for (int c = 0; c < DQ; ++c) o[c] *= alpha;
                m = s;
            }
            const float p = expf(s - m);
            l += p;
#pragma unroll
            for (int c = 0; c < DQ; ++c) o[c] = fmaf(p, vs[t][part * DQ + c], o[c]);
        }
    }
    if (qi >= a.sq) return;
    const bool empty = a.skv == 0;
    const float inv = empty ? 0.0f : 1.0f / l;
    if (a.o32) {
        float *dst = a.o32 + ((int64_t)head * a.sq + qi) * D + part * DQ;
#pragma unroll
        for (int c = 0; c < DQ; ++c) dst[c] = o[c] * inv;
    }
    if (a.otok) {
        float *dst = a.otok + (int64_t)qi * a.otok_ld + (int64_t)head * D + part * DQ;
#pragma unroll
        for (int c = 0; c < DQ; ++c) dst[c] = o[c] * inv;
    }
    if (a.lse && part == 0) a.lse[(int64_t)head * a.sq + qi] = empty ? -INFINITY : m + logf(l);
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgsF32 &g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    dim3 grid((g.N + TN - 1) / TN, (g.M + TM - 1) / TM);
    hipLaunchKernelGGL(gemm_f32_nn, grid, dim3(256), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_flash_fwd_f32(const FlashArgsF32 &a, hipStream_t stream) {
    if (a.sq <= 0) return hipSuccess;
    const int blocks = ((a.sq + 63) / 64) * a.num_heads;
    if (a.head_dim == 64)
        hipLaunchKernelGGL(flash_fwd_f32<64>, dim3(blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(flash_fwd_f32<128>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attnblk
