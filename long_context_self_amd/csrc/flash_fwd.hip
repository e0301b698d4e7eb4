// Fused attention forward for gfx950, fp16 inputs, head_dim 128, no mask:
// O = softmax(q_scaled K^T) V per head, plus the natural-log LSE of every row.
//
// Definition: scaled dot-product attention per head over the full key set
// ("Tensor Parallelism: Sharding Weights for Parallel Layer Execution",
// section 3), with the query pre-scaled (q_scaled, "Multi-Device Attention
// Inference with TensorRT", "What is hint.json?"), bidirectional (news summary
// of "Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
// Multi-Device Inference Support", context parallelism). The key loop is the
// online softmax that Ring Attention streams K/V with (same summary, the
// three context-parallel implementations); a call over one K/V block returns
// that block's normalised partial and its LSE.
//
// Design (MI355X):
// * One workgroup = 256 query rows of one head, 8 waves (2 per SIMD), 32 rows
//   per wave. K and V^T tiles of 64 keys are double-buffered in LDS (32 KiB
//   per stage) with XOR swizzles that make every ds_read_b128 conflict-free.
// * S^T = K Q^T on v_mfma_f32_32x32x16_f16 with Q held in registers as the B
//   operand. K rows are read in a permuted order so that each lane's
//   accumulator holds 16 consecutive keys of its own query; those fp32 scores
//   become, after exp and a cast, the B operand of O^T = V^T P^T without any
//   data movement between lanes. V is stored transposed (keys contiguous) so
//   its A operand is one 16-byte LDS read.
// * Softmax in the exp2 domain with the running max and sum in registers; the
//   only cross-lane step per tile is one max between the two lanes that share
//   a query. The O rescale is skipped unless some row's max grew by more than
//   2^8 (exact: O and the sum always share the same reference max).
// * Blocks are remapped so each XCD works through a contiguous range of
//   (head, query block) items and its concurrent workgroups share K/V in L2.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int D = 128;          // head_dim
constexpr int BQ = 256;         // query rows per workgroup
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int BN = 64;          // keys per tile
constexpr int K_TILE = BN * D;  // halves
constexpr int V_TILE = D * BN;  // halves
constexpr float kRescaleTau = 8.0f * kLn2;  // rescale only when a max grows by > 2^8

// Swizzled 16-byte chunk index inside a K row (16 chunks of 8 halves).
__device__ __forceinline__ int swz_k(int row) { return (row & 7) | (((row >> 4) & 1) << 3); }
// Swizzled chunk inside a V^T row (8 chunks of 8 keys).
__device__ __forceinline__ int swz_v(int d) { return (d >> 1) & 7; }
// Accumulator row i of a 32x32 S^T block holds key perm_key(i): lane half h
// then owns keys 16h..16h+15 in accumulator order.
__device__ __forceinline__ int perm_key(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

struct Stage {
    u32x4 k[2];
    u32x4 v[2];
};

// Global -> registers for the tile starting at key0. K rows past skv are
// clamped to the last key (finite values; their scores are masked). V^T keys
// past skv are zero so that masked probabilities multiply zeros.
__device__ __forceinline__ void load_tile(Stage &st, const FlashArgs &a, const half_t *kh,
                                          const half_t *vh, int key0, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        int i = tid + NTHREADS * p;
        int row = i >> 4, c = i & 15;
        int key = min(key0 + row, a.skv - 1);
        st.k[p] = ldg16(kh + (int64_t)key * D + c * 8);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        int i = tid + NTHREADS * p;
        int d = i >> 3, c = i & 7;
        int kstart = key0 + c * 8;
        const half_t *src = vh + (int64_t)d * a.v_row_stride + kstart;
        if (kstart + 8 <= a.skv) {
            st.v[p] = ldg16(src);
        } else {
            half8 t;
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = (kstart + e < a.skv) ? src[e] : (half_t)0.0f;
            st.v[p] = as_u32x4(t);
        }
    }
}

__device__ __forceinline__ void store_tile(const Stage &st, half_t *ks, half_t *vs, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        int i = tid + NTHREADS * p;
        int row = i >> 4, c = i & 15;
        *reinterpret_cast<u32x4 *>(ks + row * D + ((c ^ swz_k(row)) << 3)) = st.k[p];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        int i = tid + NTHREADS * p;
        int d = i >> 3, c = i & 7;
        *reinterpret_cast<u32x4 *>(vs + d * BN + ((c ^ swz_v(d)) << 3)) = st.v[p];
    }
}

template <bool MASK>
__device__ __forceinline__ void tile_step(const half_t *ks, const half_t *vs, const half8 (&qf)[8],
                                          floatx16 (&o)[4], float &m_run, float &l_run, int lane,
                                          int key0, int skv) {
    const int h = lane >> 5;
    // ---- S^T = K Q^T for 64 keys (two 32-key blocks) x 32 queries
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        s[kb] = floatx16{};
        const int row = 32 * kb + perm_key(lane & 31);
        const half_t *krow = ks + row * D;
        const int sw = swz_k(row);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = 2 * kk + h;
            half8 a = *reinterpret_cast<const half8 *>(krow + ((c ^ sw) << 3));
            s[kb] = mfma32(a, qf[kk], s[kb]);
        }
    }
    // ---- mask keys past the end (last tile only)
    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int key = key0 + 32 * kb + 16 * h + i;
                if (key >= skv) s[kb][i] = -INFINITY;
            }
    }
    // ---- row max over this tile (in-lane, then across the two lane halves)
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
    mt = wave_max_across_halves(mt);
    // ---- lazy rescale: only when some row's max grew by more than tau
    const bool need = mt > m_run + kRescaleTau;
    if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb] *= alpha;
    }
    // ---- p = exp(s - m), row sum, fp16 B operand of P^T
    const float mneg = -m_run * kLog2e;
    half8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * t + j], kLog2e, mneg));
                l_run += p;
                pf[kb][t][j] = (half_t)p;
            }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int d = 32 * mb + (lane & 31);
        const half_t *vrow = vs + d * BN;
        const int sw = swz_v(d);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int c = 4 * kb + 2 * h + t;
                half8 a = *reinterpret_cast<const half8 *>(vrow + ((c ^ sw) << 3));
                o[mb] = mfma32(a, pf[kb][t], o[mb]);
            }
    }
}

__global__ __launch_bounds__(NTHREADS) void flash_fwd_f16_d128(FlashArgs a) {
    __shared__ __attribute__((aligned(16))) half_t smem[2 * (K_TILE + V_TILE)];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;

    const int nqb = (a.sq + BQ - 1) / BQ;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int head = work / nqb;
    const int qb = work % nqb;

    const half_t *qh = a.q + (int64_t)head * a.q_head_stride;
    const half_t *kh = a.k + (int64_t)head * a.k_head_stride;
    const half_t *vh = a.vt + (int64_t)head * a.v_head_stride;

    // Q rows of this lane (clamped past the end), as 8 B-operand fragments.
    const int q = qb * BQ + wave * 32 + (lane & 31);
    const int qc = min(q, a.sq - 1);
    half8 qf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = as_half8(ldg16(qh + (int64_t)qc * D + kk * 16 + 8 * h));

    floatx16 o[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) o[mb] = floatx16{};
    float m_run = -INFINITY, l_run = 0.0f;

    const int ntiles = (a.skv + BN - 1) / BN;
    const int nfull = a.skv / BN;
    Stage st;
    if (ntiles > 0) {
        load_tile(st, a, kh, vh, 0, tid);
        store_tile(st, smem, smem + K_TILE, tid);
    }
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        half_t *ks = smem + (j & 1) * (K_TILE + V_TILE);
        half_t *vs = ks + K_TILE;
        const bool more = j + 1 < ntiles;
        if (more) load_tile(st, a, kh, vh, (j + 1) * BN, tid);
        if (j < nfull)
            tile_step<false>(ks, vs, qf, o, m_run, l_run, lane, j * BN, a.skv);
        else
            tile_step<true>(ks, vs, qf, o, m_run, l_run, lane, j * BN, a.skv);
        if (more) {
            half_t *ks2 = smem + ((j + 1) & 1) * (K_TILE + V_TILE);
            store_tile(st, ks2, ks2 + K_TILE, tid);
        }
        __syncthreads();
    }

    if (q >= a.sq) return;
    // ---- epilogue: combine the two lane halves' sums, normalise, store
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = a.skv == 0;
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    if (a.o32) {
        float *dst = a.o32 + ((int64_t)head * a.sq + q) * D;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                floatx4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = o[mb][4 * g + r] * inv;
                *reinterpret_cast<floatx4 *>(dst + 32 * mb + 8 * g + 4 * h) = v;
            }
    }
    if (a.o16) {
        half_t *dst = a.o16 + (int64_t)q * a.o16_ld + (int64_t)head * D;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                half4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (half_t)(o[mb][4 * g + r] * inv);
                *reinterpret_cast<half4 *>(dst + 32 * mb + 8 * g + 4 * h) = v;
            }
    }
    if (a.lse && h == 0) {
        a.lse[(int64_t)head * a.sq + q] =
            empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l_tot) * kLn2;
    }
}

}  // namespace

hipError_t launch_flash_fwd_f16(const FlashArgs &a, hipStream_t stream) {
    if (a.sq <= 0) return hipSuccess;
    const int nqb = (a.sq + BQ - 1) / BQ;
    const int blocks = nqb * a.num_heads;
    hipLaunchKernelGGL(flash_fwd_f16_d128, dim3(blocks), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attnblk
