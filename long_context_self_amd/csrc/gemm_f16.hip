// fp16 GEMM for gfx950 with fp32 accumulation: C = A B^T, A [M][K], B [N][K]
// (both K-contiguous), used for the block's two projections:
//   * QKV projection  [Q|K|V] = X [W_Q|W_K|W_V]  (B = the packed transpose),
//     with the head split, the 1/sqrt(d) pre-scale of Q (q_scaled) and the
//     per-head transpose of V fused into the epilogue;
//   * output projection Y = Concat(heads) W_O.
// Definitions: "Tensor Parallelism: Sharding Weights for Parallel Layer
// Execution", section 3 (projections, head split, concat, W_O) and section 1
// (Y = X A); q_scaled: "Multi-Device Attention Inference with TensorRT",
// "What is hint.json?".
//
// Design (MI355X): 256x256 tile per workgroup, 8 waves (2 per SIMD) of
// 128x64 each on v_mfma_f32_32x32x16_f16, K in steps of 32 double-buffered
// through LDS with an XOR swizzle (conflict-free ds_read_b128), global loads
// for step k+1 in flight during the MFMAs of step k. Tiles are grouped 4 deep
// in M and each XCD gets a contiguous range of tiles so its L2 holds the A
// and B panels its workgroups share. The epilogue stages the fp16 tile in
// LDS (transposed for V) and writes 16-byte chunks.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NTHREADS = 512;
constexpr int GROUP_M = 4;
constexpr int A_TILE = BM * BK;  // halves
constexpr int B_TILE = BN * BK;
constexpr int CP = BN + 8;       // epilogue pitch (halves)
constexpr int SMEM_MAIN = 2 * (A_TILE + B_TILE) * 2;  // bytes
constexpr int SMEM_EPI = BM * CP * 2;
constexpr int SMEM_BYTES = SMEM_MAIN > SMEM_EPI ? SMEM_MAIN : SMEM_EPI;

// 64-byte rows of 4 chunks; chunk c of row r lives at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

struct Stage {
    u32x4 a[2];
    u32x4 b[2];
};

__device__ __forceinline__ void load_stage(Stage &st, const GemmArgs &g, int m0, int n0, int k0, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        int i = tid + NTHREADS * p;
        int row = i >> 2, c = i & 3;
        int m = min(m0 + row, g.M - 1);
        st.a[p] = ldg16(g.a + (int64_t)m * g.lda + k0 + c * 8);
        int n = min(n0 + row, g.N - 1);
        st.b[p] = ldg16(g.b + (int64_t)n * g.ldb + k0 + c * 8);
    }
}

__device__ __forceinline__ void store_stage(const Stage &st, half_t *as, half_t *bs, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        int i = tid + NTHREADS * p;
        int row = i >> 2, c = i & 3;
        int off = row * BK + ((c ^ swz(row)) << 3);
        *reinterpret_cast<u32x4 *>(as + off) = st.a[p];
        *reinterpret_cast<u32x4 *>(bs + off) = st.b[p];
    }
}

__global__ __launch_bounds__(NTHREADS) void gemm_f16_nt(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char smem_raw[SMEM_BYTES];
    half_t *smem = reinterpret_cast<half_t *>(smem_raw);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int wm = wave >> 2;  // 0..1 -> rows wm*128
    const int wn = wave & 3;   // 0..3 -> cols wn*64

    // ---- tile order: XCD-contiguous ranges, then groups of GROUP_M tile rows
    const int tiles_m = (g.M + BM - 1) / BM;
    const int tiles_n = (g.N + BN - 1) / BN;
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int per_group = GROUP_M * tiles_n;
    const int group = w / per_group;
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (w % per_group) % gsize;
    const int tn = (w % per_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

    const int nk = g.K / BK;
    Stage st;
    load_stage(st, g, m0, n0, 0, tid);
    store_stage(st, smem, smem + A_TILE, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const half_t *as = smem + (kt & 1) * (A_TILE + B_TILE);
        const half_t *bs = as + A_TILE;
        const bool more = kt + 1 < nk;
        if (more) load_stage(st, g, m0, n0, (kt + 1) * BK, tid);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = 2 * kk + h;
            half8 af[4], bf[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int row = wm * 128 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const half8 *>(as + row * BK + ((c ^ swz(row)) << 3));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int row = wn * 64 + j * 32 + (lane & 31);
                bf[j] = *reinterpret_cast<const half8 *>(bs + row * BK + ((c ^ swz(row)) << 3));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
        }
        if (more) {
            half_t *as2 = smem + ((kt + 1) & 1) * (A_TILE + B_TILE);
            store_stage(st, as2, as2 + A_TILE, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: stage the fp16 tile in LDS, then 16-byte stores
    const bool v_tile = g.mode == kQkv && n0 >= 2 * g.hidden;
    // A tile may straddle the Q|K border at column h (odd head counts), so the
    // pre-scale is chosen per column; the V border 2h is a multiple of 256.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = wn * 64 + j * 32 + (lane & 31);
            const float sc = (g.mode == kQkv && n0 + col < g.hidden) ? g.q_scale : 1.0f;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int row = wm * 128 + i * 32 + 8 * gg + 4 * h;
                if (v_tile) {
                    half4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = (half_t)acc[i][j][4 * gg + r];
                    *reinterpret_cast<half4 *>(smem + col * CP + row) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) smem[(row + r) * CP + col] = (half_t)(acc[i][j][4 * gg + r] * sc);
                }
            }
        }
    __syncthreads();
#pragma unroll 4
    for (int p = 0; p < (BM * BN / 8) / NTHREADS; ++p) {
        const int i = tid + NTHREADS * p;
        const int r = i >> 5, cc = i & 31;  // r: LDS row, cc: 8-element chunk
        const u32x4 val = *reinterpret_cast<const u32x4 *>(smem + r * CP + cc * 8);
        if (v_tile) {
            // LDS row r is feature n0 + r; chunk cc holds tokens m0 + 8cc .. +8
            const int n = n0 + r;
            const int m = m0 + cc * 8;
            if (n >= g.N || m >= g.M) continue;
            const int nv = n - 2 * g.hidden;
            const int head = nv / g.head_dim, dd = nv % g.head_dim;
            stg16(g.vt + ((int64_t)head * g.head_dim + dd) * g.vt_ld + m, val);
        } else {
            const int m = m0 + r;
            const int n = n0 + cc * 8;
            if (m >= g.M || n >= g.N) continue;
            if (g.mode == kPlain) {
                stg16(g.c + (int64_t)m * g.ldc + n, val);
            } else {
                const bool is_q = n < g.hidden;
                const int nn = is_q ? n : n - g.hidden;
                const int head = nn / g.head_dim, dd = nn % g.head_dim;
                half_t *dst = is_q ? g.q : g.k;
                stg16(dst + ((int64_t)head * g.M + m) * g.head_dim + dd, val);
            }
        }
    }
}

__global__ __launch_bounds__(256) void transpose_f16(const half_t *src, int rows, int cols, half_t *dst,
                                                     int64_t ld_dst) {
    __shared__ half_t t[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int r = i / 64, c = i % 64;
        if (r0 + r < rows && c0 + c < cols) t[r][c] = src[(int64_t)(r0 + r) * cols + c0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int c = i / 64, r = i % 64;
        if (r0 + r < rows && c0 + c < cols) dst[(int64_t)(c0 + c) * ld_dst + r0 + r] = t[r][c];
    }
}

}  // namespace

hipError_t launch_gemm_f16(const GemmArgs &g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_f16_nt, dim3(tiles), dim3(NTHREADS), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_transpose_f16(const half_t *src, int rows, int cols, half_t *dst, int64_t ld_dst,
                                hipStream_t stream) {
    dim3 grid((cols + 63) / 64, (rows + 63) / 64);
    hipLaunchKernelGGL(transpose_f16, grid, dim3(256), 0, stream, src, rows, cols, dst, ld_dst);
    return hipGetLastError();
}

}  // namespace attnblk
