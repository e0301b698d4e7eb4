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
// 128x64 each on v_mfma_f32_32x32x16_f16. K advances in steps of 32 through a
// four-stage LDS ring filled by direct global->LDS loads (no staging
// registers), issued three steps ahead; one barrier per step. An XOR swizzle
// applied on the load side makes every ds_read_b128 conflict-free. Tiles are grouped 4 deep
// in M and each XCD gets a contiguous range of tiles so its L2 holds the A
// and B panels its workgroups share. The epilogue stages the fp16 tile in
// LDS (transposed for V) and writes 16-byte chunks.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NTHREADS = 512;
constexpr int STAGES = 4;
constexpr int GROUP_M = 4;
constexpr int A_TILE = BM * BK;  // halves
constexpr int B_TILE = BN * BK;
constexpr int STAGE = A_TILE + B_TILE;
constexpr int CP = BN + 8;       // epilogue pitch (halves)
constexpr int SMEM_MAIN = STAGES * STAGE * 2;  // bytes
constexpr int SMEM_EPI = BM * CP * 2;
constexpr int SMEM_BYTES = SMEM_MAIN > SMEM_EPI ? SMEM_MAIN : SMEM_EPI;


// LDS tile layout: 64-byte rows of four 16-byte chunks; logical chunk c of
// row r sits at physical chunk c ^ swz(r), which spreads the 16 rows one LDS
// pass reads over all 16 bank groups. swz depends only on bits 2-3 of the
// row, which are the same for the four row blocks (32 rows apart) a wave
// reads, so a fragment address is one base register plus an immediate.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }


// Issue the direct global->LDS loads of one K-step (A rows and B rows) into
// stage buffer `st`. A global_load_lds_dwordx4 writes 64 lanes x 16 bytes to
// consecutive LDS addresses, so each lane fetches the global chunk that its
// LDS slot must hold. Waves 0-3 move A (16 instructions), waves 4-7 move B.
// Interior tiles use one loop-invariant lane offset; edge tiles clamp rows
// past M or N to the last valid row.
template <bool EDGE>
__device__ __forceinline__ void issue_stage(const GemmArgs &g, half_t *st, int m0, int n0, int k0, int wave,
                                            int lane) {
    const bool is_a = wave < 4;
    const int w4 = wave & 3;
    const half_t *base = is_a ? g.a : g.b;
    const int64_t ld = is_a ? g.lda : g.ldb;
    const int r0 = is_a ? m0 : n0;
    const int rmax = (is_a ? g.M : g.N) - 1;
    half_t *tile = st + (is_a ? 0 : A_TILE);
    const int lrow = lane >> 2;                  // row within a 16-row instruction block
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);  // logical chunk for this LDS slot
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = 4 * w4 + i;                // instruction index 0..15: rows 16n..16n+15
        int row = r0 + 16 * n + lrow;
        if (EDGE) row = min(row, rmax);
        const half_t *src = base + (int64_t)row * ld + k0 + chunk * 8;
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)(tile + n * 512), 16, 0, 0);
    }
}

__global__ __launch_bounds__(NTHREADS) void gemm_f16_nt(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM_BYTES];
    __shared__ float rs_tile[BM];  // RMSNorm row factors of the tile's rows (pre-norm only)
    half_t *smem = reinterpret_cast<half_t *>(smem_raw);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // published to every wave by the barriers of the main loop
    if (g.row_scale && tid < BM) rs_tile[tid] = g.row_scale[min(m0 + tid, g.M - 1)];
    const bool edge = (m0 + BM > g.M) || (n0 + BN > g.N);

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

    const int nk = g.K / BK;
    // prologue: stages 0..STAGES-2 in flight
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) {
            if (edge)
                issue_stage<true>(g, smem + s * STAGE, m0, n0, s * BK, wave, lane);
            else
                issue_stage<false>(g, smem + s * STAGE, m0, n0, s * BK, wave, lane);
        }

    // fragment bases: row (lane & 31) of each 32-row block, physical chunk for k-substep kk
    const int sw = swz(lane & 31);
    const int a_off0 = (wm * 128 + (lane & 31)) * BK + (((0 + h) ^ sw) << 3);
    const int a_off1 = (wm * 128 + (lane & 31)) * BK + (((2 + h) ^ sw) << 3);
    const int b_off0 = A_TILE + (wn * 64 + (lane & 31)) * BK + (((0 + h) ^ sw) << 3);
    const int b_off1 = A_TILE + (wn * 64 + (lane & 31)) * BK + (((2 + h) ^ sw) << 3);

    // Software pipeline over K substeps of 16: the fragment reads of substep
    // t+1 are issued before the MFMAs of substep t. Barrier B_kt sits between
    // the two substeps of step kt: every wave has then finished reading step
    // kt-1 (its fragments fed MFMAs before B_kt), so its buffer can be refilled
    // with step kt+STAGES-1; and each wave waited for its own loads of step
    // kt+1 before B_kt, so step kt+1 is readable after it.
    auto read_frags = [&](const half_t *stb, int kk, half8 (&af)[4], half8 (&bf)[2]) {
        const half_t *ab = stb + (kk ? a_off1 : a_off0);
        const half_t *bb = stb + (kk ? b_off1 : b_off0);
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const half8 *>(ab + i * 32 * BK);
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const half8 *>(bb + j * 32 * BK);
    };
    auto mma = [&](const half8 (&af)[4], const half8 (&bf)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    };
    // stage 0 readable (stages 1 and 2, 4 loads each, may stay in flight)
    static_assert(STAGES == 4, "the waits below count 4 loads per stage and 3 stages in flight");
    if (nk >= 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_only(8));
    else if (nk == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_only(4));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    barrier_no_fence();
    half8 a0[4], b0[2], a1[4], b1[2];
    read_frags(smem, 0, a0, b0);
    for (int kt = 0; kt < nk; ++kt) {
        const half_t *stb = smem + (kt % STAGES) * STAGE;
        read_frags(stb, 1, a1, b1);
        mma(a0, b0);
        if (kt + 1 < nk) {
            // step kt+1 must be complete; steps up to kt+STAGES-2 may stay in flight
            const int in_flight = min(nk - 1, kt + STAGES - 2) - (kt + 1);
            if (in_flight >= 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(4));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            barrier_no_fence();
            if (kt + STAGES - 1 < nk) {
                const int sidx = (kt + STAGES - 1) % STAGES;
                if (edge)
                    issue_stage<true>(g, smem + sidx * STAGE, m0, n0, (kt + STAGES - 1) * BK, wave, lane);
                else
                    issue_stage<false>(g, smem + sidx * STAGE, m0, n0, (kt + STAGES - 1) * BK, wave, lane);
            }
            read_frags(smem + ((kt + 1) % STAGES) * STAGE, 0, a0, b0);
        }
        mma(a1, b1);
    }
    __syncthreads();  // every wave is done with the stage buffers; reuse LDS for the epilogue

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
                // RMSNorm pre-norm: output row m scales by 1 / rms(x_m)
                float rsc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                if (g.row_scale) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) rsc[r] = rs_tile[row + r];
                }
                if (v_tile) {
                    half4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = (half_t)(acc[i][j][4 * gg + r] * rsc[r]);
                    *reinterpret_cast<half4 *>(smem + col * CP + row) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        smem[(row + r) * CP + col] = (half_t)(acc[i][j][4 * gg + r] * rsc[r] * sc);
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

// dst[c][r] = src[r][c] for a rows x cols submatrix with row stride ld_src.
__global__ __launch_bounds__(256) void transpose_f16(const half_t *src, int rows, int cols, int64_t ld_src,
                                                     half_t *dst, int64_t ld_dst) {
    __shared__ half_t t[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int r = i / 64, c = i % 64;
        if (r0 + r < rows && c0 + c < cols) t[r][c] = src[(int64_t)(r0 + r) * ld_src + c0 + c];
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

hipError_t launch_transpose_f16(const half_t *src, int rows, int cols, int64_t ld_src, half_t *dst, int64_t ld_dst,
                                hipStream_t stream) {
    dim3 grid((cols + 63) / 64, (rows + 63) / 64);
    hipLaunchKernelGGL(transpose_f16, grid, dim3(256), 0, stream, src, rows, cols, ld_src, dst, ld_dst);
    return hipGetLastError();
}

}  // namespace attnblk
