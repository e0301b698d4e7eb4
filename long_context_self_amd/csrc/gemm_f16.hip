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
// 128x64 each on v_mfma_f32_16x16x32_f16, whose 4-register accumulators move
// fewer register-file bytes per flop than the 32x32 form and so leave the
// chip more clock under its power limit. K advances in steps of 64 through two
// LDS buffers: each thread loads its share of step k+2 into registers while
// step k is computed and stores step k+1 (loaded one step earlier) into the
// other buffer; one barrier per step. Scheduling groups pin the steady step's
// order, spreading the LDS stores, the next substep's fragment reads and the
// global loads among the MFMAs. An XOR swizzle makes every LDS
// read and write conflict-free. Tiles are grouped 4 deep in M and each XCD
// gets a contiguous range of tiles so its L2 holds the A and B panels its
// workgroups share. The epilogue stages the fp16 tile in LDS (transposed for
// V) and writes 16-byte chunks.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHREADS = 512;   // 8 waves (two per SIMD), 2 x 4 of 128 x 64
constexpr int GROUP_M = 4;
constexpr int A_TILE = BM * BK;  // halves
constexpr int B_TILE = BN * BK;
constexpr int BUF = A_TILE + B_TILE;
constexpr int NBUF = 2;
constexpr int CP = BN + 8;       // epilogue pitch (halves)
constexpr int SMEM_MAIN = NBUF * BUF * 2;  // bytes
constexpr int SMEM_EPI = BM * CP * 2;
constexpr int SMEM_BYTES = SMEM_MAIN > SMEM_EPI ? SMEM_MAIN : SMEM_EPI;
constexpr int LPT = (BM * BK / 8) / NTHREADS;  // 16-byte chunks per thread per operand tile (4)
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// LDS tile layout: 128-byte rows of eight 16-byte chunks; logical chunk c of
// row r sits at physical chunk c ^ swz(r). Sixteen consecutive rows then
// cover every (row parity, chunk) pair once, so a ds_read_b128 of one chunk
// column over 16 rows, and a ds_write_b128 of 2 rows x 8 chunks, hit distinct
// banks. swz uses bits 1-3 of the row only, which are the same for rows 32
// apart, so every fragment address is a per-lane base plus an immediate.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Global -> registers: thread t holds chunk t % 8 of rows t / 8 + 64 j,
// j = 0..3, of the A tile and of the B tile for k-step k0. Rows past M or N
// are clamped to the last row (their results are never stored).
__device__ __forceinline__ void load_tile(const GemmArgs &g, int m0, int n0, int k0, int tid, u32x4 (&ra)[LPT],
                                          u32x4 (&rb)[LPT]) {
    const int r = tid >> 3, c = tid & 7;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int ma = min(m0 + r + 64 * j, g.M - 1), nb = min(n0 + r + 64 * j, g.N - 1);
        ra[j] = ldg16(g.a + (int64_t)ma * g.lda + k0 + 8 * c);
        rb[j] = ldg16(g.b + (int64_t)nb * g.ldb + k0 + 8 * c);
    }
}

// Registers -> LDS buffer (swizzled). wo is this thread's offset in halves.
__device__ __forceinline__ void store_tile(half_t *buf, int wo, const u32x4 (&ra)[LPT], const u32x4 (&rb)[LPT]) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        *reinterpret_cast<u32x4 *>(buf + wo + j * 64 * BK) = ra[j];
        *reinterpret_cast<u32x4 *>(buf + A_TILE + wo + j * 64 * BK) = rb[j];
    }
}

__global__ __launch_bounds__(NTHREADS) void gemm_f16_nt(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM_BYTES];
    __shared__ float rs_tile[BM];  // RMSNorm row factors of the tile's rows (pre-norm only)
    half_t *smem = reinterpret_cast<half_t *>(smem_raw);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    floatx4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{};

    const int nk = g.K / BK;
    const int wo = (tid >> 3) * BK + (((tid & 7) ^ swz(tid >> 3)) << 3);
    u32x4 ra[LPT], rb[LPT];
    // prologue: k-step 0 into buffer 0, k-step 1 into registers
    load_tile(g, m0, n0, 0, tid, ra, rb);
    store_tile(smem, wo, ra, rb);
    if (nk > 1) load_tile(g, m0, n0, BK, tid, ra, rb);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(63));  // this wave's LDS stores are done
    barrier_no_fence();

    // fragment bases (16x16x32 layout): row (lane & 15) of each 16-row block;
    // physical chunk of k-substep kk (logical chunk 4 kk + lane / 16)
    const int sw = swz(lane & 15);
    const int q4 = lane >> 4;
    int a_off[2], b_off[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        a_off[kk] = (wm * 128 + (lane & 15)) * BK + (((4 * kk + q4) ^ sw) << 3);
        b_off[kk] = A_TILE + (wn * 64 + (lane & 15)) * BK + (((4 * kk + q4) ^ sw) << 3);
    }
    auto read_frags = [&](const half_t *buf, int kk, half8 (&af)[8], half8 (&bf)[4]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) af[i] = *reinterpret_cast<const half8 *>(buf + a_off[kk] + i * 16 * BK);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const half8 *>(buf + b_off[kk] + j * 16 * BK);
    };
    auto mma = [&](const half8 (&af)[8], const half8 (&bf)[4]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    };

    // Step kt computes from buffer kt % 2. After its first k-substep it stores
    // k-step kt+1 (in registers) into the other buffer -- last read in step
    // kt-1, before the barrier that ended it -- and loads k-step kt+2 into the
    // registers. The barrier at the end of step kt publishes k-step kt+1.
    half8 a0[8], b0[4], a1[8], b1[4];
    auto step = [&](int kt, bool store, bool load) {
        const half_t *buf = smem + (kt & 1) * BUF;
        half_t *nbuf = smem + ((kt + 1) & 1) * BUF;
        read_frags(buf, 0, a0, b0);
        mma(a0, b0);
        if (store) store_tile(nbuf, wo, ra, rb);
        if (load) load_tile(g, m0, n0, (kt + 2) * BK, tid, ra, rb);
        read_frags(buf, 1, a1, b1);
        mma(a1, b1);
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) {  // steady steps: store and load
        step(kt, true, true);
        // Issue order: the 12 fragment reads of k-substep 0; its MFMAs in
        // pairs, each pair followed by one of the 8 LDS stores of step kt+1;
        // one MFMA per fragment read of k-substep 1; then MFMAs in pairs, each
        // pair followed by one of the 8 global loads of step kt+2; the rest.
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 12, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 20, 0);
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(63));  // LDS stores and reads of this wave done
        barrier_no_fence();
    }
    for (; kt < nk; ++kt) {  // the last two steps
        step(kt, kt + 1 < nk, false);
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(63));
        barrier_no_fence();
    }

    // ---- epilogue: stage the fp16 tile in LDS, then 16-byte stores. Pass 1
    // (a Q tile with a q_scaled tap only) stages the Q columns again with the
    // tap's scale and stores them to the tap.
    const bool v_tile = g.mode == kQkv && n0 >= 2 * g.hidden;
    const int passes = (g.mode == kQkv && g.q_tap && n0 < g.hidden) ? 2 : 1;
    for (int pass = 0; pass < passes; ++pass) {
    if (pass == 1) __syncthreads();  // every wave is done reading pass 0's tile
    // A tile may straddle the Q|K border at column h (odd head counts), so the
    // pre-scale is chosen per column; the V border 2h is a multiple of 256.
    const float qsc = pass == 0 ? g.q_scale : g.q_tap_scale;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = wn * 64 + j * 16 + (lane & 15);
            const float sc = (g.mode == kQkv && n0 + col < g.hidden) ? qsc : 1.0f;
            const int row = wm * 128 + i * 16 + 4 * q4;
            // RMSNorm pre-norm: output row m scales by 1 / rms(x_m)
            float rsc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if (g.row_scale) {
#pragma unroll
                for (int r = 0; r < 4; ++r) rsc[r] = rs_tile[row + r];
            }
            if (v_tile) {
                half4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (half_t)(acc[i][j][r] * rsc[r]);
                *reinterpret_cast<half4 *>(smem + col * CP + row) = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) smem[(row + r) * CP + col] = (half_t)(acc[i][j][r] * rsc[r] * sc);
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
                if (pass == 1 && !is_q) continue;
                const int nn = is_q ? n : n - g.hidden;
                const int head = nn / g.head_dim, dd = nn % g.head_dim;
                half_t *dst = is_q ? (pass == 0 ? g.q : g.q_tap) : g.k;
                stg16(dst + ((int64_t)head * g.M + m) * g.head_dim + dd, val);
            }
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
    if (g.K <= 0 || g.K % BK != 0) return hipErrorInvalidValue;  // K = h or H d, a multiple of 64
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
