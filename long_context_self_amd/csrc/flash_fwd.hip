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
//   per wave. K and V^T tiles of 64 keys are double-buffered in LDS with
//   padded pitches that keep every ds_read_b128 conflict-free and every
//   fragment address a base register plus an immediate offset. Both waves of
//   a SIMD read LDS concurrently: on gfx950 one wave per SIMD sustains only
//   about half the LDS read bandwidth that two do.
// * Each wave's tile step issues the MFMAs of S_j = K_j Q^T together with
//   those of O += V_{j-1} P_{j-1} (independent, so they interleave), with the
//   LDS fragment reads pipelined four MFMAs ahead, then the softmax of S_j.
//   One barrier per tile; between barriers the two waves of a SIMD drift, so
//   one's softmax overlaps the other's MFMAs.
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
// LDS layouts (padded pitches, so every fragment read is one base register
// plus a compile-time offset):
// * K tile: 64 key rows of 128 halves at a pitch of 136 halves (272 B). Key k
//   is stored in row ksig(k) (bits 3 and 4 of k swapped): the 16 lanes of one
//   LDS pass then read 16 rows that are distinct mod 16, and with a pitch of
//   17 16-byte units their chunks fall in 16 distinct bank groups.
// * V^T tile: 128 rows (head dims) of 64 keys at a pitch of 72 halves (144 B):
//   16 consecutive rows at pitch 9 units are also 16 distinct bank groups.
constexpr int KP = D + 8;                     // K pitch (halves)
constexpr int VP = BN + 8;                    // V^T pitch (halves)
constexpr int K_TILE = BN * KP;               // halves
constexpr int V_TILE = D * VP;                // halves
constexpr float kRescaleTau = 8.0f * kLn2;  // rescale only when a max grows by > 2^8

__device__ __forceinline__ int ksig(int k) { return (k & ~24) | ((k & 8) << 1) | ((k & 16) >> 1); }
// Accumulator row i of a 32x32 S^T block holds key perm_key(i): lane half h
// then owns keys 16h..16h+15 in accumulator order.
__device__ __forceinline__ int perm_key(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// ---- M phase: S_j = K_j Q^T (if HAS_G1) and O^T += V_{j-1}^T P_{j-1}^T (if HAS_G2).
// The products are independent, so their MFMAs interleave. Operand fragments
// come from LDS through a double buffer of four: the reads for MFMAs n+4..n+7
// are in flight while MFMAs n..n+3 execute.
template <bool HAS_G1, bool HAS_G2>
__device__ __forceinline__ void mfma_phase(const half_t *ks, const half_t *vs, const half8 (&qf)[8],
                                           const half8 (&pf)[2][2], floatx16 (&s)[2], floatx16 (&o)[4],
                                           int lane) {
    const int h = lane >> 5;
    const half_t *kbase = ks + ksig(perm_key(lane & 31)) * KP + 8 * h;
    const half_t *vbase = vs + (lane & 31) * VP + 16 * h;
    constexpr int N = (HAS_G1 ? 16 : 0) + (HAS_G2 ? 16 : 0);
    // MFMA n of this phase: kind 0 = S block kb at k-step i; kind 1 = O block
    // mb with key block kb and half t.
    auto decode = [](int n, int &kind, int &i, int &kb, int &mb, int &t) {
        if (HAS_G1 && HAS_G2) {
            const int u = n & 3, step = n >> 2;
            kind = u >> 1;
            if (kind == 0) {
                i = step;
                kb = u & 1;
            } else {
                const int g = 2 * step + (u & 1);
                mb = g >> 2;
                kb = (g >> 1) & 1;
                t = g & 1;
            }
        } else if (HAS_G1) {
            kind = 0;
            i = n >> 1;
            kb = n & 1;
        } else {
            kind = 1;
            mb = n >> 2;
            kb = (n >> 1) & 1;
            t = n & 1;
        }
    };
    auto frag = [&](int n) -> half8 {
        int kind = 0, i = 0, kb = 0, mb = 0, t = 0;
        decode(n, kind, i, kb, mb, t);
        if (kind == 0) return *reinterpret_cast<const half8 *>(kbase + kb * 32 * KP + 16 * i);
        return *reinterpret_cast<const half8 *>(vbase + 32 * mb * VP + 32 * kb + 8 * t);
    };
    auto mma = [&](int n, const half8 &a) {
        int kind = 0, i = 0, kb = 0, mb = 0, t = 0;
        decode(n, kind, i, kb, mb, t);
        if (kind == 0)
            s[kb] = (i == 0) ? mfma32(a, qf[i], floatx16{}) : mfma32(a, qf[i], s[kb]);
        else
            o[mb] = mfma32(a, pf[kb][t], o[mb]);
    };
    half8 buf[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[0][j] = frag(j);
#pragma unroll
    for (int step = 0; step < N / 4; ++step) {
        if (step + 1 < N / 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) buf[(step + 1) & 1][j] = frag(4 * (step + 1) + j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(4 * step + j, buf[step & 1][j]);
    }
}

// ---- S phase: online softmax of S_j -> P_j (fp16), running max/sum, lazy O rescale.
template <bool MASK>
__device__ __forceinline__ void softmax_phase(floatx16 (&s)[2], half8 (&pf)[2][2], floatx16 (&o)[4],
                                              float &m_run, float &l_run, int lane, int key0, int skv) {
    const int h = lane >> 5;
    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int key = key0 + 32 * kb + 16 * h + i;
                if (key >= skv) s[kb][i] = -INFINITY;
            }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
    mt = wave_max_across_halves(mt);
    const bool need = mt > m_run + kRescaleTau;
    if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb] *= alpha;
    }
    const float mneg = -m_run * kLog2e;
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
}

// Per-thread offsets of the 16-byte chunks a thread moves for every tile (two
// of the K tile, 64 rows x 16 chunks; two of the V^T tile, 128 rows x 8
// chunks). Global offsets are relative to the tile's first key, so a tile's
// load is one scalar base plus loop-invariant offsets.
struct TileOffsets {
    int kg[2], kl[2], vg[2], vl[2], krow[2], vkey[2];
};

__device__ __forceinline__ TileOffsets tile_offsets(const FlashArgs &a, int tid) {
    TileOffsets t;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int i = tid + NTHREADS * p;
        const int row = i >> 4, c = i & 15;
        t.krow[p] = row;
        t.kg[p] = row * D + c * 8;
        t.kl[p] = ksig(row) * KP + c * 8;
        const int d = i >> 3, cv = i & 7;
        t.vkey[p] = cv * 8;
        t.vg[p] = d * (int)a.v_row_stride + cv * 8;
        t.vl[p] = d * VP + cv * 8;
    }
    return t;
}

// K tile starting at key0 -> registers. Rows past skv are clamped to the last
// key (finite values; their scores are masked).
__device__ __forceinline__ void load_k(u32x4 (&st)[2], const FlashArgs &a, const half_t *kh, int key0,
                                       const TileOffsets &t) {
    if (key0 + BN <= a.skv) {
        const half_t *kt = kh + (int64_t)key0 * D;
#pragma unroll
        for (int p = 0; p < 2; ++p) st[p] = ldg16(kt + t.kg[p]);
    } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int key = min(key0 + t.krow[p], a.skv - 1);
            st[p] = ldg16(kh + (int64_t)key * D + (t.kg[p] - t.krow[p] * D));
        }
    }
}

// V^T tile starting at key0 -> registers; keys past skv are zero so that the
// masked probabilities multiply zeros.
__device__ __forceinline__ void load_v(u32x4 (&st)[2], const FlashArgs &a, const half_t *vh, int key0,
                                       const TileOffsets &t) {
    const half_t *vt = vh + key0;
    if (key0 + BN <= a.skv) {
#pragma unroll
        for (int p = 0; p < 2; ++p) st[p] = ldg16(vt + t.vg[p]);
    } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int kstart = key0 + t.vkey[p];
            const half_t *src = vt + t.vg[p];
            half8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (kstart + e < a.skv) ? src[e] : (half_t)0.0f;
            st[p] = as_u32x4(v);
        }
    }
}

__device__ __forceinline__ void store_k(const u32x4 (&st)[2], half_t *ks, const TileOffsets &t) {
#pragma unroll
    for (int p = 0; p < 2; ++p) *reinterpret_cast<u32x4 *>(ks + t.kl[p]) = st[p];
}

__device__ __forceinline__ void store_v(const u32x4 (&st)[2], half_t *vs, const TileOffsets &t) {
#pragma unroll
    for (int p = 0; p < 2; ++p) *reinterpret_cast<u32x4 *>(vs + t.vl[p]) = st[p];
}

__device__ __forceinline__ void softmax_tile(floatx16 (&s)[2], half8 (&pf)[2][2], floatx16 (&o)[4],
                                             float &m_run, float &l_run, int lane, int j, int skv) {
    if ((j + 1) * BN <= skv)
        softmax_phase<false>(s, pf, o, m_run, l_run, lane, j * BN, skv);
    else
        softmax_phase<true>(s, pf, o, m_run, l_run, lane, j * BN, skv);
}

// Tile j holds K_j in ksm[j % 2] and V_j in vsm[j % 2]. Step j computes
// S_j = K_j Q^T and O += V_{j-1} P_{j-1}, then the softmax of S_j; meanwhile
// K_{j+1} and V_j are loaded into registers and stored at the end of the step
// into ksm[(j+1) % 2] and vsm[j % 2]. Both buffers were last read in step j-1,
// which every wave finished before the barrier that ended it; the barrier at
// the end of step j publishes them. A final step adds V_{T-1} P_{T-1}.
__global__ __launch_bounds__(NTHREADS) void flash_fwd_f16_d128(FlashArgs a) {
    __shared__ __attribute__((aligned(16))) half_t ksm[2 * K_TILE];
    __shared__ __attribute__((aligned(16))) half_t vsm[2 * V_TILE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int h = lane >> 5;

    const int nqb = (a.sq + BQ - 1) / BQ;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int head = work / nqb;
    const int qb = work % nqb;

    const half_t *qh = a.q + (int64_t)head * a.q_head_stride;
    const half_t *kh = a.k + (int64_t)head * a.k_head_stride;
    const half_t *vh = a.vt + (int64_t)head * a.v_head_stride;

    const int q = qb * BQ + wave * 32 + (lane & 31);
    const int qc = min(q, a.sq - 1);
    half8 qf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = as_half8(ldg16(qh + (int64_t)qc * D + kk * 16 + 8 * h));

    floatx16 o[4], s[2];
    half8 pf[2][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) o[mb] = floatx16{};
    float m_run = -INFINITY, l_run = 0.0f;

    const int T = (a.skv + BN - 1) / BN;
    if (T > 0) {
        const TileOffsets toff = tile_offsets(a, tid);
        u32x4 sk[2], sv[2];
        load_k(sk, a, kh, 0, toff);
        store_k(sk, ksm, toff);
        __syncthreads();
        // step 0: S_0 only
        if (T > 1) load_k(sk, a, kh, BN, toff);
        load_v(sv, a, vh, 0, toff);
        mfma_phase<true, false>(ksm, vsm, qf, pf, s, o, lane);
        softmax_tile(s, pf, o, m_run, l_run, lane, 0, a.skv);
        if (T > 1) store_k(sk, ksm + K_TILE, toff);
        store_v(sv, vsm, toff);
        __syncthreads();
        // Steady state: K_{j+1} and V_j are full tiles and S_j needs no mask,
        // so the loads are branch-free and stay in flight across the MFMAs.
        int j = 1;
        for (; j + 2 < T; ++j) {
            const half_t *kt = kh + (int64_t)(j + 1) * BN * D;
            const half_t *vt = vh + j * BN;
#pragma unroll
            for (int p = 0; p < 2; ++p) sk[p] = ldg16(kt + toff.kg[p]);
#pragma unroll
            for (int p = 0; p < 2; ++p) sv[p] = ldg16(vt + toff.vg[p]);
            mfma_phase<true, true>(ksm + (j & 1) * K_TILE, vsm + ((j - 1) & 1) * V_TILE, qf, pf, s, o, lane);
            softmax_phase<false>(s, pf, o, m_run, l_run, lane, j * BN, a.skv);
            store_k(sk, ksm + ((j + 1) & 1) * K_TILE, toff);
            store_v(sv, vsm + (j & 1) * V_TILE, toff);
            __syncthreads();
        }
        // The last (at most two) steps, whose loads may touch the partial tile.
        for (; j < T; ++j) {
            if (j + 1 < T) load_k(sk, a, kh, (j + 1) * BN, toff);
            load_v(sv, a, vh, j * BN, toff);
            mfma_phase<true, true>(ksm + (j & 1) * K_TILE, vsm + ((j - 1) & 1) * V_TILE, qf, pf, s, o, lane);
            softmax_tile(s, pf, o, m_run, l_run, lane, j, a.skv);
            if (j + 1 < T) store_k(sk, ksm + ((j + 1) & 1) * K_TILE, toff);
            store_v(sv, vsm + (j & 1) * V_TILE, toff);
            __syncthreads();
        }
        mfma_phase<false, true>(ksm, vsm + ((T - 1) & 1) * V_TILE, qf, pf, s, o, lane);
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
                for (int rr = 0; rr < 4; ++rr) v[rr] = o[mb][4 * g + rr] * inv;
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
                for (int rr = 0; rr < 4; ++rr) v[rr] = (half_t)(o[mb][4 * g + rr] * inv);
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
