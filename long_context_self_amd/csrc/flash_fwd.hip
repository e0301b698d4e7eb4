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
//   per wave; K and V^T tiles of 64 keys.
// * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_f16, Q held in
//   registers as the B operand of S. K rows are taken in a permuted order so
//   that each lane's S accumulator holds 16 consecutive keys of its own query;
//   after exp and a cast those are the B operand of the PV product, with no
//   data movement between lanes.
// * Software pipeline per wave: step t issues the MFMAs of S_{t+1} and of
//   O += V_t P_t, and while they run computes exp(S_t) -> P_t (before the PV
//   MFMAs that need it) and then the row sums of P_t and the row maxima of
//   S_{t+1}. The VALU softmax work thus hides under the wave's own matrix work
//   instead of alternating with it.
// * K/V^T reach LDS by direct global->LDS loads (no staging registers) into a
//   4-slot ring, issued three steps ahead. LDS holds every tile in MFMA
//   operand order: fragment n of a tile is 64 lanes x 16 bytes, so every
//   operand read is one lane-linear ds_read_b128 (conflict-free, base register
//   plus immediate), and each load instruction gathers exactly one fragment.
//   One barrier per step; the next step's first operands are read before it.
// * Softmax in the exp2 domain with the running max and sum in registers; the
//   O rescale is skipped unless some row's max grew by more than 2^8 (exact:
//   O and the sum always share the same reference max).
// * O is normalised and staged through LDS so every row leaves in full
//   16-byte chunks of whole lines.
// * Blocks are remapped so each XCD works through a contiguous range of
//   (head, query block) items and its concurrent workgroups share K/V in L2.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int D = 128;       // head_dim
constexpr int BQ = 256;      // query rows per workgroup
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int BN = 64;       // keys per tile
constexpr int FRAG = 64 * 8;              // halves in one MFMA operand fragment
constexpr int NFRAG = 16;                 // fragments per K tile and per V^T tile
constexpr int SLOT = 2 * NFRAG * FRAG;    // halves per ring slot: K part, then V^T part
constexpr int RING_BYTES = 4 * SLOT * 2;  // stage s lives in slot s % 4
constexpr int RA = 2;                     // operand reads in flight ahead of the MFMAs
constexpr int OP16 = D + 8;               // O staging pitch, fp16 (halves)
constexpr int OP32 = D + 4;               // O staging pitch, fp32 (floats)
constexpr int OSTAGE_BYTES = NWAVES * 32 * OP32 * 4;
constexpr int SMEM_BYTES = RING_BYTES > OSTAGE_BYTES ? RING_BYTES : OSTAGE_BYTES;
constexpr float kRescaleTau = 8.0f * kLn2;  // rescale only when a max grows by > 2^8

// Accumulator row i of a 32x32 S^T block holds key perm_key(i) of its 32-key
// block: lane half h then owns keys 16h..16h+15 in accumulator order.
__device__ __forceinline__ int perm_key(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// Stage s = {K_{s+1}, V_s}: everything step s reads. Fragment order:
// * K fragment n (MFMA n of a step): k-step kk = n / 2 (head dims 16kk..),
//   key block kb = n % 2. Lane l holds K[32kb + perm_key(l % 32)][16kk + 8(l / 32) + 0..7].
// * V^T fragment n (MFMA 16 + n): head-dim block mb = n % 4, key step ks = n / 4
//   (key block ks / 2, half ks % 2). Lane l holds
//   V^T[32mb + l % 32][32(ks / 2) + 16(l / 32) + 8(ks % 2) + 0..7], matching the
//   key order of the lane's P values.
// Wave w moves K and V^T fragments 2w and 2w + 1 of every stage.
struct LoadOffsets {
    uint32_t k[2], v[2];  // bytes from the tile's first key
};

__device__ __forceinline__ LoadOffsets load_offsets(const FlashArgs &a, int wave, int lane) {
    const int r = lane & 31, h = lane >> 5;
    LoadOffsets o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int n = 2 * wave + e;
        const int kk = n >> 1, kb = n & 1;
        o.k[e] = (uint32_t)(((kb * 32 + perm_key(r)) * D + kk * 16 + 8 * h) * 2);
        const int mb = n & 3, ks = n >> 2;
        o.v[e] = (uint32_t)(((int64_t)(32 * mb + r) * a.v_row_stride + 32 * (ks >> 1) + 16 * h + 8 * (ks & 1)) * 2);
    }
    return o;
}

struct Ctx {
    const char *kh, *vh;  // this head's K and V^T (bytes)
    char *ring;           // LDS ring (wave-uniform)
    const half_t *rl;     // LDS ring + 8 * lane (this lane's operand slot)
    LoadOffsets lo;
    int wave, lane, skv, T;
    int64_t vrs;
};

__device__ __forceinline__ char *slot_k(const Ctx &c, int s) { return c.ring + (s & 3) * SLOT * 2; }
__device__ __forceinline__ char *slot_v(const Ctx &c, int s) { return c.ring + (s & 3) * SLOT * 2 + NFRAG * FRAG * 2; }

// Buffer descriptor for raw byte addressing from `base` (stride 0, no
// range clamp): the tile base lives in scalar registers and each lane adds
// its loop-invariant 32-bit offset, so a direct load costs no vector ALU work.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, -1, 0x00020000);
}

// Full K tile `tile` -> K part of slot s (two direct loads per wave).
__device__ __forceinline__ void issue_k_full(const Ctx &c, int tile, int s) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(c.kh + (int64_t)tile * BN * D * 2);
    char *dst = slot_k(c, s) + 2 * c.wave * FRAG * 2;
#pragma unroll
    for (int e = 0; e < 2; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + e * FRAG * 2), 16, c.lo.k[e], 0, 0, 0);
}

// Full V^T tile -> V part of slot s.
__device__ __forceinline__ void issue_v_full(const Ctx &c, int tile, int s) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(c.vh + (int64_t)tile * BN * 2);
    char *dst = slot_v(c, s) + 2 * c.wave * FRAG * 2;
#pragma unroll
    for (int e = 0; e < 2; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + e * FRAG * 2), 16, c.lo.v[e], 0, 0, 0);
}

// Last, partial K tile: rows past skv are clamped to the last key (finite
// values; their scores are masked).
__device__ __forceinline__ void issue_k_partial(const Ctx &c, int tile, int s) {
    const int r = c.lane & 31, h = c.lane >> 5;
    char *dst = slot_k(c, s) + 2 * c.wave * FRAG * 2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int n = 2 * c.wave + e;
        const int kk = n >> 1, kb = n & 1;
        const int key = min(tile * BN + kb * 32 + perm_key(r), c.skv - 1);
        const char *src = c.kh + ((int64_t)key * D + kk * 16 + 8 * h) * 2;
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)(dst + e * FRAG * 2), 16, 0, 0);
    }
}

// Last, partial V^T tile through registers: keys past skv are stored as
// zeros, so the zero probabilities of masked keys never meet non-finite data.
__device__ __forceinline__ void stage_v_partial(const Ctx &c, int tile, int s) {
    const int r = c.lane & 31, h = c.lane >> 5;
    half_t *dst = reinterpret_cast<half_t *>(slot_v(c, s)) + 2 * c.wave * FRAG + 8 * c.lane;
    const half_t *vh = reinterpret_cast<const half_t *>(c.vh);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int n = 2 * c.wave + e;
        const int mb = n & 3, ks = n >> 2;
        const int key = tile * BN + 32 * (ks >> 1) + 16 * h + 8 * (ks & 1);
        const half_t *src = vh + (int64_t)(32 * mb + r) * c.vrs + key;
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (key + j < c.skv) ? src[j] : (half_t)0.0f;
        *reinterpret_cast<half8 *>(dst + e * FRAG) = v;
    }
}

// Issue stage s (any position in the key loop); returns the number of direct
// loads it left in flight (register-path loads complete before returning).
__device__ __forceinline__ int issue_stage(const Ctx &c, int s) {
    int n = 0;
    const int kt = s + 1;
    if (kt < c.T) {
        if ((kt + 1) * BN <= c.skv)
            issue_k_full(c, kt, s);
        else
            issue_k_partial(c, kt, s);
        n += 2;
    }
    if (s >= 0 && s < c.T) {
        if ((s + 1) * BN <= c.skv) {
            issue_v_full(c, s, s);
            n += 2;
        } else {
            stage_v_partial(c, s, s);
        }
    }
    return n;
}

// Wait until at most n direct loads are in flight and every LDS access of
// this wave is complete.
__device__ __forceinline__ void wait_vm_lgkm(int n) {
    if (n >= 4)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(4));
    else if (n >= 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(2));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
}

__device__ __forceinline__ half8 rd(const half_t *p) { return *reinterpret_cast<const half8 *>(p); }

// P = exp(S - m) (exp2 domain) as the fp16 B operands of the PV product:
// pf[ks] holds keys 32(ks / 2) + 16h + 8(ks % 2) + 0..7 of the lane's query.
// PRE: the scores are already (S - m) log2(e) -- Q carries the log2(e)
// factor and the first S MFMA starts from -m (see the kernel) -- so P is one
// exp2 per score; otherwise one FMA per score maps S to that argument.
template <bool PRE>
__device__ __forceinline__ void exp_and_pack(const floatx16 (&sc)[2], half8 (&pf)[4], float mneg) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            pf[2 * kb + (i >> 3)][i & 7] =
                (half_t)__builtin_amdgcn_exp2f(PRE ? sc[kb][i] : fmaf(sc[kb][i], kLog2e, mneg));
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Row sum of the fp16 probabilities (the very values the PV product
// weights), two per dot instruction with fp32 accumulation.
__device__ __forceinline__ float row_sum(const half8 (&pf)[4]) {
    const half2v one = {(half_t)1.0f, (half_t)1.0f};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            a0 = __builtin_amdgcn_fdot2(half2v{pf[ks][2 * j], pf[ks][2 * j + 1]}, one, a0, false);
            a1 = __builtin_amdgcn_fdot2(half2v{pf[ks][2 * j + 2], pf[ks][2 * j + 3]}, one, a1, false);
        }
    return a0 + a1;
}

template <bool MASK>
__device__ __forceinline__ float row_max(floatx16 (&s)[2], int key0, int skv, int h) {
    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key0 + 32 * kb + 16 * h + i >= skv) s[kb][i] = -INFINITY;
    }
    // two chains of three-operand maxima over the 32 scores
    float m0 = fmaxf(s[0][0], s[0][1]), m1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
        m0 = fmaxf(fmaxf(m0, s[0][i]), s[0][i + 1]);
        m1 = fmaxf(fmaxf(m1, s[1][i]), s[1][i + 1]);
    }
    return wave_max_across_halves(fmaxf(m0, m1));
}

// New row max mt of the next scores: raise the reference max where it grew by
// more than 2^8 and rescale O and the running sum to it (skipped when no row
// of the wave needs it).
__device__ __forceinline__ void update_max(float mt, float &m_run, float &l_run, floatx16 (&o)[4]) {
    const bool need = mt > m_run + kRescaleTau;
    if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb] *= alpha;
    }
}

// The same for PRE scores, which are relative to the reference already
// (log2 units): mt is the row max of S - m. Where it exceeds 8 the reference
// moves up by mt, and O, the sum, the pending scores and the accumulator
// start value -m of later tiles follow it.
__device__ __forceinline__ void update_max_rel(float mt, float &m_run, float &l_run, floatx16 (&o)[4],
                                               floatx16 (&s)[2], floatx16 &negm) {
    const bool need = mt > 8.0f;
    if (__ballot(need)) {
        const float delta = need ? mt : 0.0f;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        m_run += delta;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] -= delta;
        negm = -m_run;
    }
}

// Steady step t: every tile it touches is full, stage t+3 exists and is
// full, and step t+1 starts with S_{t+2} MFMAs. fr holds this step's first
// RA operands on entry and the next step's on exit.
template <bool PRE>
__device__ __forceinline__ void steady_step(const Ctx &c, int t, floatx16 (&sc)[2], floatx16 (&sn)[2],
                                            floatx16 (&o)[4], const half8 (&qf)[8], half8 (&fr)[RA],
                                            float &m_run, float &l_run, floatx16 &negm) {
    const half_t *cur = c.rl + (t & 3) * SLOT;
    const half_t *nxt = c.rl + ((t + 1) & 3) * SLOT;
    half8 pf[4];
    exp_and_pack<PRE>(sc, pf, -m_run * kLog2e);
#pragma unroll
    for (int n = 0; n < 32; ++n) {
        const half8 a = fr[n % RA];
        const int m = n + RA;
        fr[n % RA] = rd(m < 32 ? cur + m * FRAG : nxt + (m - 32) * FRAG);
        // stage t+3's direct loads go out a quarter of the way into each half
        // of the step rather than in one burst at its start
        if (n == 8) issue_k_full(c, t + 4, t + 3);
        if (n == 24) issue_v_full(c, t + 3, t + 3);
        if (n < 16) {
            const int kk = n >> 1, kb = n & 1;
            sn[kb] = mfma32(a, qf[kk], kk == 0 ? (PRE ? negm : floatx16{}) : sn[kb]);
        } else {
            const int mb = (n - 16) & 3, ks = (n - 16) >> 2;
            o[mb] = mfma32(a, pf[ks], o[mb]);
        }
    }
    l_run += row_sum(pf);
    if (PRE)
        update_max_rel(row_max<false>(sn, 0, 0, c.lane >> 5), m_run, l_run, o, sn, negm);
    else
        update_max(row_max<false>(sn, 0, 0, c.lane >> 5), m_run, l_run, o);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(4));  // stage t+2 has landed
    barrier_no_fence();
}

// Any step t (the last few of the loop): the same work with every condition
// checked, and without reading ahead into the next step.
template <bool PRE>
__device__ __forceinline__ void general_step(const Ctx &c, int t, floatx16 (&sc)[2], floatx16 (&sn)[2],
                                             floatx16 (&o)[4], const half8 (&qf)[8], float &m_run,
                                             float &l_run, floatx16 &negm) {
    const int inflight = issue_stage(c, t + 3);
    const half_t *cur = c.rl + (t & 3) * SLOT;
    half8 pf[4];
    exp_and_pack<PRE>(sc, pf, -m_run * kLog2e);
    const bool has_s = t + 1 < c.T;
    if (has_s) {
        half8 fa[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) fa[n] = rd(cur + n * FRAG);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int kk = n >> 1, kb = n & 1;
            sn[kb] = mfma32(fa[n], qf[kk], kk == 0 ? (PRE ? negm : floatx16{}) : sn[kb]);
        }
    }
    {
        half8 fb[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) fb[n] = rd(cur + (NFRAG + n) * FRAG);
#pragma unroll
        for (int n = 0; n < 16; ++n) o[n & 3] = mfma32(fb[n], pf[n >> 2], o[n & 3]);
    }
    l_run += row_sum(pf);
    if (has_s) {
        const int key0 = (t + 1) * BN;
        const float mt = (key0 + BN <= c.skv) ? row_max<false>(sn, key0, c.skv, c.lane >> 5)
                                               : row_max<true>(sn, key0, c.skv, c.lane >> 5);
        if (PRE)
            update_max_rel(mt, m_run, l_run, o, sn, negm);
        else
            update_max(mt, m_run, l_run, o);
        wait_vm_lgkm(inflight);  // stage t+2 complete (and its register-path stores)
        barrier_no_fence();
    }
}

__device__ __forceinline__ void swap_s(floatx16 (&a)[2], floatx16 (&b)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const floatx16 t = a[kb];
        a[kb] = b[kb];
        b[kb] = t;
    }
}

// Stage s holds K_{s+1} and V_s; the prologue loads K_0 as stage -1 (slot 3)
// and stages 0..2, computes S_0 and its row max. Step t (0 <= t < T) adds
// V_t P_t into O and computes S_{t+1}; it issues stage t+3 into the slot that
// stage t-1 used (all of whose reads finished before the barrier that ended
// step t-1) and ends by waiting for stage t+2 and a barrier, so step t+1 may
// read stage t+1's operands ahead of that barrier.
//
// PRE (set when q holds q_scaled * log2(e), as the block's projection writes
// it): the scores come out of the S MFMAs already as (S - m) log2(e) -- the
// log2(e) factor rides in Q and the first MFMA of each S chain starts from
// the accumulator value -m (negm) instead of 0 -- so the softmax needs no
// per-score FMA; m_run is then kept in log2 units.
template <bool PRE>
__device__ __forceinline__ void attend_item(const FlashArgs &a, int work, char *smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int h = lane >> 5;

    const int nqb = (a.sq + BQ - 1) / BQ;
    const int per_split = nqb * a.num_heads;
    const int split = a.n_split > 1 ? work / per_split : 0;
    const int head = (work - split * per_split) / nqb;
    const int qb = (work - split * per_split) % nqb;
    const int key_base = split * a.split_len;
    const int skv = a.n_split > 1 ? min(a.split_len, a.skv - key_base) : a.skv;
    float *o32 = a.o32 ? a.o32 + (int64_t)split * a.num_heads * a.sq * D : nullptr;
    float *lse_out = a.lse ? a.lse + (int64_t)split * a.num_heads * a.sq : nullptr;

    const half_t *qh = a.q + (int64_t)head * a.q_head_stride;
    const int q = qb * BQ + wave * 32 + (lane & 31);
    const int qc = min(q, a.sq - 1);
    half8 qf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = as_half8(ldg16(qh + (int64_t)qc * D + kk * 16 + 8 * h));

    floatx16 o[4], sa[2], sb[2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) o[mb] = floatx16{};
    float m_run = -INFINITY, l_run = 0.0f;
    floatx16 negm = floatx16{};  // PRE: accumulator start value -m of the S MFMAs

    Ctx c;
    c.kh = reinterpret_cast<const char *>(a.k + (int64_t)head * a.k_head_stride + (int64_t)key_base * D);
    c.vh = reinterpret_cast<const char *>(a.vt + (int64_t)head * a.v_head_stride + key_base);
    c.ring = smem;
    c.rl = reinterpret_cast<const half_t *>(smem) + 8 * lane;
    c.lo = load_offsets(a, wave, lane);
    c.wave = wave;
    c.lane = lane;
    c.skv = skv;
    c.T = (skv + BN - 1) / BN;
    c.vrs = a.v_row_stride;
    const int T = c.T;

    if (T > 0) {
        issue_stage(c, -1);
        issue_stage(c, 0);
        issue_stage(c, 1);
        wait_vm_lgkm(issue_stage(c, 2));  // stages -1, 0, 1 complete
        barrier_no_fence();
        {
            const half_t *k0 = c.rl + 3 * SLOT;
            half8 fa[16];
#pragma unroll
            for (int n = 0; n < 16; ++n) fa[n] = rd(k0 + n * FRAG);
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const int kk = n >> 1, kb = n & 1;
                sa[kb] = mfma32(fa[n], qf[kk], kk == 0 ? floatx16{} : sa[kb]);
            }
        }
        const float mt = (BN <= skv) ? row_max<false>(sa, 0, skv, h) : row_max<true>(sa, 0, skv, h);
        if (PRE) {
            // the first tile sets the reference: S_0 came out relative to 0
            m_run = mt;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sa[kb] -= mt;
            negm = -mt;
        } else {
            update_max(mt, m_run, l_run, o);
        }
        // Step 0 refills slot 3: every wave must be done reading K_0.
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(63));
        barrier_no_fence();

        // Steady steps need stage t+3 full (t + 4 <= last full tile) and run
        // in pairs, so the two S register sets swap roles without copies.
        const int last_full = (skv % BN == 0) ? T - 1 : T - 2;
        const int n_steady = max(0, last_full - 3);
        int t = 0;
        if (n_steady >= 2) {
            half8 fr[RA];
#pragma unroll
            for (int n = 0; n < RA; ++n) fr[n] = rd(c.rl + n * FRAG);
            for (; t + 1 < n_steady; t += 2) {
                steady_step<PRE>(c, t, sa, sb, o, qf, fr, m_run, l_run, negm);
                steady_step<PRE>(c, t + 1, sb, sa, o, qf, fr, m_run, l_run, negm);
            }
        }
        for (; t < T; ++t) {
            general_step<PRE>(c, t, sa, sb, o, qf, m_run, l_run, negm);
            swap_s(sa, sb);
        }
    }

    // ---- epilogue: combine the two lane halves' sums, normalise, stage the
    // wave's 32 x 128 block through LDS and store whole rows.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = skv == 0;
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
    barrier_no_fence();  // every wave is done with the ring
    const int q0 = qb * BQ + wave * 32;
    const int rows = min(32, a.sq - q0);
    const int qr = lane & 31;
    if (o32) {
        float *st = reinterpret_cast<float *>(smem) + wave * 32 * OP32;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                floatx4 v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = o[mb][4 * g + rr] * inv;
                *reinterpret_cast<floatx4 *>(st + qr * OP32 + 32 * mb + 8 * g + 4 * h) = v;
            }
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
        __builtin_amdgcn_wave_barrier();
        float *dst = o32 + ((int64_t)head * a.sq + q0) * D;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 2 * i + (lane >> 5), chunk = lane & 31;
            if (row < rows)
                *reinterpret_cast<floatx4 *>(dst + (int64_t)row * D + 4 * chunk) =
                    *reinterpret_cast<const floatx4 *>(st + row * OP32 + 4 * chunk);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
        __builtin_amdgcn_wave_barrier();
    }
    if (a.o16) {
        half_t *st = reinterpret_cast<half_t *>(smem) + wave * 32 * OP16;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                half4 v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = (half_t)(o[mb][4 * g + rr] * inv);
                *reinterpret_cast<half4 *>(st + qr * OP16 + 32 * mb + 8 * g + 4 * h) = v;
            }
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
        __builtin_amdgcn_wave_barrier();
        half_t *dst = a.o16 + (int64_t)q0 * a.o16_ld + (int64_t)head * D;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4), chunk = lane & 15;
            if (row < rows)
                *reinterpret_cast<u32x4 *>(dst + (int64_t)row * a.o16_ld + 8 * chunk) =
                    *reinterpret_cast<const u32x4 *>(st + row * OP16 + 8 * chunk);
        }
    }
    if (lse_out && h == 0 && q < a.sq) {
        // natural-log LSE; __builtin_amdgcn_logf is log2
        const float lse = PRE ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2
                              : m_run + __builtin_amdgcn_logf(l_tot) * kLn2;
        lse_out[(int64_t)head * a.sq + q] = empty ? -INFINITY : lse;
    }
}

// One workgroup per (key split, head, 256-row query block) item, remapped so
// each XCD works through a contiguous range of items and its concurrent
// workgroups share one head's K/V in L2.
template <bool PRE>
__global__ __launch_bounds__(NTHREADS) void flash_fwd_f16_d128(FlashArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
    attend_item<PRE>(a, xcd_remap(blockIdx.x, gridDim.x), smem);
}

}  // namespace

hipError_t launch_flash_fwd_f16(const FlashArgs &a, hipStream_t stream) {
    if (a.sq <= 0) return hipSuccess;
    const int nqb = (a.sq + BQ - 1) / BQ;
    const int blocks = nqb * a.num_heads * (a.n_split > 1 ? a.n_split : 1);
    if (a.q_log2e)
        hipLaunchKernelGGL(flash_fwd_f16_d128<true>, dim3(blocks), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL(flash_fwd_f16_d128<false>, dim3(blocks), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attnblk
