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
// * One workgroup = 384 query rows of one head, 8 waves (2 per SIMD), 48 rows
//   per wave as three 16-row blocks; K and V^T stages of 64 keys, worked in
//   two 32-key halves. A 256-row form (two 16-row blocks per wave) serves
//   grids that fill the CUs better in smaller pieces.
// * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_f16, Q held in
//   registers as the B operand of S. Every K or V^T fragment read from LDS
//   feeds three MFMAs (one per query block), so a wave moves two thirds of
//   the LDS operand bytes per product that a 32-row wave would, and each K/V
//   stage brought into LDS serves 384 rows.
// * K rows are taken in a permuted order so that each lane's S accumulators
//   hold 8 consecutive keys of its own query; after exp and a cast those are
//   the B operand of the PV product, with no data movement between lanes.
// * Software pipeline per wave: each half-step issues the MFMAs of the next
//   32 keys' scores and of O += V P for the current 32 keys (P computed by the
//   half-step before). Beside them it adds up the current P, and once the
//   scores are in, computes their P and checks them against the reference
//   max, so the softmax VALU work shares the wave's instruction stream with
//   its own matrix work and one score buffer serves every half-step.
// * K/V^T reach LDS by direct global->LDS loads (no staging registers) into a
//   4-slot ring, issued three stages ahead. LDS holds every tile in MFMA
//   operand order: fragment n of a stage is 64 lanes x 16 bytes, so every
//   operand read is one lane-linear ds_read_b128 (conflict-free, base register
//   plus immediate), and each load instruction gathers exactly one fragment.
//   One barrier per stage; the next stage's first operands are read before it.
// * Softmax in the exp2 domain with the running max and sum in registers; the
//   O rescale is skipped unless some row's max grew by more than 2^8 (exact:
//   O and the sum always share the same reference max).
// * O is normalised and staged through LDS so every row leaves in full
//   16-byte chunks of whole lines.
// * Blocks are remapped so each XCD works through a contiguous range of
//   (head, query block) items and its concurrent workgroups share K/V in L2.
// * Every fp16 attention call is planned (plan_attention_f16, launch_plan.hpp):
//   when the last round of workgroups would leave CUs idle, the last query
//   rows of each head run as a tail, in the other workgroup size over all keys
//   or split over key ranges and merged by LSE.

#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int D = 128;       // head_dim
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int kMaxNQ = 3;             // 16-row query blocks per wave: 3 (384-row workgroups) or 2 (256)
constexpr int BN = 64;                // keys per stage
static_assert(plan::kRowsPerNq == NWAVES * 16 && plan::kMaxNQ == kMaxNQ && plan::kKeyStep == BN &&
                  plan::kHeadDim == D,
              "the launch plan's shape constants are the kernel's");
constexpr int FRAG = 64 * 8;          // halves in one MFMA operand fragment
constexpr int HFRAG = 16;             // fragments per half-stage: 8 of K, then 8 of V^T
constexpr int SLOT = 2 * HFRAG * FRAG;    // halves per ring slot
constexpr int RING_BYTES = 4 * SLOT * 2;  // stage s lives in slot s % 4
constexpr int RA = 2;                     // operand reads in flight ahead of the MFMAs
constexpr int OP16 = D + 8;               // O staging pitch, fp16 (halves)
constexpr int OP32 = D + 4;               // O staging pitch, fp32 (floats)
constexpr int OSTAGE16 = NWAVES * 16 * kMaxNQ * OP16 * 2;
constexpr int OSTAGE32 = NWAVES * 16 * OP32 * 4;
constexpr int SMEM_BYTES = RING_BYTES;
static_assert(OSTAGE16 <= RING_BYTES && OSTAGE32 <= RING_BYTES, "O staging reuses the ring");
// The read-ahead registers are used round-robin by fragment index within a
// half-step; the rotation carries over half-step and stage boundaries only
// when it divides the fragments of a half-step.
static_assert(HFRAG % RA == 0, "read-ahead must divide the fragments of a half-step");
constexpr float kRescaleTau = 8.0f * kLn2;  // rescale only when a max grows by > 2^8

// v_mfma_f32_16x16x32_f16: C[16x16] += A[16x32] * B[32x16]. Lane l supplies A
// row (l % 16), k = 8*(l/16) + j, j < 8, and B column (l % 16) with the same
// k; accumulator element r of lane l is C[4*(l/16) + r][l % 16].
__device__ __forceinline__ floatx4 mfma16(const half8 &a, const half8 &b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 splat4(float v) { return floatx4{v, v, v, v}; }

// Row m of the 16-row S^T block kb (0 or 1) of a 32-key half holds key
// kperm(kb, m) of that half, so that accumulator element r of lane l holds key
// 8*(l/16) + 4*kb + r: the lane's two blocks together hold keys
// 8*(l/16)..8*(l/16)+7 of its query, in order.
__device__ __forceinline__ int kperm(int kb, int m) { return 8 * (m >> 2) + 4 * kb + (m & 3); }

// Stage s: half u (0, 1) holds K of key half 2s+1+u and V^T of key half 2s+u
// (32 keys each), so step s reads only stage s. Fragment order within half u:
// * K fragment n < 8 (head-dim step kk = n / 2, key block kb = n % 2): lane l
//   holds K[kperm(kb, l % 16)][32kk + 8(l / 16) + 0..7] of its key half.
// * V^T fragment 8 + mb (head-dim block mb < 8): lane l holds
//   V^T[16mb + l % 16][8(l / 16) + 0..7] of its key half.
// Wave w moves K fragments 2w, 2w + 1 and V^T fragments 2w, 2w + 1 of the 16
// of each kind in a stage (index 8u + n), so waves 0-3 fill half 0.
struct LoadOffsets {
    uint32_t k[2], v[2];  // bytes from the stage's first key of that kind
};

// half_base: the K base the loads add these to is the first key of the
// wave's own half (CAT), not of the stage's K part, so the half's 32 keys are
// left out of the K offsets.
__device__ __forceinline__ LoadOffsets load_offsets(int64_t v_row_stride, int wave, int lane, bool half_base) {
    const int r = lane & 15, g = lane >> 4;
    LoadOffsets o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 2 * wave + e;  // 0..15
        const int u = f >> 3, n = f & 7;
        const int kk = n >> 1, kb = n & 1;
        o.k[e] = (uint32_t)((((half_base ? 0 : 32 * u) + kperm(kb, r)) * D + 32 * kk + 8 * g) * 2);
        o.v[e] = (uint32_t)(((int64_t)(16 * n + r) * v_row_stride + 32 * u + 8 * g) * 2);
    }
    return o;
}

struct Ctx {
    const char *kh, *vh;  // this head's K and V^T (bytes)
    char *ring;           // LDS ring (wave-uniform)
    const half_t *rl;     // LDS ring + 8 * lane (this lane's operand slot)
    LoadOffsets lo;
    int wave, lane, skv, NH, T;  // NH: 32-key halves, T: stages
    int64_t vrs;
    // CAT (keys in equal blocks of 2^lg_len, read as one sequence): the block
    // table, this item's head and its first key in that sequence
    const FlashArgs *a;
    int head, key_base, lg_len;
};

// This head's K row and V^T column of the first key of 32-key half `half`
// (bytes). CAT: the key lies in block (key_base + 32 half) >> lg_len; a half
// never straddles two blocks, whose length is a multiple of 64.
template <bool CAT>
__device__ __forceinline__ const char *k_half(const Ctx &c, int half) {
    if constexpr (CAT) {
        const int key = c.key_base + 32 * half, b = key >> c.lg_len;
        return reinterpret_cast<const char *>(c.a->kv_k[b] + (int64_t)c.head * c.a->kv_k_head_stride[b] +
                                              (int64_t)(key - (b << c.lg_len)) * D);
    } else {
        return c.kh + (int64_t)half * 32 * D * 2;
    }
}
template <bool CAT>
__device__ __forceinline__ const char *v_half(const Ctx &c, int half) {
    if constexpr (CAT) {
        const int key = c.key_base + 32 * half, b = key >> c.lg_len;
        return reinterpret_cast<const char *>(c.a->kv_vt[b] + (int64_t)c.head * c.a->kv_v_head_stride[b] +
                                              (key - (b << c.lg_len)));
    } else {
        return c.vh + (int64_t)half * 32 * 2;
    }
}

// LDS byte address of the e-th fragment of kind K (0) or V^T (1) that this
// wave loads, in the slot of stage s.
__device__ __forceinline__ char *frag_dst(const Ctx &c, int s, int kind, int e) {
    const int f = 2 * c.wave + e;
    const int u = f >> 3, n = f & 7;
    return c.ring + ((s & 3) * SLOT + (u * HFRAG + kind * 8 + n) * FRAG) * 2;
}

// Buffer descriptor for raw byte addressing from `base` (stride 0, no
// range clamp): the tile base lives in scalar registers and each lane adds
// its loop-invariant 32-bit offset, so a direct load costs no vector ALU work.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, -1, 0x00020000);
}

// K of stage s >= 0 (keys 64s + 32 .. 64s + 96, all present) -> slot s. The
// wave's two fragments lie in one 32-key half, 2s + 1 + wave / 4.
template <bool CAT>
__device__ __forceinline__ void issue_k_full(const Ctx &c, int s) {
    const __amdgpu_buffer_rsrc_t r =
        CAT ? tile_rsrc(k_half<CAT>(c, 2 * s + 1 + (c.wave >> 2))) : tile_rsrc(c.kh + ((int64_t)s * BN + 32) * D * 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)frag_dst(c, s, 0, e), 16, c.lo.k[e], 0, 0, 0);
}

// V^T of stage s >= 0 (keys 64s .. 64s + 64, all present) -> slot s.
template <bool CAT>
__device__ __forceinline__ void issue_v_full(const Ctx &c, int s) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(v_half<CAT>(c, 2 * s));
#pragma unroll
    for (int e = 0; e < 2; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)frag_dst(c, s, 1, e), 16, c.lo.v[e], 0, 0, 0);
}

// This wave's K fragments of stage s when a key half of it is partial or
// missing: halves outside [0, NH) are skipped, rows past skv are clamped to
// the last key (finite values; their scores are masked). Returns the number
// of direct loads issued.
template <bool CAT>
__device__ __forceinline__ int issue_k_partial(const Ctx &c, int s) {
    const int r = c.lane & 15, g = c.lane >> 4;
    int n_issued = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 2 * c.wave + e;
        const int u = f >> 3, n = f & 7;
        const int kk = n >> 1, kb = n & 1;
        const int half = 2 * s + 1 + u;
        if (half < 0 || half >= c.NH) continue;  // wave-uniform
        const int key = min(32 * half + kperm(kb, r), c.skv - 1);
        const char *src = k_half<CAT>(c, half) + ((int64_t)(key - 32 * half) * D + 32 * kk + 8 * g) * 2;
        __builtin_amdgcn_global_load_lds((gbl_void *)src, (lds_void *)frag_dst(c, s, 0, e), 16, 0, 0);
        ++n_issued;
    }
    return n_issued;
}

// This wave's V^T fragments of stage s through registers: keys past skv are
// stored as zeros, so the zero probabilities of masked keys never meet
// non-finite data.
template <bool CAT>
__device__ __forceinline__ void stage_v_partial(const Ctx &c, int s) {
    const int r = c.lane & 15, g = c.lane >> 4;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 2 * c.wave + e;
        const int u = f >> 3, mb = f & 7;
        const int half = 2 * s + u;
        if (half < 0 || half >= c.NH) continue;  // wave-uniform
        const int key = 32 * half + 8 * g;
        const half_t *src = reinterpret_cast<const half_t *>(v_half<CAT>(c, half)) + (int64_t)(16 * mb + r) * c.vrs +
                            8 * g;
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (key + j < c.skv) ? src[j] : (half_t)0.0f;
        *reinterpret_cast<half8 *>(frag_dst(c, s, 1, e) + 16 * c.lane) = v;
    }
}

// Issue stage s (any position in the key loop); returns the number of direct
// loads it left in flight (register-path stores complete before returning).
template <bool CAT>
__device__ __forceinline__ int issue_stage(const Ctx &c, int s) {
    int n = 0;
    if (2 * s + 1 < c.NH) {  // some K half of the stage exists
        if (s >= 0 && (int64_t)s * BN + 96 <= c.skv) {
            issue_k_full<CAT>(c, s);
            n += 2;
        } else {
            n += issue_k_partial<CAT>(c, s);
        }
    }
    if (s >= 0 && 2 * s < c.NH) {  // some V^T half of the stage exists
        if ((int64_t)(s + 1) * BN <= c.skv) {
            issue_v_full<CAT>(c, s);
            n += 2;
        } else {
            stage_v_partial<CAT>(c, s);
        }
    }
    return n;
}

// Wait until at most n (<= 4) direct loads are in flight and every LDS access
// of this wave is complete.
__device__ __forceinline__ void wait_vm_lgkm(int n) {
    if (n >= 4)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(4));
    else if (n == 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(3));
    else if (n == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(2));
    else if (n == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(1));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
}

// The larger of two scores as IEEE maximum (a NaN wins): gfx950 forms
// v_maximum3_f32 from chains of it directly, where fmaxf's maxNum would first
// quiet every MFMA result with an extra v_max_f32 per operand. The two agree on
// every non-NaN input, and a NaN score makes its row's output NaN either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ half8 rd(const half_t *p) { return *reinterpret_cast<const half8 *>(p); }

// Everything that depends on the number NQ of 16-row query blocks per wave:
// three (384-row workgroups, the default) or two (256 rows, for grids that
// fill the CUs better in smaller pieces). Per-row arithmetic is the same.
template <int NQ>
struct Rows {
    static constexpr int BQ = NWAVES * 16 * NQ;  // query rows per workgroup
    typedef floatx4 SBlk[2][NQ];  // scores of one 32-key half: [key block][query block]

    // P = exp(S - m) (exp2 domain) as the fp16 B operands of the PV product:
    // pf[j] holds keys 8(l / 16) + 0..7 of the lane's query in block j.
    // PRE: the scores are already (S - m) log2(e) -- Q carries the log2(e)
    // factor and the first S MFMA starts from -m (see the kernel) -- so P is one
    // exp2 per score; otherwise one FMA per score maps S to that argument.
    template <bool PRE>
    static __device__ __forceinline__ void exp_and_pack(const SBlk &sc, half8 (&pf)[NQ], const float (&m_run)[NQ]) {
    #pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const float mneg = -m_run[j] * kLog2e;
    #pragma unroll
            for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                for (int r = 0; r < 4; ++r)
                    pf[j][4 * kb + r] =
                        (half_t)__builtin_amdgcn_exp2f(PRE ? sc[kb][j][r] : fmaf(sc[kb][j][r], kLog2e, mneg));
        }
    }

    typedef _Float16 half2v __attribute__((ext_vector_type(2)));

    // Add the fp16 probabilities (the very values the PV product weights) to the
    // lane's running sums, two per dot instruction with fp32 accumulation.
    static __device__ __forceinline__ void add_row_sums(const half8 (&pf)[NQ], float (&l_run)[NQ]) {
        const half2v one = {(half_t)1.0f, (half_t)1.0f};
    #pragma unroll
        for (int j = 0; j < NQ; ++j)
    #pragma unroll
            for (int i = 0; i < 8; i += 2)
                l_run[j] = __builtin_amdgcn_fdot2(half2v{pf[j][i], pf[j][i + 1]}, one, l_run[j], false);
    }

    // max(v) over lanes i, i ^ 16, i ^ 32, i ^ 48 (the four lanes that hold one
    // query's keys). v_permlane16_swap trades the odd 16-lane rows of one
    // register with the even rows of the other; applied to two copies of v it
    // yields v of lane i and of lane i ^ 16 in every lane i.
    static __device__ __forceinline__ float max_over_key_lanes(float v) {
        v = wave_max_across_halves(v);
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }

    // Each lane's maximum over its own 8 scores of every query block, for key
    // half `half`, masking keys past skv. The row maximum is that over the four
    // lanes of the query (max_over_key_lanes).
    template <bool MASK>
    static __device__ __forceinline__ void local_max(SBlk &s, int half, int skv, int g, float (&lm)[NQ]) {
        if (MASK) {
    #pragma unroll
            for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool out = 32 * half + 8 * g + 4 * kb + r >= skv;
    #pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        if (out) s[kb][j][r] = -INFINITY;
                }
        }
    #pragma unroll
        for (int j = 0; j < NQ; ++j) {
            // three-operand max chains: four instructions for eight values
            const float a = vmax(vmax(s[0][j][0], s[0][j][1]), s[0][j][2]);
            const float b = vmax(vmax(s[0][j][3], s[1][j][0]), s[1][j][1]);
            lm[j] = vmax(vmax(vmax(a, b), s[1][j][2]), s[1][j][3]);
        }
    }

    // Given the lanes' local maxima lm of the next scores: where some row's max
    // grew by more than 2^8, raise its reference to the new row max and rescale O
    // and the running sum to it. A lane whose own scores stay within 2^8 of the
    // reference says nothing about the rest of its row, so the row maxima (a
    // reduction over four lanes) are formed only when some lane of the wave is
    // over; otherwise every score of the wave is within 2^8 and nothing changes.
    static __device__ __forceinline__ bool update_max(const float (&lm)[NQ], float (&m_run)[NQ], float (&l_run)[NQ],
                                               floatx4 (&o)[8][NQ]) {
        bool over = false;
    #pragma unroll
        for (int j = 0; j < NQ; ++j) over = over || lm[j] > m_run[j] + kRescaleTau;
        if (!__ballot(over)) return false;
        {
    #pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const float mt = max_over_key_lanes(lm[j]);
                const float m_new = mt > m_run[j] + kRescaleTau ? mt : m_run[j];
                const float alpha = __builtin_amdgcn_exp2f((m_run[j] - m_new) * kLog2e);
                m_run[j] = m_new;
                l_run[j] *= alpha;
    #pragma unroll
                for (int mb = 0; mb < 8; ++mb) o[mb][j] *= alpha;
            }
        }
        return true;
    }

    // The same for PRE scores, which are relative to the reference already
    // (log2 units): the row max mt of S - m. Where it exceeds 8 the reference
    // moves up by mt, and O, the sum and the pending scores follow it (later
    // halves start their S accumulators from the new -m).
    static __device__ __forceinline__ bool update_max_rel(const float (&lm)[NQ], float (&m_run)[NQ], float (&l_run)[NQ],
                                                   floatx4 (&o)[8][NQ], SBlk &s, floatx4 (&negm)[NQ]) {
        bool over = false;
    #pragma unroll
        for (int j = 0; j < NQ; ++j) over = over || lm[j] > 8.0f;
        if (!__ballot(over)) return false;
        {
    #pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const float mt = max_over_key_lanes(lm[j]);
                const float delta = mt > 8.0f ? mt : 0.0f;
                const float alpha = __builtin_amdgcn_exp2f(-delta);
                m_run[j] += delta;
                l_run[j] *= alpha;
    #pragma unroll
                for (int mb = 0; mb < 8; ++mb) o[mb][j] *= alpha;
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb) s[kb][j] -= delta;
                negm[j] = splat4(-m_run[j]);
            }
        }
        return true;
    }

    struct State {
        floatx4 o[8][NQ];  // O^T accumulators [head-dim block][query block]
        half8 qf[NQ][4];   // Q as B operands [query block][head-dim step]
        floatx4 negm[NQ];  // PRE: -m, the start value of each S accumulation chain
        float m_run[NQ], l_run[NQ];
    };

    // Half U of step t: O += V P over key half 2t+U (pf, from the half-step
    // before), the scores of key half 2t+U+1 into sc, and their P into pf (after
    // the rescale check, redone if the reference moved). STEADY: every half this
    // step touches and stage t+3 are full;
    // fr holds the next RA operands on entry and exit, running on into the next
    // stage, and stage t+3's direct loads go out at fixed points. Otherwise every
    // condition is checked and reads stay within the half.
    template <bool PRE, bool CAT, bool STEADY, int U>
    static __device__ __forceinline__ void half_step(const Ctx &c, int t, SBlk &sc, half8 (&pf)[NQ], State &st,
                                              half8 (&fr)[RA]) {
        const half_t *cur = c.rl + (t & 3) * SLOT;
        const half_t *nxt = c.rl + ((t + 1) & 3) * SLOT;
        const int hv = 2 * t + U;  // key half of this PV
        const bool has_pv = STEADY || hv < c.NH;
        const bool has_s = STEADY || hv + 1 < c.NH;
    #pragma unroll
        for (int n = 0; n < HFRAG; ++n) {
            if (!(n < 8 ? has_s : has_pv)) continue;  // wave-uniform
            half8 a;
            if (STEADY) {
                a = fr[n % RA];
                const int m = U * HFRAG + n + RA;
                fr[n % RA] = rd(m < 2 * HFRAG ? cur + m * FRAG : nxt + (m - 2 * HFRAG) * FRAG);
                // stage t+3's direct loads go out a quarter of the way into each
                // half-step (K, then V^T) rather than in one burst at the step's start
                if (U == 0 && n == 4) issue_k_full<CAT>(c, t + 3);
                if (U == 1 && n == 4) issue_v_full<CAT>(c, t + 3);
            } else {
                a = rd(cur + (U * HFRAG + n) * FRAG);
            }
            if (n < 8) {
                const int kk = n >> 1, kb = n & 1;
    #pragma unroll
                for (int j = 0; j < NQ; ++j)
                    sc[kb][j] = mfma16(a, st.qf[j][kk], kk == 0 ? (PRE ? st.negm[j] : floatx4{}) : sc[kb][j]);
            } else {
                const int mb = n - 8;
    #pragma unroll
                for (int j = 0; j < NQ; ++j) st.o[mb][j] = mfma16(a, pf[j], st.o[mb][j]);
            }
        }
        if (has_pv) add_row_sums(pf, st.l_run);
        if (has_s) {
            float lm[NQ];
            const int g = c.lane >> 4;
            if (STEADY || 32 * (hv + 2) <= c.skv)
                local_max<false>(sc, hv + 1, c.skv, g, lm);
            else
                local_max<true>(sc, hv + 1, c.skv, g, lm);
            // P of the next half against the current reference, before the check:
            // redone only when the check moves the reference
            exp_and_pack<PRE>(sc, pf, st.m_run);
            // keep that work ahead of the branch (in the block with the MFMAs),
            // where the compiler would otherwise sink it into the no-rescale path
            if constexpr (NQ == 3)
                asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(pf[2]));
            else
                asm volatile("" ::"v"(pf[0]), "v"(pf[1]));
            const bool moved = PRE ? update_max_rel(lm, st.m_run, st.l_run, st.o, sc, st.negm)
                                   : update_max(lm, st.m_run, st.l_run, st.o);
            if (moved) exp_and_pack<PRE>(sc, pf, st.m_run);
        }
    }

    // Stage s holds K of key halves 2s+1, 2s+2 and V^T of halves 2s, 2s+1; the
    // prologue loads K of half 0 as stage -1 (slot 3) and stages 0..2, and
    // computes S of half 0 and its row max. Step t (0 <= t < T) adds V P of
    // halves 2t, 2t+1 into O and computes S of halves 2t+1, 2t+2; it issues stage
    // t+3 into the slot that stage t-1 used (all of whose reads finished before
    // the barrier that ended step t-1) and ends by waiting for stage t+2 and a
    // barrier, so step t+1 may read stage t+1's operands ahead of that barrier.
    //
    // PRE (set when q holds q_scaled * log2(e), as the block's projection writes
    // it): the scores come out of the S MFMAs already as (S - m) log2(e) -- the
    // log2(e) factor rides in Q and the first MFMA of each S chain starts from
    // the accumulator value -m (negm, four copies of the row's reference) instead
    // of 0 -- so the softmax needs no per-score FMA; m_run is then kept in log2
    // units.
    template <bool PRE, bool CAT>
    static __device__ __forceinline__ void attend_item(const FlashArgs &a, int work, char *smem) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
        const int g = lane >> 4;

        const int nqb = (a.sq + BQ - 1) / BQ;
        const int per_split = nqb * a.num_heads;
        // a key split, or one of several K/V blocks (both give a packed partial per part)
        const bool blocks = !CAT && a.n_kv_blocks > 0;
        const int split = (a.n_split > 1 || blocks) ? work / per_split : 0;
        const int head = (work - split * per_split) / nqb;
        const int qb = (work - split * per_split) % nqb;
        const int key_base = a.n_split > 1 ? split * a.split_len : 0;
        const int skv = blocks ? a.kv_len[split] : a.n_split > 1 ? min(a.split_len, a.skv - key_base) : a.skv;
        const half_t *kbase = blocks ? a.kv_k[split] + (int64_t)head * a.kv_k_head_stride[split]
                                     : a.k + (int64_t)head * a.k_head_stride + (int64_t)key_base * D;
        const half_t *vbase = blocks ? a.kv_vt[split] + (int64_t)head * a.kv_v_head_stride[split]
                                     : a.vt + (int64_t)head * a.v_head_stride + key_base;
        const int64_t vrs = CAT ? a.kv_v_row_stride[0] : blocks ? a.kv_v_row_stride[split] : a.v_row_stride;
        float *o32 = a.o32 ? a.o32 + (int64_t)split * a.num_heads * a.sq * D : nullptr;
        float *lse_out = a.lse ? a.lse + (int64_t)split * a.num_heads * a.sq : nullptr;
        const int64_t o32_hs = a.o32_head_stride ? a.o32_head_stride : (int64_t)a.sq * D;
        const int64_t lse_hs = a.lse_head_stride ? a.lse_head_stride : (int64_t)a.sq;

        const half_t *qh = a.q + (int64_t)head * a.q_head_stride;
        const int q0 = qb * BQ + wave * 16 * NQ;  // first query row of the wave
        State st;
    #pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int qc = min(q0 + 16 * j + (lane & 15), a.sq - 1);
    #pragma unroll
            for (int kk = 0; kk < 4; ++kk) st.qf[j][kk] = as_half8(ldg16(qh + (int64_t)qc * D + kk * 32 + 8 * g));
        }
    #pragma unroll
        for (int mb = 0; mb < 8; ++mb)
    #pragma unroll
            for (int j = 0; j < NQ; ++j) st.o[mb][j] = floatx4{};
    #pragma unroll
        for (int j = 0; j < NQ; ++j) {
            st.m_run[j] = -INFINITY;
            st.l_run[j] = 0.0f;
        }

        Ctx c;
        c.kh = reinterpret_cast<const char *>(kbase);
        c.vh = reinterpret_cast<const char *>(vbase);
        c.ring = smem;
        c.rl = reinterpret_cast<const half_t *>(smem) + 8 * lane;
        c.lo = load_offsets(vrs, wave, lane, CAT);
        c.wave = wave;
        c.lane = lane;
        c.skv = skv;
        c.NH = (skv + 31) / 32;
        c.T = (skv + BN - 1) / BN;
        c.vrs = vrs;
        c.a = &a;
        c.head = head;
        c.key_base = key_base;
        c.lg_len = a.kv_lg_len;
        const int T = c.T;

        if (T > 0) {
            SBlk sa;
            half8 pf[NQ];
            issue_stage<CAT>(c, -1);
            issue_stage<CAT>(c, 0);
            issue_stage<CAT>(c, 1);
            wait_vm_lgkm(issue_stage<CAT>(c, 2));  // stages -1, 0, 1 complete
            barrier_no_fence();
            {
                // S of key half 0 from stage -1's second K half (slot 3)
                const half_t *k0 = c.rl + 3 * SLOT + HFRAG * FRAG;
    #pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const half8 f = rd(k0 + n * FRAG);
                    const int kk = n >> 1, kb = n & 1;
    #pragma unroll
                    for (int j = 0; j < NQ; ++j) sa[kb][j] = mfma16(f, st.qf[j][kk], kk == 0 ? floatx4{} : sa[kb][j]);
                }
            }
            float lm[NQ];
            if (32 <= skv)
                local_max<false>(sa, 0, skv, g, lm);
            else
                local_max<true>(sa, 0, skv, g, lm);
            if (PRE) {
                // the first half sets the reference: its scores came out relative to 0
    #pragma unroll
                for (int j = 0; j < NQ; ++j) {
                    const float mt = max_over_key_lanes(lm[j]);
                    st.m_run[j] = mt;
    #pragma unroll
                    for (int kb = 0; kb < 2; ++kb) sa[kb][j] -= mt;
                    st.negm[j] = splat4(-mt);
                }
            } else {
                update_max(lm, st.m_run, st.l_run, st.o);
            }
            exp_and_pack<PRE>(sa, pf, st.m_run);
            // Step 0 refills slot 3: every wave must be done reading it.
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(63));
            barrier_no_fence();

            // Step t is steady when stage t+3 is full: 64t + 288 <= skv.
            const int n_steady = skv >= 288 ? (skv - 288) / BN + 1 : 0;
            half8 fr[RA];
            int t = 0;
            if (n_steady > 0) {
    #pragma unroll
                for (int n = 0; n < RA; ++n) fr[n] = rd(c.rl + n * FRAG);
                for (; t < n_steady; ++t) {
                    half_step<PRE, CAT, true, 0>(c, t, sa, pf, st, fr);
                    half_step<PRE, CAT, true, 1>(c, t, sa, pf, st, fr);
                    __builtin_amdgcn_s_waitcnt(vmcnt_only(4));  // stage t+2 has landed
                    barrier_no_fence();
                }
            }
            for (; t < T; ++t) {
                const int inflight = issue_stage<CAT>(c, t + 3);
                half_step<PRE, CAT, false, 0>(c, t, sa, pf, st, fr);
                half_step<PRE, CAT, false, 1>(c, t, sa, pf, st, fr);
                if (t + 1 < T) {
                    wait_vm_lgkm(inflight);  // stage t+2 complete (and its register-path stores)
                    barrier_no_fence();
                }
            }
        }

        // ---- epilogue: combine the four lane groups' sums, normalise, stage the
        // wave's rows through LDS and store whole rows.
        const bool empty = skv == 0;
        float inv[NQ], l_tot[NQ];
    #pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float l = st.l_run[j];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            l_tot[j] = l;
            inv[j] = empty ? 0.0f : 1.0f / l;
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
        barrier_no_fence();  // every wave is done with the ring
        const int qr = lane & 15;
        if (o32) {
            float *stg = reinterpret_cast<float *>(smem) + wave * 16 * OP32;
    #pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const int qj = q0 + 16 * j;
                const int rows = min(16, a.sq - qj);
    #pragma unroll
                for (int mb = 0; mb < 8; ++mb)
                    *reinterpret_cast<floatx4 *>(stg + qr * OP32 + 16 * mb + 4 * g) = st.o[mb][j] * inv[j];
                __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
                __builtin_amdgcn_wave_barrier();
                float *dst = o32 + (int64_t)head * o32_hs + (int64_t)qj * D;
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int row = 2 * i + (lane >> 5), chunk = lane & 31;
                    if (row < rows)
                        *reinterpret_cast<floatx4 *>(dst + (int64_t)row * D + 4 * chunk) =
                            *reinterpret_cast<const floatx4 *>(stg + row * OP32 + 4 * chunk);
                }
                __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
                __builtin_amdgcn_wave_barrier();
            }
        }
        if (a.o16) {
            half_t *stg = reinterpret_cast<half_t *>(smem) + wave * 16 * NQ * OP16;
    #pragma unroll
            for (int j = 0; j < NQ; ++j)
    #pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    half4 v;
    #pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = (half_t)(st.o[mb][j][r] * inv[j]);
                    *reinterpret_cast<half4 *>(stg + (16 * j + qr) * OP16 + 16 * mb + 4 * g) = v;
                }
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
            __builtin_amdgcn_wave_barrier();
            const int rows = min(16 * NQ, a.sq - q0);
            half_t *dst = a.o16 + (int64_t)q0 * a.o16_ld + (int64_t)head * D;
    #pragma unroll
            for (int i = 0; i < 4 * NQ; ++i) {
                const int row = 4 * i + (lane >> 4), chunk = lane & 15;
                if (row < rows)
                    *reinterpret_cast<u32x4 *>(dst + (int64_t)row * a.o16_ld + 8 * chunk) =
                        *reinterpret_cast<const u32x4 *>(stg + row * OP16 + 8 * chunk);
            }
        }
        if (lse_out && g == 0) {
    #pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const int q = q0 + 16 * j + qr;
                if (q < a.sq) {
                    // natural-log LSE; __builtin_amdgcn_logf is log2
                    const float lse = PRE ? (st.m_run[j] + __builtin_amdgcn_logf(l_tot[j])) * kLn2
                                          : st.m_run[j] + __builtin_amdgcn_logf(l_tot[j]) * kLn2;
                    lse_out[(int64_t)head * lse_hs + q] = empty ? -INFINITY : lse;
                }
            }
        }
    }

};  // struct Rows

// One workgroup per (key split, head, query block of 128 NQ rows) item, remapped
// so each XCD works through a contiguous range of items and its concurrent
// workgroups share one head's K/V in L2.
template <int NQ, bool PRE, bool CAT>
__global__ __launch_bounds__(NTHREADS) void flash_fwd_f16_d128(FlashArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
    Rows<NQ>::template attend_item<PRE, CAT>(a, xcd_remap(blockIdx.x, gridDim.x), smem);
}

template <int NQ>
void launch_rows(const FlashArgs &a, int blocks, hipStream_t stream) {
    if (a.kv_concat)
        hipLaunchKernelGGL((flash_fwd_f16_d128<NQ, false, true>), dim3(blocks), dim3(NTHREADS), 0, stream, a);
    else if (a.q_log2e)
        hipLaunchKernelGGL((flash_fwd_f16_d128<NQ, true, false>), dim3(blocks), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((flash_fwd_f16_d128<NQ, false, false>), dim3(blocks), dim3(NTHREADS), 0, stream, a);
}

}  // namespace

hipError_t launch_flash_fwd_f16(const FlashArgs &a, hipStream_t stream) {
    if (a.sq <= 0) return hipSuccess;
    const int nq = a.nq ? a.nq : kMaxNQ;
    if (nq != 2 && nq != 3) return hipErrorInvalidValue;
    // keys in equal blocks read as one sequence: q_scaled from the caller
    if (a.kv_concat && (a.q_log2e || a.n_kv_blocks <= 0)) return hipErrorInvalidValue;
    const int bq = NWAVES * 16 * nq;
    const int nqb = (a.sq + bq - 1) / bq;
    const int parts = (a.n_kv_blocks > 0 && !a.kv_concat) ? a.n_kv_blocks : a.n_split > 1 ? a.n_split : 1;
    const int blocks = nqb * a.num_heads * parts;
    if (nq == 3)
        launch_rows<3>(a, blocks, stream);
    else
        launch_rows<2>(a, blocks, stream);
    return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (256 on an MI355X).
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace

// The plan for this device (launch_plan.hpp).
AttnPlan plan_attention_f16(int num_heads, int sq, int skv, int64_t max_o_elems) {
    return plan_attention(cu_count(), num_heads, sq, skv, max_o_elems);
}

hipError_t launch_attention_f16(const FlashArgs &args, const AttnPlan &p, float *ws_o, float *ws_lse,
                                hipStream_t stream) {
    FlashArgs a = args;
    a.nq = p.nq;
    if (p.main_rows >= a.sq || a.n_split > 1 || (a.n_kv_blocks > 0 && !a.kv_concat) || (a.o16 && a.o32) ||
        (!a.o16 && !a.o32) || (p.n_split > 1 && (!ws_o || !ws_lse)))
        return launch_flash_fwd_f16(a, stream);
    hipError_t e = hipSuccess;
    const int64_t o32_hs = a.o32_head_stride ? a.o32_head_stride : (int64_t)a.sq * D;
    const int64_t lse_hs = a.lse_head_stride ? a.lse_head_stride : (int64_t)a.sq;
    if (p.main_rows > 0) {
        FlashArgs m = a;
        m.sq = p.main_rows;
        m.o32_head_stride = o32_hs;
        m.lse_head_stride = lse_hs;
        e = launch_flash_fwd_f16(m, stream);
        if (e != hipSuccess) return e;
    }
    const int tail = a.sq - p.main_rows;
    FlashArgs t = a;
    t.nq = p.tail_nq;
    t.q = a.q + (int64_t)p.main_rows * D;
    t.sq = tail;
    if (p.n_split <= 1) {  // the tail rows over all keys, into the outputs
        if (a.o16) t.o16 = a.o16 + (int64_t)p.main_rows * a.o16_ld;
        if (a.o32) {
            t.o32 = a.o32 + (int64_t)p.main_rows * D;
            t.o32_head_stride = o32_hs;
        }
        if (a.lse) {
            t.lse = a.lse + p.main_rows;
            t.lse_head_stride = lse_hs;
        }
        return launch_flash_fwd_f16(t, stream);
    }
    t.o16 = nullptr;
    t.o32 = ws_o;
    t.lse = ws_lse;
    t.o32_head_stride = 0;
    t.lse_head_stride = 0;
    t.n_split = p.n_split;
    t.split_len = p.split_len;
    e = launch_flash_fwd_f16(t, stream);
    if (e != hipSuccess) return e;
    MergeArgs mg{};
    mg.n_parts = p.n_split;
    mg.num_heads = a.num_heads;
    mg.head_dim = D;
    mg.sq = tail;
    mg.o_parts = ws_o;
    mg.lse_parts = ws_lse;
    if (a.o16) {
        mg.o_out = a.o16 + (int64_t)p.main_rows * a.o16_ld;
        mg.o_ld = a.o16_ld;
        mg.o_hs = D;
        mg.out_f16 = 1;
    } else {
        mg.o_out = a.o32 + (int64_t)p.main_rows * D;
        mg.o_ld = D;
        mg.o_hs = o32_hs;
        mg.out_f16 = 0;
    }
    if (a.lse) {
        mg.lse_out = a.lse + p.main_rows;
        mg.lse_hs = lse_hs;
    }
    return launch_lse_merge(mg, stream);
}

}  // namespace attnblk
