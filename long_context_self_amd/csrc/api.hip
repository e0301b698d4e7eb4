// C ABI of libattnblock.so (declared in include/attn_block.h): argument
// validation, block lifecycle (packed weights + workspace) and the enqueueing
// of the kernels for each entry point. No exception or abort crosses it.

#include <algorithm>
#include <cmath>
#include <cstring>

#include "attn_block.h"
#include "common.hpp"
#include "kernels.hpp"
#include "status.hpp"
#include "validate.hpp"

using namespace attnblk;

struct attn_block {
    int hidden;     // model width: x and y are [S][hidden]
    int heads;      // heads this block computes (all of them, or one rank's share)
    int head_dim;
    int width;      // heads * head_dim: width of the block's Q, K, V and attention output
    int n_ranks, rank;  // tensor-parallel shard (1, 0 for the whole block)
    int dt, device;
    int64_t max_tokens;
    void *w_qkv;  // fp16: [3*width][hidden] = [W_Q|W_K|W_V]^T (this shard's columns); fp32: [hidden][3*width]
    void *w_o;    // fp16: [hidden][width] = W_O^T (this shard's rows);              fp32: [width][hidden]
    void *ws_q, *ws_k, *ws_vt, *ws_o;
    float *ws_split_o;    // fp16: key-split attention partials (fp32), ws_split_elems floats
    float *ws_split_lse;  // fp16: their LSEs, ws_split_elems / head_dim floats
    int64_t ws_split_elems;
    int prenorm;      // RMSNorm of the input enabled (gain folded into w_qkv)
    float norm_eps;
    float *ws_rs;     // [max_tokens] per-row 1 / rms(x), when prenorm
};

namespace {

void free_block(attn_block *b) {
    if (!b) return;
    void *ptrs[] = {b->w_qkv, b->w_o, b->ws_q, b->ws_k, b->ws_vt, b->ws_o, b->ws_rs, b->ws_split_o, b->ws_split_lse};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
    delete b;
}

}  // namespace

ATTN_API const char *attn_last_error(void) { return last_error_buffer(); }

namespace {

constexpr double kLog2eD = 1.4426950408889634;

// Pack the weight shard of `rank` (heads [rank*H/N, (rank+1)*H/N): columns
// [c0, c0+width) of W_Q, W_K, W_V and rows [c0, c0+width) of W_O) and
// allocate the workspace. n_ranks = 1 is the whole block.
attn_status_t create_block(attn_block_t **out, int hidden, int num_heads, int n_ranks, int rank, int dt,
                           const void *wq, const void *wk, const void *wv, const void *wo, int64_t max_tokens,
                           hipStream_t stream) {
    *out = nullptr;
    attn_block *b = new (std::nothrow) attn_block();
    if (!b) return set_error(kOom, "attn_block_create: host allocation failed");
    std::memset(b, 0, sizeof(*b));
    b->hidden = hidden;
    b->head_dim = hidden / num_heads;
    b->heads = num_heads / n_ranks;
    b->width = b->heads * b->head_dim;
    b->n_ranks = n_ranks;
    b->rank = rank;
    b->dt = dt;
    b->max_tokens = max_tokens;
    hipError_t e = hipGetDevice(&b->device);
    if (e != hipSuccess) {
        free_block(b);
        return hip_fail("attn_block_create: hipGetDevice", e);
    }
    const size_t es = elem_size(b->dt);
    const size_t h = hidden, w = b->width, c0 = (size_t)rank * w;
    const size_t qk_bytes = (size_t)max_tokens * w * es;
    const size_t vt_bytes = (size_t)ATTN_VT_LD(max_tokens) * w * es;
    struct {
        void **p;
        size_t bytes;
    } allocs[] = {{&b->w_qkv, 3 * w * h * es}, {&b->w_o, w * h * es}, {&b->ws_q, qk_bytes},
                  {&b->ws_k, qk_bytes},        {&b->ws_vt, vt_bytes}, {&b->ws_o, qk_bytes}};
    for (auto &a : allocs) {
        e = hipMalloc(a.p, a.bytes);
        if (e != hipSuccess) {
            *a.p = nullptr;
            free_block(b);
            (void)hipGetLastError();
            return set_error(kOom, "attn_block_create: device allocation failed");
        }
    }
    if (b->dt == kF16) {
        // partials of the key-split tail of the attention launches (plan_attention_f16)
        b->ws_split_elems = std::min<int64_t>(kSplitWsFloats, 16 * (int64_t)b->width * max_tokens);
        e = hipMalloc(reinterpret_cast<void **>(&b->ws_split_o), (size_t)b->ws_split_elems * sizeof(float));
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void **>(&b->ws_split_lse),
                          (size_t)(b->ws_split_elems / b->head_dim) * sizeof(float));
        if (e != hipSuccess) {
            free_block(b);
            (void)hipGetLastError();
            return set_error(kOom, "attn_block_create: device allocation failed");
        }
    }
    const void *w3[3] = {wq, wk, wv};
    if (b->dt == kF16) {
        for (int r = 0; r < 3 && e == hipSuccess; ++r)
            e = launch_transpose_f16(static_cast<const _Float16 *>(w3[r]) + c0, hidden, (int)w, hidden,
                                     static_cast<_Float16 *>(b->w_qkv) + (size_t)r * w * h, hidden, stream);
        if (e == hipSuccess)
            e = launch_transpose_f16(static_cast<const _Float16 *>(wo) + c0 * h, (int)w, hidden, hidden,
                                     static_cast<_Float16 *>(b->w_o), (int64_t)w, stream);
    } else {
        for (int r = 0; r < 3 && e == hipSuccess; ++r)
            e = hipMemcpy2DAsync(static_cast<char *>(b->w_qkv) + r * w * es, 3 * w * es,
                                 static_cast<const char *>(w3[r]) + c0 * es, h * es, w * es, h,
                                 hipMemcpyDeviceToDevice, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(b->w_o, static_cast<const char *>(wo) + c0 * h * es, w * h * es,
                               hipMemcpyDeviceToDevice, stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        free_block(b);
        return hip_fail("attn_block_create: weight packing", e);
    }
    *out = b;
    return ATTN_OK;
}

}  // namespace

ATTN_API attn_status_t attn_block_create(attn_block_t **out, int hidden, int num_heads, attn_dtype_t dt,
                                         const void *wq, const void *wk, const void *wv, const void *wo,
                                         int64_t max_tokens, hipStream_t stream) {
    Check c = validate_create(out == nullptr, hidden, num_heads, (int)dt, wq, wk, wv, wo, max_tokens);
    if (c.status != kOk) {
        if (out) *out = nullptr;
        return report(c);
    }
    return create_block(out, hidden, num_heads, 1, 0, (int)dt, wq, wk, wv, wo, max_tokens, stream);
}

ATTN_API attn_status_t attn_block_create_shard(attn_block_t **out, int hidden, int num_heads, int n_ranks,
                                               int rank, attn_dtype_t dt, const void *wq, const void *wk,
                                               const void *wv, const void *wo, int64_t max_tokens,
                                               hipStream_t stream) {
    Check c = validate_create(out == nullptr, hidden, num_heads, (int)dt, wq, wk, wv, wo, max_tokens);
    if (c.status == kOk) c = validate_shard(num_heads, n_ranks, rank);
    if (c.status != kOk) {
        if (out) *out = nullptr;
        return report(c);
    }
    return create_block(out, hidden, num_heads, n_ranks, rank, (int)dt, wq, wk, wv, wo, max_tokens, stream);
}

ATTN_API void attn_block_destroy(attn_block_t *blk) {
    if (!blk) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(blk->device);
    (void)hipDeviceSynchronize();
    free_block(blk);
    (void)hipSetDevice(cur);
}

ATTN_API attn_status_t attn_block_set_prenorm(attn_block_t *blk, const void *gain, float eps, hipStream_t stream) {
    Check c = validate_set_prenorm(blk == nullptr, eps, blk && blk->prenorm);
    if (c.status != kOk) return report(c);
    if (gain && !aligned(gain, 4)) return set_error(kInvalid, "attn_block_set_prenorm: gain misaligned");
    if (!blk->ws_rs) {
        hipError_t e = hipMalloc(reinterpret_cast<void **>(&blk->ws_rs), (size_t)blk->max_tokens * sizeof(float));
        if (e != hipSuccess) {
            blk->ws_rs = nullptr;
            (void)hipGetLastError();
            return set_error(kOom, "attn_block_set_prenorm: device allocation failed");
        }
    }
    if (gain) {
        HIP_TRY("attn_block_set_prenorm: gain folding",
                launch_fold_gain(blk->w_qkv, blk->dt == kF16, blk->hidden, 3 * (int64_t)blk->width, gain, stream));
        HIP_TRY("attn_block_set_prenorm: hipStreamSynchronize", hipStreamSynchronize(stream));
    }
    blk->prenorm = 1;
    blk->norm_eps = eps;
    return ATTN_OK;
}

ATTN_API attn_status_t attn_block_forward(attn_block_t *blk, const void *x, void *y, int64_t seq, int64_t batch,
                                          const attn_taps_t *taps, hipStream_t stream) {
    TapsView tv{};
    if (taps)
        tv = TapsView{taps->q_scaled, taps->k, taps->v_t, taps->attn_out, taps->lse, taps->qkv_only, taps->events,
                      taps->v};
    Check c = validate_forward(blk == nullptr, blk ? blk->dt : 0, blk ? blk->hidden : 0,
                               blk ? blk->max_tokens : 0, x, y, seq, batch, taps ? &tv : nullptr);
    if (c.status != kOk) return report(c);
    if (seq == 0) return ATTN_OK;
    const int S = (int)(seq * batch);
    const int h = blk->hidden, d = blk->head_dim, H = blk->heads, wd = blk->width;
    const int64_t vt_ld = ATTN_VT_LD(S);
    const float q_scale = (float)(1.0 / std::sqrt((double)d));
    // fp16: the block's own Q holds q_scaled * log2(e) (one rounding from the
    // fp32 accumulator, like q_scaled itself), so its attention needs no
    // per-score multiply; a q_scaled tap gets the plain q_scaled in addition.
    const float q_scale_log2e = (float)(kLog2eD / std::sqrt((double)d));
    void *q = (taps && taps->q_scaled) ? taps->q_scaled : blk->ws_q;
    void *k = (taps && taps->k) ? taps->k : blk->ws_k;
    void *vt = (taps && taps->v_t) ? taps->v_t : blk->ws_vt;
    void *o = (taps && taps->attn_out) ? taps->attn_out : blk->ws_o;
    float *lse = taps ? taps->lse : nullptr;
    const bool qkv_only = taps && taps->qkv_only;
    hipEvent_t *ev = taps ? taps->events : nullptr;
    void *v_rows = taps ? taps->v : nullptr;  // row-major V tap: transposed back from V^T
#define MARK(i) \
    if (ev) HIP_TRY("attn_block_forward: hipEventRecord", hipEventRecord(ev[i], stream))
    MARK(0);
    const float *row_scale = nullptr;
    if (blk->prenorm) {
        HIP_TRY("attn_block_forward: RMSNorm row scales",
                launch_rms_rowscale(x, blk->dt == kF16, S, h, blk->norm_eps, blk->ws_rs, stream));
        row_scale = blk->ws_rs;
    }

    if (blk->dt == kF16) {
        GemmArgs g{};
        g.a = static_cast<const _Float16 *>(x);
        g.lda = h;
        g.b = static_cast<const _Float16 *>(blk->w_qkv);
        g.ldb = h;
        g.M = S;
        g.N = 3 * wd;
        g.K = h;
        g.mode = kQkv;
        g.q = static_cast<_Float16 *>(blk->ws_q);
        g.k = static_cast<_Float16 *>(k);
        g.vt = static_cast<_Float16 *>(vt);
        g.vt_ld = vt_ld;
        g.hidden = wd;
        g.head_dim = d;
        g.q_scale = q_scale_log2e;
        g.row_scale = row_scale;
        g.q_tap = (taps && taps->q_scaled) ? static_cast<_Float16 *>(taps->q_scaled) : nullptr;
        g.q_tap_scale = q_scale;
        HIP_TRY("attn_block_forward: QKV projection", launch_gemm_f16(g, stream));
        if (v_rows)
            HIP_TRY("attn_block_forward: V tap",
                    launch_transpose_heads(vt, (int64_t)d * vt_ld, vt_ld, v_rows, (int64_t)S * d, d, H, d, d, S, 2,
                                           stream));
        MARK(1);
        if (qkv_only) return ATTN_OK;
        FlashArgs fa{};
        fa.q = g.q;
        fa.q_log2e = 1;
        fa.k = g.k;
        fa.vt = g.vt;
        fa.q_head_stride = (int64_t)S * d;
        fa.k_head_stride = (int64_t)S * d;
        fa.v_head_stride = (int64_t)d * vt_ld;
        fa.v_row_stride = vt_ld;
        fa.sq = S;
        fa.skv = S;
        fa.num_heads = H;
        fa.o16 = static_cast<_Float16 *>(o);
        fa.o16_ld = wd;
        fa.lse = lse;
        const AttnPlan plan = plan_attention_f16(H, S, S, blk->ws_split_elems);
        HIP_TRY("attn_block_forward: attention",
                launch_attention_f16(fa, plan, blk->ws_split_o, blk->ws_split_lse, stream));
        MARK(2);
        GemmArgs go{};
        go.a = static_cast<const _Float16 *>(o);
        go.lda = wd;
        go.b = static_cast<const _Float16 *>(blk->w_o);
        go.ldb = wd;
        go.M = S;
        go.N = h;
        go.K = wd;
        go.mode = kPlain;
        go.c = static_cast<_Float16 *>(y);
        go.ldc = h;
        HIP_TRY("attn_block_forward: output projection", launch_gemm_f16(go, stream));
        MARK(3);
    } else {
        GemmArgsF32 g{};
        g.a = static_cast<const float *>(x);
        g.lda = h;
        g.w = static_cast<const float *>(blk->w_qkv);
        g.ldw = 3 * wd;
        g.M = S;
        g.N = 3 * wd;
        g.K = h;
        g.mode = kQkv;
        g.q = static_cast<float *>(q);
        g.k = static_cast<float *>(k);
        g.vt = static_cast<float *>(vt);
        g.vt_ld = vt_ld;
        g.hidden = wd;
        g.head_dim = d;
        g.q_scale = q_scale;
        g.row_scale = row_scale;
        HIP_TRY("attn_block_forward: QKV projection", launch_gemm_f32(g, stream));
        if (v_rows)
            HIP_TRY("attn_block_forward: V tap",
                    launch_transpose_heads(vt, (int64_t)d * vt_ld, vt_ld, v_rows, (int64_t)S * d, d, H, d, d, S, 4,
                                           stream));
        MARK(1);
        if (qkv_only) return ATTN_OK;
        FlashArgsF32 fa{};
        fa.q = g.q;
        fa.k = g.k;
        fa.vt = g.vt;
        fa.q_head_stride = (int64_t)S * d;
        fa.k_head_stride = (int64_t)S * d;
        fa.v_head_stride = (int64_t)d * vt_ld;
        fa.v_row_stride = vt_ld;
        fa.sq = S;
        fa.skv = S;
        fa.num_heads = H;
        fa.head_dim = d;
        fa.otok = static_cast<float *>(o);
        fa.otok_ld = wd;
        fa.lse = lse;
        HIP_TRY("attn_block_forward: attention", launch_flash_fwd_f32(fa, stream));
        MARK(2);
        GemmArgsF32 go{};
        go.a = static_cast<const float *>(o);
        go.lda = wd;
        go.w = static_cast<const float *>(blk->w_o);
        go.ldw = h;
        go.M = S;
        go.N = h;
        go.K = wd;
        go.mode = kPlain;
        go.c = static_cast<float *>(y);
        go.ldc = h;
        HIP_TRY("attn_block_forward: output projection", launch_gemm_f32(go, stream));
        MARK(3);
    }
#undef MARK
    return ATTN_OK;
}

ATTN_API attn_status_t attn_merge_lse(int n_parts, int num_heads, int head_dim, int64_t sq, const float *o_parts,
                                      const float *lse_parts, void *o_out, attn_dtype_t out_dt, float *lse_out,
                                      hipStream_t stream) {
    Check c = validate_merge(n_parts, num_heads, head_dim, sq, o_parts, lse_parts, o_out, (int)out_dt, lse_out);
    if (c.status != kOk) return report(c);
    if (sq == 0) return ATTN_OK;
    MergeArgs m{};
    m.n_parts = n_parts;
    m.num_heads = num_heads;
    m.head_dim = head_dim;
    m.sq = sq;
    m.o_parts = o_parts;
    m.lse_parts = lse_parts;
    m.o_out = o_out;
    m.out_f16 = out_dt == ATTN_F16;
    m.lse_out = lse_out;
    HIP_TRY("attn_merge_lse", launch_lse_merge(m, stream));
    return ATTN_OK;
}

ATTN_API attn_status_t attn_heads_forward(int num_heads, int head_dim, attn_dtype_t dt, const void *q_scaled,
                                          const void *k, const void *v_t, int64_t seq, void *o, int64_t o_ld,
                                          float *lse, hipStream_t stream) {
    Check c = validate_heads_forward(num_heads, head_dim, (int)dt, q_scaled, k, v_t, seq, o, o_ld, lse);
    if (c.status != kOk) return report(c);
    if (seq == 0) return ATTN_OK;
    const int64_t vt_ld = ATTN_VT_LD(seq);
    if (dt == ATTN_F16) {
        FlashArgs fa{};
        fa.q = static_cast<const _Float16 *>(q_scaled);
        fa.k = static_cast<const _Float16 *>(k);
        fa.vt = static_cast<const _Float16 *>(v_t);
        fa.q_head_stride = seq * head_dim;
        fa.k_head_stride = seq * head_dim;
        fa.v_head_stride = (int64_t)head_dim * vt_ld;
        fa.v_row_stride = vt_ld;
        fa.sq = (int)seq;
        fa.skv = (int)seq;
        fa.num_heads = num_heads;
        fa.o16 = static_cast<_Float16 *>(o);
        fa.o16_ld = o_ld;
        fa.lse = lse;
        const AttnPlan plan = plan_attention_f16(num_heads, (int)seq, (int)seq, kSplitWsFloats);
        if (plan.n_split <= 1) {
            HIP_TRY("attn_heads_forward", launch_attention_f16(fa, plan, nullptr, nullptr, stream));
            return ATTN_OK;
        }
        hipMemPool_t pool = nullptr;
        HIP_TRY("attn_heads_forward: pool", staging_pool(&pool));
        void *ws = nullptr;
        const hipError_t ea =
            hipMallocFromPoolAsync(&ws, (size_t)(plan.o_elems + plan.lse_elems) * sizeof(float), pool, stream);
        if (ea != hipSuccess) {
            (void)hipGetLastError();
            return set_error(kOom, "attn_heads_forward: split workspace allocation failed");
        }
        float *wo = static_cast<float *>(ws);
        const hipError_t el = launch_attention_f16(fa, plan, wo, wo + plan.o_elems, stream);
        // released in stream order after the kernels that use it
        const hipError_t ef = hipFreeAsync(ws, stream);
        HIP_TRY("attn_heads_forward", el);
        HIP_TRY("attn_heads_forward: workspace release", ef);
    } else {
        FlashArgsF32 fa{};
        fa.q = static_cast<const float *>(q_scaled);
        fa.k = static_cast<const float *>(k);
        fa.vt = static_cast<const float *>(v_t);
        fa.q_head_stride = seq * head_dim;
        fa.k_head_stride = seq * head_dim;
        fa.v_head_stride = (int64_t)head_dim * vt_ld;
        fa.v_row_stride = vt_ld;
        fa.sq = (int)seq;
        fa.skv = (int)seq;
        fa.num_heads = num_heads;
        fa.head_dim = head_dim;
        fa.otok = static_cast<float *>(o);
        fa.otok_ld = o_ld;
        fa.lse = lse;
        HIP_TRY("attn_heads_forward", launch_flash_fwd_f32(fa, stream));
    }
    return ATTN_OK;
}

ATTN_API attn_status_t attn_ulysses_gather(int n_ranks, int num_heads_local, int head_dim, attn_dtype_t dt,
                                           int64_t seq, const void *recv_q, const void *recv_k,
                                           const void *recv_vt, void *q_scaled, void *k, void *v_t,
                                           hipStream_t stream) {
    Check c = validate_ulysses_gather(n_ranks, num_heads_local, head_dim, (int)dt, seq, recv_q, recv_k, recv_vt,
                                      q_scaled, k, v_t);
    if (c.status != kOk) return report(c);
    if (seq == 0) return ATTN_OK;
    const int64_t es = elem_size((int)dt), ch = seq / n_ranks, d = head_dim, hl = num_heads_local;
    // Q, K: block p of head jj ([ch][d], contiguous) -> rows [p*ch, (p+1)*ch) of head jj
    const void *srcs[2] = {recv_q, recv_k};
    void *dsts[2] = {q_scaled, k};
    for (int t = 0; t < 2; ++t) {
        SegCopyArgs a{};
        a.src = static_cast<const char *>(srcs[t]);
        a.dst = static_cast<char *>(dsts[t]);
        a.n_outer = (uint32_t)n_ranks;
        a.n_inner = (uint32_t)hl;
        a.src_so = hl * ch * d * es;
        a.src_si = ch * d * es;
        a.dst_so = ch * d * es;
        a.dst_si = seq * d * es;
        a.chunks_per_seg = (uint32_t)(ch * d * es / 16);
        HIP_TRY("attn_ulysses_gather: Q/K", launch_seg_copy(a, stream));
    }
    // V^T: row (jj, c) of block p ([ch] keys, contiguous) -> keys [p*ch, (p+1)*ch) of that row
    SegCopyArgs a{};
    a.src = static_cast<const char *>(recv_vt);
    a.dst = static_cast<char *>(v_t);
    a.n_outer = (uint32_t)n_ranks;
    a.n_inner = (uint32_t)(hl * d);
    a.src_so = hl * d * ch * es;
    a.src_si = ch * es;
    a.dst_so = ch * es;
    a.dst_si = ATTN_VT_LD(seq) * es;
    a.chunks_per_seg = (uint32_t)(ch * es / 16);
    HIP_TRY("attn_ulysses_gather: V^T", launch_seg_copy(a, stream));
    return ATTN_OK;
}

ATTN_API attn_status_t attn_ulysses_unpack_o(int n_ranks, int num_heads, int head_dim, attn_dtype_t dt, int64_t rows,
                                             const void *recv_o, void *o, hipStream_t stream) {
    Check c = validate_ulysses_unpack(n_ranks, num_heads, head_dim, (int)dt, rows, recv_o, o);
    if (c.status != kOk) return report(c);
    if (rows == 0) return ATTN_OK;
    const int64_t es = elem_size((int)dt), wl = (int64_t)(num_heads / n_ranks) * head_dim;
    // block r, row i ([wl] columns) -> row i, columns [r*wl, (r+1)*wl)
    SegCopyArgs a{};
    a.src = static_cast<const char *>(recv_o);
    a.dst = static_cast<char *>(o);
    a.n_outer = (uint32_t)n_ranks;
    a.n_inner = (uint32_t)rows;
    a.src_so = rows * wl * es;
    a.src_si = wl * es;
    a.dst_so = wl * es;
    a.dst_si = n_ranks * wl * es;
    a.chunks_per_seg = (uint32_t)(wl * es / 16);
    HIP_TRY("attn_ulysses_unpack_o", launch_seg_copy(a, stream));
    return ATTN_OK;
}
