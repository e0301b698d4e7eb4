// Argument validation for every C entry point. Pure C++ with no HIP calls, so
// a failed check provably enqueues nothing, and the checks can be compiled
// and tested on a host without a GPU.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>

namespace attnblk {

// Mirrors attn_status_t / attn_dtype_t of include/attn_block.h.
enum Status { kOk = 0, kInvalid = 1, kUnsupported = 2, kOom = 3, kHip = 4 };
enum Dtype { kF16 = 0, kF32 = 1 };

constexpr int64_t kMaxTokens = int64_t(1) << 24;  // per forward / per partial side
constexpr int kMaxHidden = 32768;
constexpr int kMaxParts = 4096;

struct Check {
    int status;
    char msg[256];
};

inline Check ok() {
    Check c;
    c.status = kOk;
    c.msg[0] = '\0';
    return c;
}

inline Check fail(int status, const char *fmt, ...) {
    Check c;
    c.status = status;
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(c.msg, sizeof(c.msg), fmt, ap);
    va_end(ap);
    return c;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int elem_size(int dt) { return dt == kF16 ? 2 : 4; }
inline bool dtype_known(int dt) { return dt == kF16 || dt == kF32; }
inline bool head_dim_supported(int dt, int d) { return dt == kF16 ? d == 128 : (d == 64 || d == 128); }
// Element count alignment of strides used by 16-byte vector accesses.
inline int64_t vec_elems(int dt) { return dt == kF16 ? 8 : 4; }

inline bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

inline Check validate_create(bool out_null, int hidden, int num_heads, int dt, const void *wq,
                             const void *wk, const void *wv, const void *wo, int64_t max_tokens) {
    if (out_null) return fail(kInvalid, "attn_block_create: out is NULL");
    if (!dtype_known(dt)) return fail(kInvalid, "attn_block_create: unknown dtype %d", dt);
    if (num_heads < 1) return fail(kInvalid, "attn_block_create: num_heads %d < 1", num_heads);
    if (hidden < 1 || hidden % num_heads != 0)
        return fail(kInvalid, "attn_block_create: hidden %d is not a multiple of num_heads %d", hidden,
                    num_heads);
    if (hidden > kMaxHidden) return fail(kUnsupported, "attn_block_create: hidden %d > %d", hidden, kMaxHidden);
    const int d = hidden / num_heads;
    if (!head_dim_supported(dt, d))
        return fail(kUnsupported, "attn_block_create: head_dim %d not supported for dtype %d", d, dt);
    if (!wq || !wk || !wv || !wo) return fail(kInvalid, "attn_block_create: a weight pointer is NULL");
    if (!aligned(wq, 16) || !aligned(wk, 16) || !aligned(wv, 16) || !aligned(wo, 16))
        return fail(kInvalid, "attn_block_create: weights must be 16-byte aligned");
    if (max_tokens < 1) return fail(kInvalid, "attn_block_create: max_tokens %lld < 1", (long long)max_tokens);
    if (max_tokens > kMaxTokens)
        return fail(kUnsupported, "attn_block_create: max_tokens %lld > %lld", (long long)max_tokens,
                    (long long)kMaxTokens);
    return ok();
}

struct TapsView {
    const void *q_scaled, *k, *v_t, *attn_out;
    const float *lse;
    int qkv_only;
    const void *events;  // array of 4 events; entries are checked by the caller
    const void *v;
};

inline Check validate_forward(bool blk_null, int dt, int hidden, int64_t max_tokens, const void *x,
                              const void *y, int64_t seq, int64_t batch, const TapsView *taps) {
    if (blk_null) return fail(kInvalid, "attn_block_forward: blk is NULL");
    if (batch < 1) return fail(kInvalid, "attn_block_forward: batch %lld < 1", (long long)batch);
    if (batch != 1) return fail(kUnsupported, "attn_block_forward: batch %lld != 1", (long long)batch);
    if (seq < 0) return fail(kInvalid, "attn_block_forward: seq %lld < 0", (long long)seq);
    if (seq * batch > max_tokens)
        return fail(kInvalid, "attn_block_forward: seq*batch %lld exceeds max_tokens %lld",
                    (long long)(seq * batch), (long long)max_tokens);
    if (seq == 0) return ok();
    const bool qkv_only = taps && taps->qkv_only;
    if (!x) return fail(kInvalid, "attn_block_forward: x is NULL");
    if (!qkv_only && !y) return fail(kInvalid, "attn_block_forward: y is NULL");
    if (!aligned(x, 16) || (y && !aligned(y, 16)))
        return fail(kInvalid, "attn_block_forward: x and y must be 16-byte aligned");
    const int64_t bytes = seq * batch * hidden * elem_size(dt);
    if (y && !qkv_only && overlap(x, bytes, y, bytes)) return fail(kInvalid, "attn_block_forward: x and y overlap");
    if (taps) {
        const void *p16[5] = {taps->q_scaled, taps->k, taps->v_t, taps->attn_out, taps->v};
        for (const void *p : p16)
            if (p && !aligned(p, 16)) return fail(kInvalid, "attn_block_forward: tap buffers must be 16-byte aligned");
        if (taps->lse && !aligned(taps->lse, 4)) return fail(kInvalid, "attn_block_forward: lse tap misaligned");
    }
    return ok();
}

// Checks shared by the partial entry points: sizes, q and the outputs.
inline Check validate_partial_common(const char *what, int num_heads, int head_dim, int dt, const void *q,
                                     int64_t sq, int64_t qhs, int64_t skv, const float *o_part,
                                     const float *lse_part) {
    if (!dtype_known(dt)) return fail(kInvalid, "%s: unknown dtype %d", what, dt);
    if (num_heads < 1) return fail(kInvalid, "%s: num_heads %d < 1", what, num_heads);
    if (!head_dim_supported(dt, head_dim))
        return fail(kUnsupported, "%s: head_dim %d not supported for dtype %d", what, head_dim, dt);
    if (sq < 0 || skv < 0) return fail(kInvalid, "%s: negative sq or skv", what);
    if (sq > kMaxTokens || skv > kMaxTokens)
        return fail(kUnsupported, "%s: sq or skv above %lld", what, (long long)kMaxTokens);
    if (sq == 0) return ok();
    if (!q || !o_part || !lse_part) return fail(kInvalid, "%s: q, o_part or lse_part is NULL", what);
    if (!aligned(q, 16) || !aligned(o_part, 16))
        return fail(kInvalid, "%s: q and o_part must be 16-byte aligned", what);
    if (!aligned(lse_part, 4)) return fail(kInvalid, "%s: lse_part misaligned", what);
    if (qhs < 0) return fail(kInvalid, "%s: negative stride", what);
    if (qhs % vec_elems(dt))
        return fail(kInvalid, "%s: head strides must be multiples of %lld", what, (long long)vec_elems(dt));
    if (num_heads > 1 && qhs < sq * head_dim)
        return fail(kInvalid, "%s: q_head_stride %lld < sq*head_dim", what, (long long)qhs);
    return ok();
}

// attn_partial_forward_vt: K [H][skv][d] and V^T [H][d][v_row_stride].
inline Check validate_partial(int num_heads, int head_dim, int dt, const void *q, int64_t sq, int64_t qhs,
                              const void *k, int64_t skv, int64_t khs, const void *vt, int64_t vhs,
                              int64_t vrs, const float *o_part, const float *lse_part) {
    const char *what = "attn_partial_forward_vt";
    Check c = validate_partial_common(what, num_heads, head_dim, dt, q, sq, qhs, skv, o_part, lse_part);
    if (c.status != kOk || sq == 0) return c;
    if (skv > 0 && (!k || !vt)) return fail(kInvalid, "%s: k or v_t is NULL", what);
    if (skv > 0 && (!aligned(k, 16) || !aligned(vt, 16)))
        return fail(kInvalid, "%s: k and v_t must be 16-byte aligned", what);
    const int64_t ve = vec_elems(dt);
    if (khs < 0 || vhs < 0 || vrs < 0) return fail(kInvalid, "%s: negative stride", what);
    if (khs % ve || vhs % ve || vrs % ve)
        return fail(kInvalid, "%s: head strides and v_row_stride must be multiples of %lld", what, (long long)ve);
    if (skv > 0) {
        if (vrs < skv) return fail(kInvalid, "%s: v_row_stride %lld < skv", what, (long long)vrs);
        if (vrs > kMaxTokens)  // keeps every in-head V^T offset within 32 bits
            return fail(kUnsupported, "%s: v_row_stride above %lld", what, (long long)kMaxTokens);
        if (num_heads > 1 && (khs < skv * head_dim || vhs < head_dim * vrs))
            return fail(kInvalid, "%s: k/v head strides smaller than one head", what);
    }
    return ok();
}

// attn_partial_forward: K and V both [H][skv][d] with one head stride.
inline Check validate_partial_rows(const char *what, int num_heads, int head_dim, int dt, const void *q, int64_t sq,
                                   int64_t qhs, const void *k, const void *v, int64_t skv, int64_t kvhs,
                                   const float *o_part, const float *lse_part) {
    Check c = validate_partial_common(what, num_heads, head_dim, dt, q, sq, qhs, skv, o_part, lse_part);
    if (c.status != kOk || sq == 0) return c;
    if (skv > 0 && (!k || !v)) return fail(kInvalid, "%s: k or v is NULL", what);
    if (skv > 0 && (!aligned(k, 16) || !aligned(v, 16)))
        return fail(kInvalid, "%s: k and v must be 16-byte aligned", what);
    if (kvhs < 0) return fail(kInvalid, "%s: negative stride", what);
    if (kvhs % vec_elems(dt))
        return fail(kInvalid, "%s: head strides must be multiples of %lld", what, (long long)vec_elems(dt));
    if (skv > 0 && num_heads > 1 && kvhs < skv * head_dim)
        return fail(kInvalid, "%s: kv_head_stride %lld < skv*head_dim", what, (long long)kvhs);
    return ok();
}

inline Check validate_set_prenorm(bool blk_null, float eps, bool already_set) {
    if (blk_null) return fail(kInvalid, "attn_block_set_prenorm: blk is NULL");
    if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(kInvalid, "attn_block_set_prenorm: eps must be finite and >= 0");
    if (already_set) return fail(kInvalid, "attn_block_set_prenorm: pre-norm is already enabled on this block");
    return ok();
}

inline Check validate_shard(int num_heads, int n_ranks, int rank) {
    if (n_ranks < 1) return fail(kInvalid, "attn_block_create_shard: n_ranks %d < 1", n_ranks);
    if (num_heads % n_ranks != 0)
        return fail(kInvalid, "attn_block_create_shard: num_heads %d is not a multiple of n_ranks %d", num_heads,
                    n_ranks);
    if (rank < 0 || rank >= n_ranks) return fail(kInvalid, "attn_block_create_shard: rank %d outside [0, %d)", rank,
                                                 n_ranks);
    return ok();
}

inline Check validate_heads_forward(int num_heads, int head_dim, int dt, const void *q, const void *k,
                                    const void *vt, int64_t seq, const void *o, int64_t o_ld, const float *lse) {
    if (!dtype_known(dt)) return fail(kInvalid, "attn_heads_forward: unknown dtype %d", dt);
    if (num_heads < 1) return fail(kInvalid, "attn_heads_forward: num_heads %d < 1", num_heads);
    if (!head_dim_supported(dt, head_dim))
        return fail(kUnsupported, "attn_heads_forward: head_dim %d not supported for dtype %d", head_dim, dt);
    if (seq < 0) return fail(kInvalid, "attn_heads_forward: negative seq");
    if (seq > kMaxTokens) return fail(kUnsupported, "attn_heads_forward: seq above %lld", (long long)kMaxTokens);
    if (seq == 0) return ok();
    if (!q || !k || !vt || !o) return fail(kInvalid, "attn_heads_forward: q, k, v_t or o is NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(o, 16))
        return fail(kInvalid, "attn_heads_forward: q, k, v_t and o must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(kInvalid, "attn_heads_forward: lse misaligned");
    if (o_ld < (int64_t)num_heads * head_dim || o_ld % vec_elems(dt))
        return fail(kInvalid, "attn_heads_forward: o_ld %lld must be >= num_heads*head_dim and a multiple of %lld",
                    (long long)o_ld, (long long)vec_elems(dt));
    return ok();
}

// Ulysses layouts: seq split into n_ranks chunks of seq/n_ranks rows, each a
// multiple of 8 so that every moved segment is a whole number of 16-byte
// chunks (fp16) and V^T rows need no padding.
inline Check validate_ulysses(const char *what, int n_ranks, int num_heads, int head_dim, int dt, int64_t seq) {
    if (!dtype_known(dt)) return fail(kInvalid, "%s: unknown dtype %d", what, dt);
    if (n_ranks < 1 || num_heads < 1) return fail(kInvalid, "%s: n_ranks and num_heads must be >= 1", what);
    if (!head_dim_supported(dt, head_dim))
        return fail(kUnsupported, "%s: head_dim %d not supported for dtype %d", what, head_dim, dt);
    if (seq < 0 || seq % n_ranks != 0 || (seq / n_ranks) % 8 != 0)
        return fail(kInvalid, "%s: seq %lld must be n_ranks x a multiple of 8", what, (long long)seq);
    if (seq > kMaxTokens) return fail(kUnsupported, "%s: seq above %lld", what, (long long)kMaxTokens);
    return ok();
}

inline Check validate_ulysses_gather(int n_ranks, int num_heads_local, int head_dim, int dt, int64_t seq,
                                     const void *rq, const void *rk, const void *rvt, const void *q, const void *k,
                                     const void *vt) {
    Check c = validate_ulysses("attn_ulysses_gather", n_ranks, num_heads_local, head_dim, dt, seq);
    if (c.status != kOk || seq == 0) return c;
    const void *ps[6] = {rq, rk, rvt, q, k, vt};
    for (const void *p : ps) {
        if (!p) return fail(kInvalid, "attn_ulysses_gather: NULL buffer");
        if (!aligned(p, 16)) return fail(kInvalid, "attn_ulysses_gather: buffers must be 16-byte aligned");
    }
    return ok();
}

inline Check validate_ulysses_unpack(int n_ranks, int num_heads, int head_dim, int dt, int64_t rows,
                                     const void *recv, const void *o) {
    if (!dtype_known(dt)) return fail(kInvalid, "attn_ulysses_unpack_o: unknown dtype %d", dt);
    if (n_ranks < 1 || num_heads < 1 || num_heads % n_ranks != 0)
        return fail(kInvalid, "attn_ulysses_unpack_o: num_heads %d must be a positive multiple of n_ranks %d",
                    num_heads, n_ranks);
    if (!head_dim_supported(dt, head_dim))
        return fail(kUnsupported, "attn_ulysses_unpack_o: head_dim %d not supported for dtype %d", head_dim, dt);
    if (rows < 0) return fail(kInvalid, "attn_ulysses_unpack_o: negative rows");
    if (rows > kMaxTokens) return fail(kUnsupported, "attn_ulysses_unpack_o: rows above %lld", (long long)kMaxTokens);
    if (rows == 0) return ok();
    if (!recv || !o) return fail(kInvalid, "attn_ulysses_unpack_o: NULL buffer");
    if (!aligned(recv, 16) || !aligned(o, 16))
        return fail(kInvalid, "attn_ulysses_unpack_o: buffers must be 16-byte aligned");
    return ok();
}

inline Check validate_ring_create(bool out_null, int num_heads, int head_dim, int dt, int n_blocks, int64_t max_sq,
                                  int64_t max_block) {
    if (out_null) return fail(kInvalid, "attn_ring_create: out is NULL");
    if (!dtype_known(dt)) return fail(kInvalid, "attn_ring_create: unknown dtype %d", dt);
    if (num_heads < 1) return fail(kInvalid, "attn_ring_create: num_heads %d < 1", num_heads);
    if (!head_dim_supported(dt, head_dim))
        return fail(kUnsupported, "attn_ring_create: head_dim %d not supported for dtype %d", head_dim, dt);
    if (n_blocks < 1) return fail(kInvalid, "attn_ring_create: n_blocks %d < 1", n_blocks);
    if (n_blocks > kMaxParts) return fail(kUnsupported, "attn_ring_create: n_blocks %d > %d", n_blocks, kMaxParts);
    if (max_sq < 1 || max_block < 1) return fail(kInvalid, "attn_ring_create: max_sq and max_block_len must be >= 1");
    if (max_sq > kMaxTokens || max_block > kMaxTokens)
        return fail(kUnsupported, "attn_ring_create: max_sq or max_block_len above %lld", (long long)kMaxTokens);
    return ok();
}

inline Check validate_ring_forward(bool ring_null, int n_blocks, int64_t max_sq, int64_t max_block, const void *q,
                                   int64_t sq, const void *const *kb, const void *const *vb, const int64_t *lens,
                                   const void *o, const float *lse) {
    if (ring_null) return fail(kInvalid, "attn_ring_forward: ring is NULL");
    if (sq < 0 || sq > max_sq) return fail(kInvalid, "attn_ring_forward: sq %lld outside [0, %lld]", (long long)sq,
                                           (long long)max_sq);
    if (sq == 0) return ok();
    if (!q || !o || !kb || !vb || !lens) return fail(kInvalid, "attn_ring_forward: NULL argument");
    if (!aligned(q, 16) || !aligned(o, 16)) return fail(kInvalid, "attn_ring_forward: q and o must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(kInvalid, "attn_ring_forward: lse misaligned");
    for (int b = 0; b < n_blocks; ++b) {
        if (lens[b] < 0 || lens[b] > max_block)
            return fail(kInvalid, "attn_ring_forward: block %d length %lld outside [0, %lld]", b, (long long)lens[b],
                        (long long)max_block);
        if (lens[b] > 0 && (!kb[b] || !vb[b])) return fail(kInvalid, "attn_ring_forward: block %d K or V^T is NULL", b);
    }
    return ok();
}

inline Check validate_merge(int n_parts, int num_heads, int head_dim, int64_t sq, const float *o_parts,
                            const float *lse_parts, const void *o_out, int out_dt, const float *lse_out) {
    if (n_parts < 1) return fail(kInvalid, "attn_merge_lse: n_parts %d < 1", n_parts);
    if (n_parts > kMaxParts) return fail(kUnsupported, "attn_merge_lse: n_parts %d > %d", n_parts, kMaxParts);
    if (!dtype_known(out_dt)) return fail(kInvalid, "attn_merge_lse: unknown dtype %d", out_dt);
    if (num_heads < 1) return fail(kInvalid, "attn_merge_lse: num_heads %d < 1", num_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(kUnsupported, "attn_merge_lse: head_dim %d not supported", head_dim);
    if (sq < 0) return fail(kInvalid, "attn_merge_lse: sq %lld < 0", (long long)sq);
    if (sq > kMaxTokens) return fail(kUnsupported, "attn_merge_lse: sq above %lld", (long long)kMaxTokens);
    if (sq == 0) return ok();
    if (!o_parts || !lse_parts || !o_out) return fail(kInvalid, "attn_merge_lse: NULL input or output");
    if (!aligned(o_parts, 16) || !aligned(lse_parts, 4) || !aligned(o_out, out_dt == kF16 ? 8 : 16) ||
        (lse_out && !aligned(lse_out, 4)))
        return fail(kInvalid, "attn_merge_lse: misaligned pointer");
    return ok();
}

}  // namespace attnblk
