// Ring-style streaming of K/V blocks on one GPU: the blocks arrive by
// asynchronous copy on a copy stream while the attention of earlier blocks
// runs on the caller's stream, and the per-block partial results are merged
// by log-sum-exp at the end. This is the pattern of Ring Attention -- K/V
// streamed around the ranks, each rank overlapping its local Q computation
// with the transfer and combining the blocks by online softmax, never
// holding the full K/V (news summary of "Scaling AI Inference Across Multiple
// GPUs Using NVIDIA TensorRT with Multi-Device Inference Support", the three
// context-parallel implementations).
//
// Schedule, for block b in slot b % 2 of a two-slot staging buffer:
//   copy stream:    [wait freed[b%2]] copy K_b, V_b -> slot; record arrived[b%2]
//   compute stream: wait arrived[b%2]; partial(Q, slot) -> (O_b, LSE_b); record freed[b%2]
// so the copy of block b+1 runs while block b's partial computes, and no copy
// overwrites a slot whose previous block is still being read. The sources
// may be device memory or pinned host memory (hipMemcpyAsync with
// hipMemcpyDefault), standing in for a peer's link.

#include <algorithm>
#include <cstring>

#include "attn_block.h"
#include "common.hpp"
#include "kernels.hpp"
#include "status.hpp"
#include "validate.hpp"

using namespace attnblk;

struct attn_ring {
    int heads, head_dim, dt, n_blocks, device;
    int64_t max_sq, max_block;
    void *slot_k[2], *slot_vt[2];  // K [H][len][d], V^T [H][d][ATTN_VT_LD(len)] of the block in the slot
    float *o_parts;                // [n_blocks][H][max_sq][d] (each block's part packed for the sq of a call)
    float *lse_parts;              // [n_blocks][H][max_sq]
    float *split_ws;               // fp16: partials of a block's split tail (plan_attention_f16), split_elems floats
    int64_t split_elems;
    hipStream_t copy;
    hipEvent_t start, arrived[2], freed[2];
};

namespace {

void free_ring(attn_ring *r) {
    if (!r) return;
    void *ptrs[] = {r->slot_k[0], r->slot_k[1], r->slot_vt[0], r->slot_vt[1], r->o_parts, r->lse_parts, r->split_ws};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
    hipEvent_t evs[] = {r->start, r->arrived[0], r->arrived[1], r->freed[0], r->freed[1]};
    for (hipEvent_t e : evs)
        if (e) (void)hipEventDestroy(e);
    if (r->copy) (void)hipStreamDestroy(r->copy);
    delete r;
}

// True when p is device memory of `device` (ordinary or managed allocations
// report other types and are copied).
bool on_device(const void *p, int device) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // e.g. unregistered host memory: not device memory
        return false;
    }
    return attr.type == hipMemoryTypeDevice && attr.device == device;
}

}  // namespace

ATTN_API attn_status_t attn_ring_create(attn_ring_t **out, int num_heads, int head_dim, attn_dtype_t dt,
                                        int n_blocks, int64_t max_sq, int64_t max_block_len) {
    Check c = validate_ring_create(out == nullptr, num_heads, head_dim, (int)dt, n_blocks, max_sq, max_block_len);
    if (c.status != kOk) {
        if (out) *out = nullptr;
        return report(c);
    }
    *out = nullptr;
    attn_ring *r = new (std::nothrow) attn_ring();
    if (!r) return set_error(kOom, "attn_ring_create: host allocation failed");
    std::memset(r, 0, sizeof(*r));
    r->heads = num_heads;
    r->head_dim = head_dim;
    r->dt = (int)dt;
    r->n_blocks = n_blocks;
    r->max_sq = max_sq;
    r->max_block = max_block_len;
    hipError_t e = hipGetDevice(&r->device);
    const size_t es = elem_size(r->dt), hd = (size_t)num_heads * head_dim;
    // the partial entry points' budget; rows plus one LSE per head_dim of them
    if (r->dt == kF16)
        r->split_elems = std::min<int64_t>(kPartialWsFloats, 16 * (int64_t)hd * max_sq) * (head_dim + 1) / head_dim;
    struct {
        void **p;
        size_t bytes;
    } allocs[] = {{&r->slot_k[0], hd * max_block_len * es},
                  {&r->slot_k[1], hd * max_block_len * es},
                  {&r->slot_vt[0], hd * ATTN_VT_LD(max_block_len) * es},
                  {&r->slot_vt[1], hd * ATTN_VT_LD(max_block_len) * es},
                  {reinterpret_cast<void **>(&r->o_parts), (size_t)n_blocks * hd * max_sq * sizeof(float)},
                  {reinterpret_cast<void **>(&r->lse_parts), (size_t)n_blocks * num_heads * max_sq * sizeof(float)},
                  {reinterpret_cast<void **>(&r->split_ws), (size_t)r->split_elems * sizeof(float)}};
    for (auto &a : allocs) {
        if (e != hipSuccess) break;
        if (a.bytes == 0) continue;
        e = hipMalloc(a.p, a.bytes);
        if (e != hipSuccess) {
            *a.p = nullptr;
            free_ring(r);
            (void)hipGetLastError();
            return set_error(kOom, "attn_ring_create: device allocation failed");
        }
    }
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&r->copy, hipStreamNonBlocking);
    hipEvent_t *evs[] = {&r->start, &r->arrived[0], &r->arrived[1], &r->freed[0], &r->freed[1]};
    for (hipEvent_t *ev : evs)
        if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (e != hipSuccess) {
        free_ring(r);
        return hip_fail("attn_ring_create", e);
    }
    *out = r;
    return ATTN_OK;
}

ATTN_API void attn_ring_destroy(attn_ring_t *ring) {
    if (!ring) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(ring->device);
    (void)hipDeviceSynchronize();
    free_ring(ring);
    (void)hipSetDevice(cur);
}

ATTN_API attn_status_t attn_ring_forward(attn_ring_t *ring, const void *q_scaled, int64_t sq,
                                         const void *const *k_blocks, const void *const *vt_blocks,
                                         const int64_t *block_lens, void *o_out, float *lse_out,
                                         hipStream_t stream) {
    Check c = validate_ring_forward(ring == nullptr, ring ? ring->n_blocks : 0, ring ? ring->max_sq : 0,
                                    ring ? ring->max_block : 0, q_scaled, sq, k_blocks, vt_blocks, block_lens,
                                    o_out, lse_out);
    if (c.status != kOk) return report(c);
    if (sq == 0) return ATTN_OK;
    const int H = ring->heads, d = ring->head_dim, nb = ring->n_blocks;
    const size_t es = elem_size(ring->dt);
    MergeArgs m{};
    m.n_parts = nb;
    m.num_heads = H;
    m.head_dim = d;
    m.sq = sq;
    m.o_parts = ring->o_parts;
    m.lse_parts = ring->lse_parts;
    m.o_out = o_out;
    m.out_f16 = ring->dt == kF16;
    m.lse_out = lse_out;
    // Every block already in this device's memory: one launch computes all the
    // blocks' partials as workgroups over (block, head, query rows). The 8
    // blocks of a rank share then fill whole rounds of the CUs, where 8 launches
    // of one block each leave part of a round idle.
    bool all_resident = ring->dt == kF16 && nb <= kMaxKvBlocks;
    for (int b = 0; b < nb && all_resident; ++b)
        all_resident = block_lens[b] == 0 || (on_device(k_blocks[b], ring->device) &&
                                              on_device(vt_blocks[b], ring->device));
    // Equal blocks of a power-of-two length: they are one key sequence, so the
    // launch is an ordinary planned attention over all nb * len keys with no
    // per-block partials and no merge of them.
    int lg = 0;
    bool equal_pow2 = all_resident && block_lens[0] >= 64 && (block_lens[0] & (block_lens[0] - 1)) == 0;
    for (int b = 1; b < nb && equal_pow2; ++b) equal_pow2 = block_lens[b] == block_lens[0];
    if (equal_pow2) {
        while ((int64_t(1) << lg) < block_lens[0]) ++lg;
        const int64_t len = block_lens[0], ld = ATTN_VT_LD(len);
        FlashArgs fa{};
        fa.q = static_cast<const _Float16 *>(q_scaled);
        fa.q_head_stride = sq * d;
        fa.sq = (int)sq;
        fa.skv = (int)(nb * len);
        fa.num_heads = H;
        fa.o16 = static_cast<_Float16 *>(o_out);
        fa.o16_ld = (int64_t)H * d;
        fa.lse = lse_out;
        fa.n_kv_blocks = nb;
        fa.kv_concat = 1;
        fa.kv_lg_len = lg;
        for (int b = 0; b < nb; ++b) {
            fa.kv_k[b] = static_cast<const _Float16 *>(k_blocks[b]);
            fa.kv_vt[b] = static_cast<const _Float16 *>(vt_blocks[b]);
            fa.kv_k_head_stride[b] = len * d;
            fa.kv_v_head_stride[b] = (int64_t)d * ld;
            fa.kv_v_row_stride[b] = ld;
            fa.kv_len[b] = (int)len;
        }
        const AttnPlan plan = plan_attention_f16(H, (int)sq, fa.skv, kPartialWsFloats);
        HIP_TRY("attn_ring_forward: attention",
                launch_attention_f16(fa, plan, ring->split_ws, ring->split_ws + plan.o_elems, stream));
        return ATTN_OK;
    }
    if (all_resident) {
        FlashArgs fa{};
        fa.q = static_cast<const _Float16 *>(q_scaled);
        fa.q_head_stride = sq * d;
        fa.sq = (int)sq;
        fa.num_heads = H;
        fa.o32 = ring->o_parts;
        fa.lse = ring->lse_parts;
        fa.n_kv_blocks = nb;
        for (int b = 0; b < nb; ++b) {
            const int64_t len = block_lens[b], ld = ATTN_VT_LD(len);
            fa.kv_k[b] = static_cast<const _Float16 *>(k_blocks[b]);
            fa.kv_vt[b] = static_cast<const _Float16 *>(vt_blocks[b]);
            fa.kv_k_head_stride[b] = len * d;
            fa.kv_v_head_stride[b] = (int64_t)d * ld;
            fa.kv_v_row_stride[b] = ld;
            fa.kv_len[b] = (int)len;
        }
        HIP_TRY("attn_ring_forward: partials", launch_flash_fwd_f16(fa, stream));
        HIP_TRY("attn_ring_forward: merge", launch_lse_merge(m, stream));
        return ATTN_OK;
    }
    // copies of this call start after the work already on `stream` (q, the caller's
    // buffers, and an earlier call's use of the slots)
    HIP_TRY("attn_ring_forward: hipEventRecord", hipEventRecord(ring->start, stream));
    HIP_TRY("attn_ring_forward: hipStreamWaitEvent", hipStreamWaitEvent(ring->copy, ring->start, 0));
    for (int b = 0; b < nb; ++b) {
        const int slot = b & 1;
        const int64_t len = block_lens[b];
        const int64_t ld = ATTN_VT_LD(len);
        // A block already in this device's memory is read where it is; any other
        // block (pinned host memory, a peer's memory) is copied into a slot.
        const bool in_place = len > 0 && on_device(k_blocks[b], ring->device) && on_device(vt_blocks[b], ring->device);
        const void *kb = in_place ? k_blocks[b] : ring->slot_k[slot];
        const void *vb = in_place ? vt_blocks[b] : ring->slot_vt[slot];
        if (!in_place) {
            if (b >= 2)
                HIP_TRY("attn_ring_forward: hipStreamWaitEvent", hipStreamWaitEvent(ring->copy, ring->freed[slot], 0));
            if (len > 0) {
                HIP_TRY("attn_ring_forward: K copy", hipMemcpyAsync(ring->slot_k[slot], k_blocks[b],
                                                                    (size_t)H * len * d * es, hipMemcpyDefault,
                                                                    ring->copy));
                HIP_TRY("attn_ring_forward: V copy", hipMemcpyAsync(ring->slot_vt[slot], vt_blocks[b],
                                                                    (size_t)H * d * ld * es, hipMemcpyDefault,
                                                                    ring->copy));
            }
            HIP_TRY("attn_ring_forward: hipEventRecord", hipEventRecord(ring->arrived[slot], ring->copy));
            HIP_TRY("attn_ring_forward: hipStreamWaitEvent", hipStreamWaitEvent(stream, ring->arrived[slot], 0));
        }
        float *ob = ring->o_parts + (size_t)b * H * sq * d;
        float *lb = ring->lse_parts + (size_t)b * H * sq;
        if (ring->dt == kF16) {
            FlashArgs fa{};
            fa.q = static_cast<const _Float16 *>(q_scaled);
            fa.k = static_cast<const _Float16 *>(kb);
            fa.vt = static_cast<const _Float16 *>(vb);
            fa.q_head_stride = sq * d;
            fa.k_head_stride = len * d;
            fa.v_head_stride = (int64_t)d * ld;
            fa.v_row_stride = ld;
            fa.sq = (int)sq;
            fa.skv = (int)len;
            fa.num_heads = H;
            fa.o32 = ob;
            fa.lse = lb;
            // the plan of attn_partial_forward_vt for the same shape, so the
            // ring equals partials + merge bit for bit
            const AttnPlan plan = plan_attention_f16(H, (int)sq, (int)len, kPartialWsFloats);
            HIP_TRY("attn_ring_forward: partial",
                    launch_attention_f16(fa, plan, ring->split_ws, ring->split_ws + plan.o_elems, stream));
        } else {
            FlashArgsF32 fa{};
            fa.q = static_cast<const float *>(q_scaled);
            fa.k = static_cast<const float *>(kb);
            fa.vt = static_cast<const float *>(vb);
            fa.q_head_stride = sq * d;
            fa.k_head_stride = len * d;
            fa.v_head_stride = (int64_t)d * ld;
            fa.v_row_stride = ld;
            fa.sq = (int)sq;
            fa.skv = (int)len;
            fa.num_heads = H;
            fa.head_dim = d;
            fa.o32 = ob;
            fa.lse = lb;
            HIP_TRY("attn_ring_forward: partial", launch_flash_fwd_f32(fa, stream));
        }
        HIP_TRY("attn_ring_forward: hipEventRecord", hipEventRecord(ring->freed[slot], stream));
    }
    HIP_TRY("attn_ring_forward: merge", launch_lse_merge(m, stream));
    return ATTN_OK;
}
