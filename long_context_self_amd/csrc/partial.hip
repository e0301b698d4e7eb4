// C ABI of the rank-share partial (attention of a query chunk against one
// K/V block, all heads): attn_partial_forward takes V row-major [H][skv][d],
// attn_partial_forward_vt takes V transposed per head. Both end in the same
// attention kernels; the row-major form first transposes V into a staging
// buffer from a library-owned stream-ordered pool, and
// attn_partial_forward_noalloc stages it in a fixed device array instead.
//
// Definition: a rank keeps its own Q slice and attends to the gathered K/V,
// or to K/V streamed in blocks whose normalised partials and LSEs are
// combined by online softmax (news summary of "Scaling AI Inference Across
// Multiple GPUs Using NVIDIA TensorRT with Multi-Device Inference Support",
// the three context-parallel implementations; "Multi-Device Attention
// Inference with TensorRT", "What is hint.json?": q_scaled stays local).

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "attn_block.h"
#include "common.hpp"
#include "kernels.hpp"
#include "status.hpp"
#include "validate.hpp"

using namespace attnblk;

namespace attnblk {

namespace {

constexpr int kMaxDevices = 64;

// One stream-ordered pool per device for the staging of the partial entry
// points. Its release threshold is unlimited, so memory freed on a stream
// stays in the pool and later calls reuse it without going back to the
// driver.
struct StagingPool {
    std::once_flag once;
    hipMemPool_t pool = nullptr;
    hipError_t err = hipSuccess;
};
StagingPool g_pools[kMaxDevices];

}  // namespace

hipError_t staging_pool(hipMemPool_t *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    StagingPool &p = g_pools[dev];
    std::call_once(p.once, [&p, dev] {
        hipMemPoolProps props{};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        p.err = hipMemPoolCreate(&p.pool, &props);
        if (p.err == hipSuccess) {
            uint64_t keep = UINT64_MAX;
            p.err = hipMemPoolSetAttribute(p.pool, hipMemPoolAttrReleaseThreshold, &keep);
        }
    });
    *out = p.pool;
    return p.err;
}

}  // namespace attnblk

namespace {

constexpr int kMaxDevices = 64;

// Attention kernels over keys given as K [H][skv][d] and V^T [H][d][vrs].
// fp16 launches follow plan_attention_f16 with the partial paths' budget; a
// split tail keeps its partials in `ws` (at least kPartialWsFloats *
// (head_dim + 1) / head_dim floats) when given, else in a block of the pool.
attn_status_t enqueue_partial(const char *what, int num_heads, int head_dim, int dt, const void *q, int64_t sq,
                              int64_t qhs, const void *k, int64_t skv, int64_t khs, const void *vt, int64_t vhs,
                              int64_t vrs, float *o_part, float *lse_part, float *ws, hipStream_t stream) {
    if (dt == kF16) {
        FlashArgs fa{};
        fa.q = static_cast<const _Float16 *>(q);
        fa.k = static_cast<const _Float16 *>(k);
        fa.vt = static_cast<const _Float16 *>(vt);
        fa.q_head_stride = qhs;
        fa.k_head_stride = khs;
        fa.v_head_stride = vhs;
        fa.v_row_stride = vrs;
        fa.sq = (int)sq;
        fa.skv = (int)skv;
        fa.num_heads = num_heads;
        fa.o32 = o_part;
        fa.lse = lse_part;
        const AttnPlan plan = plan_attention_f16(num_heads, (int)sq, (int)skv, kPartialWsFloats);
        if (plan.n_split <= 1) {
            HIP_TRY(what, launch_attention_f16(fa, plan, nullptr, nullptr, stream));
            return ATTN_OK;
        }
        void *pooled = nullptr;
        if (!ws) {
            hipMemPool_t pool = nullptr;
            HIP_TRY(what, staging_pool(&pool));
            const hipError_t e =
                hipMallocFromPoolAsync(&pooled, (size_t)(plan.o_elems + plan.lse_elems) * sizeof(float), pool, stream);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                char msg[160];
                std::snprintf(msg, sizeof(msg), "%s: split workspace allocation failed", what);
                return set_error(kOom, msg);
            }
            ws = static_cast<float *>(pooled);
        }
        const hipError_t el = launch_attention_f16(fa, plan, ws, ws + plan.o_elems, stream);
        // released in stream order after the kernels that use it
        const hipError_t ef = pooled ? hipFreeAsync(pooled, stream) : hipSuccess;
        HIP_TRY(what, el);
        HIP_TRY(what, ef);
    } else {
        FlashArgsF32 fa{};
        fa.q = static_cast<const float *>(q);
        fa.k = static_cast<const float *>(k);
        fa.vt = static_cast<const float *>(vt);
        fa.q_head_stride = qhs;
        fa.k_head_stride = khs;
        fa.v_head_stride = vhs;
        fa.v_row_stride = vrs;
        fa.sq = (int)sq;
        fa.skv = (int)skv;
        fa.num_heads = num_heads;
        fa.head_dim = head_dim;
        fa.o32 = o_part;
        fa.lse = lse_part;
        HIP_TRY(what, launch_flash_fwd_f32(fa, stream));
    }
    return ATTN_OK;
}

// Row-major V [H][skv][d] (head stride kvhs) -> V^T [H][d][ld] at vt, then the
// attention kernels.
attn_status_t enqueue_partial_rows(const char *what, int num_heads, int head_dim, int dt, const void *q, int64_t sq,
                                   int64_t qhs, const void *k, const void *v, int64_t skv, int64_t kvhs, void *vt,
                                   float *o_part, float *lse_part, float *ws, hipStream_t stream) {
    const int64_t ld = ATTN_VT_LD(skv);
    if (skv > 0)
        HIP_TRY(what, launch_transpose_heads(v, kvhs, head_dim, vt, (int64_t)head_dim * ld, ld, num_heads, skv, ld,
                                             head_dim, elem_size(dt), stream));
    return enqueue_partial(what, num_heads, head_dim, dt, q, sq, qhs, k, skv, kvhs, vt, (int64_t)head_dim * ld, ld,
                           o_part, lse_part, ws, stream);
}

// Fixed staging for attn_partial_forward_noalloc, for callers that cannot
// allocate: the V^T staging (up to kVtScratchBytes) and after it the
// partials of a key-split tail (the partial paths' budget, kPartialWsFloats
// floats of rows and one LSE per 128 of them). Each device the library runs
// on holds its own copy of this array from the time the library's code is
// loaded on it until the process ends. In host code `scratch` names a
// host-side stand-in, never device memory: the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kVtScratchBytes = size_t(64) << 20;
constexpr size_t kScratchBytes = kVtScratchBytes + (size_t)kPartialWsFloats * sizeof(float) * 129 / 128;
__device__ __align__(256) char scratch[kScratchBytes];

struct ScratchAddr {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[kMaxDevices];

// Device address of this device's `scratch` (the device must be current).
hipError_t scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchAddr &s = g_scratch[dev];
    std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    *out = s.ptr;
    return s.err;
}

}  // namespace

ATTN_API attn_status_t attn_partial_forward_noalloc(int num_heads, int head_dim, attn_dtype_t dt,
                                                    const void *q_scaled, int64_t sq, int64_t q_head_stride,
                                                    const void *k, const void *v, int64_t skv,
                                                    int64_t kv_head_stride, float *o_part, float *lse_part,
                                                    hipStream_t stream) {
    const char *what = "attn_partial_forward_noalloc";
    Check c = validate_partial_rows(what, num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k, v, skv,
                                    kv_head_stride, o_part, lse_part);
    if (c.status != kOk) return report(c);
    const size_t bytes = (size_t)num_heads * head_dim * ATTN_VT_LD(skv) * elem_size((int)dt);
    if (bytes > kVtScratchBytes) {
        char msg[256];
        std::snprintf(msg, sizeof(msg),
                      "%s: V^T staging needs %zu bytes (num_heads * head_dim * ATTN_VT_LD(skv) elements), above the "
                      "fixed %zu-byte scratch; use attn_partial_forward",
                      what, bytes, kVtScratchBytes);
        return set_error(kUnsupported, msg);
    }
    if (sq == 0) return ATTN_OK;
    void *vt = nullptr;
    HIP_TRY("attn_partial_forward_noalloc: scratch address", scratch_ptr(&vt));
    float *ws = reinterpret_cast<float *>(static_cast<char *>(vt) + kVtScratchBytes);
    return enqueue_partial_rows(what, num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k, v, skv,
                                kv_head_stride, vt, o_part, lse_part, ws, stream);
}

ATTN_API attn_status_t attn_partial_forward_vt(int num_heads, int head_dim, attn_dtype_t dt, const void *q_scaled,
                                               int64_t sq, int64_t q_head_stride, const void *k, int64_t skv,
                                               int64_t k_head_stride, const void *v_t, int64_t v_head_stride,
                                               int64_t v_row_stride, float *o_part, float *lse_part,
                                               hipStream_t stream) {
    Check c = validate_partial(num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k, skv, k_head_stride,
                               v_t, v_head_stride, v_row_stride, o_part, lse_part);
    if (c.status != kOk) return report(c);
    if (sq == 0) return ATTN_OK;
    return enqueue_partial("attn_partial_forward_vt", num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k,
                           skv, k_head_stride, v_t, v_head_stride, v_row_stride, o_part, lse_part, nullptr, stream);
}

ATTN_API attn_status_t attn_partial_forward(int num_heads, int head_dim, attn_dtype_t dt, const void *q_scaled,
                                            int64_t sq, int64_t q_head_stride, const void *k, const void *v,
                                            int64_t skv, int64_t kv_head_stride, float *o_part, float *lse_part,
                                            hipStream_t stream) {
    const char *what = "attn_partial_forward";
    Check c = validate_partial_rows(what, num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k, v, skv,
                                    kv_head_stride, o_part, lse_part);
    if (c.status != kOk) return report(c);
    if (sq == 0) return ATTN_OK;
    if (skv == 0)
        return enqueue_partial(what, num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k, 0, 0, nullptr, 0,
                               0, o_part, lse_part, nullptr, stream);
    hipMemPool_t pool = nullptr;
    HIP_TRY("attn_partial_forward: staging pool", staging_pool(&pool));
    const size_t bytes = (size_t)num_heads * head_dim * ATTN_VT_LD(skv) * elem_size((int)dt);
    void *vt = nullptr;
    hipError_t e = hipMallocFromPoolAsync(&vt, bytes, pool, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(kOom, "attn_partial_forward: V^T staging allocation failed");
    }
    const attn_status_t st = enqueue_partial_rows(what, num_heads, head_dim, (int)dt, q_scaled, sq, q_head_stride, k,
                                                  v, skv, kv_head_stride, vt, o_part, lse_part, nullptr, stream);
    // Released in stream order after the kernels (also after a failed launch,
    // which enqueued nothing that reads it).
    const hipError_t ef = hipFreeAsync(vt, stream);
    if (st != ATTN_OK) return st;
    HIP_TRY("attn_partial_forward: staging release", ef);
    return ATTN_OK;
}
