// Receive-side layouts of the two all-to-alls of Ulysses context parallelism
// (news summary of "Scaling AI Inference Across Multiple GPUs Using NVIDIA
// TensorRT with Multi-Device Inference Support", the three context-parallel
// implementations: an all-to-all on Q, K, V gives each GPU the whole sequence
// for a subset of heads; a second all-to-all restores the head and sequence
// dimensions).
//
// Every rearrangement here is a batch of equal-length contiguous segments
// moved between two strided positions, so one kernel serves all of them:
// segment (o, i) goes from src + o*src_so + i*src_si to dst + o*dst_so +
// i*dst_si. HBM-bound: the 16-byte chunks of all segments are numbered in
// one index space that the workgroups split evenly, four chunks per thread in
// flight, so segments of any length (1 KiB rows as well as 1 MiB blocks) keep
// every thread busy; a chunk's segment comes from two multiply-shift
// divisions by launch constants.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &d) {
    return (uint32_t)(((uint64_t)n * d.m) >> (32 + d.s));
}

__global__ __launch_bounds__(kThreads) void seg_copy(SegCopyArgs a) {
    const uint32_t c0 = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    u32x4 v[kUnroll];
    const char *s[kUnroll];
    char *d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t id = c0 + u * kThreads;
        s[u] = nullptr;
        if (id < a.total_chunks) {
            const uint32_t seg = fast_div(id, a.div_cps);
            const uint32_t c = id - seg * a.chunks_per_seg;
            const uint32_t o = fast_div(seg, a.div_inner);
            const uint32_t i = seg - o * a.n_inner;
            s[u] = a.src + o * a.src_so + i * a.src_si + (int64_t)c * 16;
            d[u] = a.dst + o * a.dst_so + i * a.dst_si + (int64_t)c * 16;
            v[u] = ldg16(s[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        if (s[u]) stg16(d[u], v[u]);
}

}  // namespace

hipError_t launch_seg_copy(SegCopyArgs a, hipStream_t stream) {
    if (a.n_outer == 0 || a.n_inner == 0 || a.chunks_per_seg == 0) return hipSuccess;
    const uint64_t total = (uint64_t)a.n_outer * a.n_inner * a.chunks_per_seg;
    // chunk indices, segment indices and divisors must stay below 2^31
    if (total >= 0x80000000ull || a.chunks_per_seg >= 0x80000000u || a.n_inner >= 0x80000000u)
        return hipErrorInvalidConfiguration;
    a.total_chunks = (uint32_t)total;
    a.div_cps = make_fast_div(a.chunks_per_seg);
    a.div_inner = make_fast_div(a.n_inner);
    const uint64_t blocks = (total + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    hipLaunchKernelGGL(seg_copy, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attnblk
