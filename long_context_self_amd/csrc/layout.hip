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
// i*dst_si. HBM-bound: 16-byte loads and stores, four per thread in flight;
// one workgroup covers part of one segment, so the segment index is a
// per-workgroup scalar.

#include "common.hpp"
#include "kernels.hpp"

namespace attnblk {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void seg_copy(SegCopyArgs a) {
    const uint32_t seg = blockIdx.x / a.blocks_per_seg;
    const uint32_t part = blockIdx.x - seg * a.blocks_per_seg;
    const uint32_t o = seg / a.n_inner;
    const uint32_t i = seg - o * a.n_inner;
    const char *s = a.src + o * a.src_so + i * a.src_si;
    char *d = a.dst + o * a.dst_so + i * a.dst_si;
    const uint32_t c0 = part * kThreads * kUnroll + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = c0 + u * kThreads;
        if (c < a.chunks_per_seg) v[u] = ldg16(s + (int64_t)c * 16);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = c0 + u * kThreads;
        if (c < a.chunks_per_seg) stg16(d + (int64_t)c * 16, v[u]);
    }
}

}  // namespace

hipError_t launch_seg_copy(SegCopyArgs a, hipStream_t stream) {
    if (a.n_outer == 0 || a.n_inner == 0 || a.chunks_per_seg == 0) return hipSuccess;
    a.blocks_per_seg = (a.chunks_per_seg + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const uint64_t blocks = (uint64_t)a.n_outer * a.n_inner * a.blocks_per_seg;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(seg_copy, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attnblk
