// Data-movement kernels. (1) Receive-side layouts of the two all-to-alls of
// Ulysses context parallelism
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
// (2) A batched per-head transpose, which turns a caller's row-major V
// [H][keys][d] into the keys-contiguous V^T the attention kernel reads, and
// back for the V tap of the block.

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

// Batched transpose, one E x E block (E = 16 bytes / element) per thread:
// E row loads of 16 bytes, a register transpose, E column stores of 16 bytes.
// A wave covers 8 x 8 blocks: lane % 8 steps the column block and lane / 8
// the row block, so every load instruction reads 128 contiguous bytes of 8
// source rows and every store writes 128 contiguous bytes of 8 destination
// rows (whole lines both ways; no LDS needed).
struct TransposeArgs {
    const char *src;
    char *dst;
    int64_t src_hs, src_rs, dst_hs, dst_rs;  // elements
    int64_t rows, rows_out, cols;
    uint32_t row_tiles, col_tiles, waves;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_heads(TransposeArgs a) {
    constexpr int E = 16 / sizeof(T);
    typedef T vecE __attribute__((ext_vector_type(E)));
    const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wave >= a.waves) return;
    const int lane = threadIdx.x & 63;
    const uint32_t ct = wave % a.col_tiles;
    const uint32_t rt = (wave / a.col_tiles) % a.row_tiles;
    const uint32_t b = wave / (a.col_tiles * a.row_tiles);
    const int64_t r0 = (int64_t)rt * 8 * E + (lane >> 3) * E;
    const int64_t c0 = (int64_t)ct * 8 * E + (lane & 7) * E;
    const T *src = reinterpret_cast<const T *>(a.src) + b * a.src_hs;
    T *dst = reinterpret_cast<T *>(a.dst) + b * a.dst_hs;
    vecE in[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (r0 + j < a.rows && c0 < a.cols)
            in[j] = *reinterpret_cast<const vecE *>(src + (r0 + j) * a.src_rs + c0);
        else
            in[j] = vecE{};
    }
    if (r0 >= a.rows_out) return;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        vecE out;
#pragma unroll
        for (int j = 0; j < E; ++j) out[j] = in[j][i];
        if (c0 + i < a.cols) *reinterpret_cast<vecE *>(dst + (c0 + i) * a.dst_rs + r0) = out;
    }
}

}  // namespace

hipError_t launch_transpose_heads(const void *src, int64_t src_hs, int64_t src_rs, void *dst, int64_t dst_hs,
                                  int64_t dst_rs, int heads, int64_t rows, int64_t rows_out, int64_t cols,
                                  int elem_bytes, hipStream_t stream) {
    if (heads <= 0 || rows_out <= 0 || cols <= 0) return hipSuccess;
    const int E = 16 / elem_bytes;
    if ((elem_bytes != 2 && elem_bytes != 4) || rows_out % E != 0 || rows_out < rows) return hipErrorInvalidValue;
    TransposeArgs a{};
    a.src = static_cast<const char *>(src);
    a.dst = static_cast<char *>(dst);
    a.src_hs = src_hs;
    a.src_rs = src_rs;
    a.dst_hs = dst_hs;
    a.dst_rs = dst_rs;
    a.rows = rows;
    a.rows_out = rows_out;
    a.cols = cols;
    const int64_t rt = (rows_out + 8 * E - 1) / (8 * E), ct = (cols + 8 * E - 1) / (8 * E);
    const int64_t waves = rt * ct * heads;
    if (waves >= 0x80000000ll) return hipErrorInvalidConfiguration;
    a.row_tiles = (uint32_t)rt;
    a.col_tiles = (uint32_t)ct;
    a.waves = (uint32_t)waves;
    const unsigned blocks = (unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64));
    if (elem_bytes == 2)
        hipLaunchKernelGGL(transpose_heads<half_t>, dim3(blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(transpose_heads<float>, dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

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
