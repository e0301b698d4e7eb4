// Device-side building blocks shared by the gfx950 kernels: vector types,
// 16-byte loads and stores, XCD-aware block remapping, wait-count encodings,
// the bare workgroup barrier and a cross-lane max.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace attnblk {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ half8 as_half8(const u32x4 &v) {
    return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ u32x4 ldg16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void stg16(void *p, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Work-item index for block `bid` of `nblocks` such that the blocks the
// hardware dispatches to one XCD (bid % 8 == x) get a contiguous range of
// work items, so neighbouring tiles share that XCD's L2. Identity when the
// count does not divide evenly.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    if (nblocks % kXcd != 0) return bid;
    return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

// Address spaces of the direct global->LDS load builtin's operands.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// s_waitcnt immediate that waits for vmcnt <= n and leaves expcnt and lgkmcnt
// unconstrained (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt bits 6:4,
// lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14).
constexpr int vmcnt_only(int n) { return (n & 0xF) | 0x70 | 0xF00 | ((n >> 4) << 14); }

// Workgroup barrier without the release fence of __syncthreads(): that fence
// would wait for every in-flight global->LDS load (they count as LDS stores),
// emptying a prefetch ring at each step. Visibility of a stage comes from
// each wave's explicit vmcnt wait before the barrier; the memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate that waits for vmcnt <= n and lgkmcnt == 0.
constexpr int vmcnt_lgkm0(int n) { return (n & 0xF) | 0x70 | ((n >> 4) << 14); }

// max(v of lane i, v of lane i ^ 32) in every lane. v_permlane32_swap trades
// the upper half of one register with the lower half of the other (a VALU
// operation, where __shfl_xor would go through the LDS crossbar); applied to
// two copies of v it yields, in each lane i, v[i % 32] in one result and
// v[i % 32 + 32] in the other (checked lane by lane on an MI355X).
__device__ __forceinline__ float wave_max_across_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace attnblk
