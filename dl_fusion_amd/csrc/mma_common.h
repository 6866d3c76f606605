// Pipeline helpers shared by the MFMA kernels (GEMM / implicit-GEMM and the
// halo convolution): explicit memory-counter waits, a barrier that does not
// drain LDS-DMA loads, scheduling hints and the LDS-DMA load itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlf {
namespace {

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4 left
// at its maximum, lgkmcnt 11:8).  Waiting for lgkmcnt(0) as well makes sure this wave's
// LDS reads of the previous slice are complete before the barrier that lets other waves
// overwrite it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the implied memory fence of __syncthreads() (which
// would drain every outstanding LDS-DMA load); the asm statement keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scheduling hint for one pipeline step: alternate its MF MFMAs with the R LDS
// reads of the next step's fragments and the G global->LDS loads of a future
// slice, so the matrix pipe never waits on an LDS round trip.
template <int MF, int R, int G, int W = 0>
__device__ __forceinline__ void interleave() {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        if (i < W) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
        if (i < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        if (i < G) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one VMEM load
    }
    if constexpr (W > MF) __builtin_amdgcn_sched_group_barrier(0x200, W - MF, 0);
    if constexpr (R > MF) __builtin_amdgcn_sched_group_barrier(0x100, R - MF, 0);
    if constexpr (G > MF) __builtin_amdgcn_sched_group_barrier(0x020, G - MF, 0);
}

// One 16-byte global load per lane straight into LDS: lane i's data lands at
// lds_wave_base + 16 i (the base must be uniform across the wave).
__device__ __forceinline__ void load_lds16(const void* g, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

}  // namespace
}  // namespace dlf
