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

// s_waitcnt vmcnt(N) lgkmcnt(L): as wait_vmcnt, but up to L of this wave's newest LDS
// reads may stay in flight (LDS reads complete in issue order when no scalar loads are
// outstanding).
template <int N, int L>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64 && L >= 0 && L < 16, "counter ranges");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (L << 8));
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

// Buffer resource over [base, base + bytes) for the buffer form of the LDS-DMA load (word 3
// is the raw-buffer format of the gfx9 family: no swizzle, no stride, 32-bit offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// Offset that lies outside every buffer: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Cache-policy operand of a buffer store that writes through to device scope (sc1): the line
// goes on towards memory when stored, instead of staying dirty in the XCD's L2 until the
// release at the end of the kernel writes it back.  Worth it where every store instruction
// writes whole 128-byte lines; stores of partial lines were slower this way.
constexpr int kStoreDevice = 16;

// One 16-byte load per lane from buffer r at byte offset voff into LDS (lane i's data lands at
// lds_wave_base + 16 i; the base must be uniform across the wave).  Offsets past the buffer
// read as zero.  Unlike the global form it is not a FLAT instruction, so the compiler does not
// have to assume it may touch LDS through a generic address, and keeps counting this wave's
// outstanding LDS reads exactly while it is in flight.
__device__ __forceinline__ void load_lds16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, voff,
                                             0, 0, 0);
}

}  // namespace
}  // namespace dlf
