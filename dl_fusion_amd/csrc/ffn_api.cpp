// C ABI of the fused feed-forward block: the load-time weight packing (host) and the one-
// kernel FC1 -> activation -> FC2 launch.  Every check happens before the first HIP call.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/dlfusion.h"
#include "device_common.h"
#include "kernels.h"
#include "status.h"

namespace {

using dlf::fail;
using dlf::ok;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

extern "C" dlf_status dlf_ffn_pack(int64_t rows, int64_t k, const uint16_t* w, uint16_t* packed) {
    if (rows < 0 || k < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (rows % 32 != 0 || k % 16 != 0)
        return fail(DLF_ERR_INVALID_ARG, "rows must be a multiple of 32 and k of 16");
    if (rows == 0 || k == 0) return ok();
    if (!w || !packed) return fail(DLF_ERR_INVALID_ARG, "w and packed must be non-NULL");
    if (overlaps(w, static_cast<size_t>(rows * k) * 2, packed, static_cast<size_t>(rows * k) * 2))
        return fail(DLF_ERR_ALIAS, "packed overlaps w");
    const int64_t ks = k / 16;
    for (int64_t rb = 0; rb < rows / 32; ++rb)
        for (int64_t s = 0; s < ks; ++s)
            for (int lane = 0; lane < 64; ++lane) {
                const uint16_t* src = w + (32 * rb + lane % 32) * k + 16 * s + 8 * (lane / 32);
                std::memcpy(packed + ((rb * ks + s) * 64 + lane) * 8, src, 16);
            }
    return ok();
}

namespace {

// the descriptor's checks; fills the sizes and the activation code
dlf_status check_ffn_desc(const dlf_ffn_desc* d, dlf::FfnArgs* a, int* act) {
    if (!d) return fail(DLF_ERR_INVALID_ARG, "ffn descriptor is NULL");
    if (d->m < 0 || d->d_model < 0 || d->d_ff < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (d->act != DLF_ACT_NONE && d->act != DLF_ACT_RELU && d->act != DLF_ACT_GELU_TANH &&
        d->act != DLF_ACT_GELU_ERF)
        return fail(DLF_ERR_INVALID_ARG, "unknown activation %d", static_cast<int>(d->act));
    if (d->dtype != DLF_BF16) {
        if (d->dtype != DLF_F32 && d->dtype != DLF_FP8_E4M3) return fail(DLF_ERR_INVALID_ARG, "unknown dtype");
        return fail(DLF_ERR_UNSUPPORTED, "the fused feed-forward block is bf16 only");
    }
    if (d->d_model != 256 && d->d_model != 512 && d->d_model != 768 && d->d_model != 1024)
        return fail(DLF_ERR_UNSUPPORTED, "d_model must be 256, 512, 768 or 1024 (got %lld)",
                    static_cast<long long>(d->d_model));
    if (d->d_ff <= 0 || d->d_ff % 256 != 0 || d->d_ff > (int64_t(1) << 24))
        return fail(DLF_ERR_UNSUPPORTED, "d_ff must be a positive multiple of 256 below 2^24");
    if (d->m > (int64_t(1) << 36)) return fail(DLF_ERR_UNSUPPORTED, "too many tokens");
    *a = dlf::FfnArgs{};
    a->M = d->m;
    a->D = static_cast<int>(d->d_model);
    a->F = static_cast<int>(d->d_ff);
    a->parts = 1;
    *act = d->act == DLF_ACT_RELU ? dlf::kActRelu
         : d->act == DLF_ACT_GELU_TANH ? dlf::kActGelu
         : d->act == DLF_ACT_GELU_ERF ? dlf::kActGeluErf : dlf::kActNone;
    return ok();
}

// every check of the fused block's arguments, before any HIP call; fills a
dlf_status check_ffn(const dlf_ffn_desc* d, const void* x, const void* w1_packed, const float* b1,
                     const void* w2_packed, const float* b2, const void* residual, void* y, dlf::FfnArgs* a,
                     int* act) {
    const dlf_status st = check_ffn_desc(d, a, act);
    if (st != DLF_OK || d->m == 0) return st;
    if (!x || !w1_packed || !w2_packed || !y) return fail(DLF_ERR_INVALID_ARG, "x, weights and y must be non-NULL");
    if (!aligned16(x) || !aligned16(w1_packed) || !aligned16(w2_packed) || !aligned16(y) ||
        (b1 && !aligned16(b1)) || (b2 && !aligned16(b2)) || (residual && !aligned16(residual)))
        return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t act_bytes = static_cast<size_t>(d->m * d->d_model) * 2;
    const size_t w_bytes = static_cast<size_t>(d->d_ff * d->d_model) * 2;
    if (overlaps(y, act_bytes, x, act_bytes) || overlaps(y, act_bytes, w1_packed, w_bytes) ||
        overlaps(y, act_bytes, w2_packed, w_bytes) || overlaps(y, act_bytes, b1, static_cast<size_t>(d->d_ff) * 4) ||
        overlaps(y, act_bytes, b2, static_cast<size_t>(d->d_model) * 4) || overlaps(y, act_bytes, residual, act_bytes))
        return fail(DLF_ERR_ALIAS, "output overlaps an input");
    a->x = static_cast<const uint16_t*>(x);
    a->w1p = static_cast<const uint16_t*>(w1_packed);
    a->b1 = b1;
    a->w2p = static_cast<const uint16_t*>(w2_packed);
    a->b2 = b2;
    a->res = static_cast<const uint16_t*>(residual);
    a->y = static_cast<uint16_t*>(y);
    return ok();
}

// parts of the d_ff split, and the bytes of their partial sums (0 where the block does not split)
int ffn_split(const dlf_ffn_desc* d) {
    return dlf::ffn_parts(d->m, static_cast<int>(d->d_model), static_cast<int>(d->d_ff));
}
size_t ffn_ws_bytes(const dlf_ffn_desc* d) {
    const int parts = ffn_split(d);
    return parts > 1 ? static_cast<size_t>(parts * d->m * d->d_model) * 4 : 0;
}

}  // namespace

extern "C" dlf_status dlf_ffn_fused(const dlf_ffn_desc* d, const void* x, const void* w1_packed,
                                    const float* b1, const void* w2_packed, const float* b2,
                                    const void* residual, void* y, void* stream) {
    dlf::FfnArgs a;
    int act = 0;
    const dlf_status st = check_ffn(d, x, w1_packed, b1, w2_packed, b2, residual, y, &a, &act);
    if (st != DLF_OK || d->m == 0) return st;
    const hipError_t e = dlf::launch_ffn(a, act, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DLF_ERR_HIP, "dlf_ffn_fused: %s", hipGetErrorString(e));
    return ok();
}

extern "C" dlf_status dlf_ffn_workspace_bytes(const dlf_ffn_desc* d, size_t* bytes) {
    if (!bytes) return fail(DLF_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    dlf::FfnArgs a;
    int act = 0;
    const dlf_status st = check_ffn_desc(d, &a, &act);
    if (st != DLF_OK) return st;
    *bytes = ffn_ws_bytes(d);
    return ok();
}

extern "C" dlf_status dlf_ffn_fused_ws(const dlf_ffn_desc* d, const void* x, const void* w1_packed,
                                       const float* b1, const void* w2_packed, const float* b2,
                                       const void* residual, void* y, void* workspace, size_t workspace_bytes,
                                       void* stream) {
    dlf::FfnArgs a;
    int act = 0;
    const dlf_status st = check_ffn(d, x, w1_packed, b1, w2_packed, b2, residual, y, &a, &act);
    if (st != DLF_OK || d->m == 0) return st;
    const size_t need = ffn_ws_bytes(d);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(DLF_ERR_INVALID_ARG, "workspace of %zu bytes needed (dlf_ffn_workspace_bytes), got %zu",
                        need, workspace ? workspace_bytes : size_t(0));
        if (!aligned16(workspace)) return fail(DLF_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        const size_t act_bytes = static_cast<size_t>(d->m * d->d_model) * 2;
        const size_t w_bytes = static_cast<size_t>(d->d_ff * d->d_model) * 2;
        if (overlaps(workspace, need, x, act_bytes) || overlaps(workspace, need, y, act_bytes) ||
            overlaps(workspace, need, residual, act_bytes) || overlaps(workspace, need, w1_packed, w_bytes) ||
            overlaps(workspace, need, w2_packed, w_bytes) ||
            overlaps(workspace, need, b1, static_cast<size_t>(d->d_ff) * 4) ||
            overlaps(workspace, need, b2, static_cast<size_t>(d->d_model) * 4))
            return fail(DLF_ERR_ALIAS, "workspace overlaps an operand");
        a.parts = ffn_split(d);
        a.ws = static_cast<float*>(workspace);
    }
    const hipError_t e = dlf::launch_ffn(a, act, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DLF_ERR_HIP, "dlf_ffn_fused_ws: %s", hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------------------------
// No-allocation form: the d_ff split's fp32 partial sums go to a static device array instead of
// a caller's workspace.  Each device the library runs on holds its own copy of the array until
// the process ends; its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[DLF_FFN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of scratch on each device, once looked up

dlf_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DLF_ERR_HIP, "dlf_ffn_fused_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DLF_ERR_UNSUPPORTED, "dlf_ffn_fused_noalloc: device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(DLF_ERR_HIP, "dlf_ffn_fused_noalloc: hipGetSymbolAddress(scratch): %s",
                        e != hipSuccess ? hipGetErrorString(e) : "null address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

extern "C" dlf_status dlf_ffn_fused_noalloc(const dlf_ffn_desc* d, const void* x, const void* w1_packed,
                                            const float* b1, const void* w2_packed, const float* b2,
                                            const void* residual, void* y, void* stream) {
    dlf::FfnArgs a;
    int act = 0;
    const dlf_status st = check_ffn(d, x, w1_packed, b1, w2_packed, b2, residual, y, &a, &act);
    if (st != DLF_OK || d->m == 0) return st;
    const size_t need = ffn_ws_bytes(d);
    if (need > DLF_FFN_NOALLOC_SCRATCH_BYTES)
        return fail(DLF_ERR_INVALID_ARG,
                    "dlf_ffn_fused_noalloc: the d_ff split needs %zu bytes of scratch, the static scratch holds %zu "
                    "(dlf_ffn_fused_ws takes a workspace of any size)",
                    need, static_cast<size_t>(DLF_FFN_NOALLOC_SCRATCH_BYTES));
    if (need > 0) {
        void* ptr = nullptr;
        const dlf_status sst = scratch_on_current_device(&ptr);
        if (sst != DLF_OK) return sst;
        // every partial sum is written before it is read: nothing needs clearing between calls
        a.parts = ffn_split(d);
        a.ws = static_cast<float*>(ptr);
    }
    const hipError_t e = dlf::launch_ffn(a, act, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DLF_ERR_HIP, "dlf_ffn_fused_noalloc: %s", hipGetErrorString(e));
    return ok();
}
