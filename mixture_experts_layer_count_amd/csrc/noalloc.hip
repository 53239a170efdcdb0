// moe_forward_noalloc: the whole-layer forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). It runs exactly moe_forward's kernels; the
// workspace moe_forward takes from the caller lives here instead, in a
// fixed-size array in device global memory that the code object itself
// provides on every GPU the library runs on.
#include <mutex>

#include "common.h"

namespace {

// moe_forward's workspace, at most this many bytes: every decode batch of the
// repository's layer shapes fits (the largest, the DeepSeek-V3-shaped layer
// with a bf16 shared expert at 64 tokens, needs 137 MiB). The array is
// zero-initialised .bss of the code object: no file size, but each GPU that
// loads the library holds it until the process ends.
constexpr size_t kScratchBytes = size_t(256) << 20;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` per GPU. In host code `scratch` names a
// host-side stand-in, not the device array, so kernels and copies only ever
// see these addresses, taken with hipGetSymbolAddress on each device once.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_on(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        // `dev` is the current device here (checked by the caller)
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_forward_noalloc_max_bytes(void) { return kScratchBytes; }

moe_status moe_forward_noalloc(const moe_layer_desc *desc, const void *X, int T, void *Y, hipStream_t stream,
                               float *logits_out, int32_t *topk_idx_out, float *topk_w_out,
                               int32_t *counts_out, hipEvent_t const *events) {
    if (!desc || T < 0) return MOE_ERR_INVALID_ARG;
    if (T == 0) return moe_forward(desc, X, 0, Y, nullptr, 0, stream, logits_out, topk_idx_out, topk_w_out,
                                   counts_out, events);
    // size check on the host, before the device is touched
    const size_t need = moe_forward_workspace_bytes(desc, T);
    if (need == 0) {
        // invalid or unsupported descriptor or size: moe_forward names which
        return moe_forward(desc, X, T, Y, nullptr, 0, stream, logits_out, topk_idx_out, topk_w_out, counts_out,
                           events);
    }
    if (need > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (stream) {
        hipDevice_t sdev;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_HIP;
        if ((int)sdev != dev) return MOE_ERR_INVALID_ARG;  // the stream must belong to the current device
    }
    void *ws = nullptr;
    const moe_status st = scratch_on(dev, &ws);
    if (st != MOE_OK) return st;
    return moe_forward(desc, X, T, Y, ws, kScratchBytes, stream, logits_out, topk_idx_out, topk_w_out, counts_out,
                       events);
}

}  // extern "C"
