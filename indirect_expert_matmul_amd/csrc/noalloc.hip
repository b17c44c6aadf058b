// moe_ffn_fused_noalloc: the fused MoE FFN for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It runs the
// same kernels as moe_ffn_fused with the workspace taken from a fixed device array the
// library owns, instead of one the caller passes.
//
// The array lives in the library's code object: every device the library runs on holds
// its own copy, allocated when the code object is loaded there and kept until the
// process ends. Host code never uses the array's name as an address (on the host it is
// only a stand-in); the device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept per device.
#include <cstdio>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // MOE_NOALLOC_SCRATCH_BYTES in moe.h
static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "moe.h states the scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[moe::kMaxDevices];   // device address of scratch, per device (null: not yet)

// Device address of this device's scratch array, looked up on the first call on the
// device. Returns nullptr (and sets *err) if the lookup fails.
void* scratch_ptr(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= moe::kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        if (!p) {
            *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_ffn_fused_noalloc(const moe_weights* gate, const moe_weights* up,
                                            const moe_weights* down, const moe_weights* sh_gate,
                                            const moe_weights* sh_up, const moe_weights* sh_down,
                                            const void* x, moe_dtype x_type, const int32_t* ids,
                                            const float* route_w, int64_t n_tokens, int32_t n_used,
                                            float* out, const moe_options* opt, void* stream) {
    // the workspace this call needs (0 for invalid arguments, which moe_ffn_fused then
    // reports with its own status and message)
    const size_t need = moe_ffn_fused_workspace_size(gate, sh_gate, x_type, n_tokens, n_used, opt);
    if (need > kScratchBytes) {
        // validate everything else first (a zero-byte workspace makes moe_ffn_fused stop at
        // the size check, before enqueueing anything), then report the limit
        const moe_status s = moe_ffn_fused(gate, up, down, sh_gate, sh_up, sh_down, x, x_type, ids,
                                           route_w, n_tokens, n_used, out, opt, nullptr, 0, stream);
        if (s != MOE_EWORKSPACE) return s;
        char msg[160];
        snprintf(msg, sizeof msg, "this call needs %zu bytes of scratch; the library holds %zu per device",
                 need, kScratchBytes);
        moe::set_last_error(msg);
        return MOE_ELIMIT;
    }
    hipError_t e = hipSuccess;
    void* ws = scratch_ptr(&e);
    if (!ws) {
        char msg[160];
        snprintf(msg, sizeof msg, "scratch address lookup: %s", hipGetErrorString(e));
        moe::set_last_error(msg);
        return MOE_EHIP;
    }
    return moe_ffn_fused(gate, up, down, sh_gate, sh_up, sh_down, x, x_type, ids, route_w, n_tokens,
                         n_used, out, opt, ws, kScratchBytes, stream);
}
