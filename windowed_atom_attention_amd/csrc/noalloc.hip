// noalloc.hip -- atom_attn_block_noalloc: the block call with its scratch
// memory in a static per-device array instead of a caller workspace, for
// callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc). Same kernels, same checks and the same
// results as atom_attn_encoder / atom_attn_decoder.
//
// The array below is a device global: every GPU the library runs on holds
// its own copy (kStaticScratchBytes) from the first call on that device
// until the process ends. In host code its name is only a handle, not a
// device address; the address is taken once per device with
// hipGetSymbolAddress and that pointer is what the kernels receive.
#include <atomic>
#include <mutex>

#include "../../include/atom_attn.h"
#include "kernels.hpp"

namespace waa {
int block_call(const atom_attn_dims *d, int style, int stage, int dtype,
               const atom_attn_inputs *in, const atom_attn_params *par, double eps,
               int64_t radius, atom_attn_outputs *out, void *workspace,
               size_t ws_bytes, void *stream);
int block_workspace_bytes(const atom_attn_dims *d, int style, int stage, int dtype,
                          size_t *bytes);
} // namespace waa

namespace {

constexpr size_t kStaticScratchBytes = (size_t)64 << 20;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (looked up on the first
// call on the device, with that device current); nullptr on failure.
void *scratch_ptr(int dev) {
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr)
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

} // namespace

extern "C" {

size_t atom_attn_noalloc_max_bytes(void) { return kStaticScratchBytes; }

int atom_attn_block_noalloc(const atom_attn_dims *dims, int style, int stage, int dtype,
                            const atom_attn_inputs *in, const atom_attn_params *par,
                            double eps, int64_t radius, atom_attn_outputs *out,
                            void *stream) {
    size_t need = 0;
    int rc = waa::block_workspace_bytes(dims, style, stage, dtype, &need);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (need > kStaticScratchBytes)
        return ATOM_ATTN_ESCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ATOM_ATTN_ELAUNCH;
    void *ws = scratch_ptr(dev);
    if (ws == nullptr)
        return ATOM_ATTN_ELAUNCH;
    return waa::block_call(dims, style, stage, dtype, in, par, eps, radius, out, ws,
                           kStaticScratchBytes, stream);
}

} // extern "C"
