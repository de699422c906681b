// noalloc.hip -- ft_moe_ffn_noalloc: the grouped expert FFN with its
// workspace in a static device array, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops or harnesses
// that forbid hipMalloc).
//
// The FFN's workspace holds h (the SwiGLU activations between the two
// projections) and the M-tile list of the matrix-core path.  Here it is the
// file-scope array `scratch`, which the HIP runtime places on every GPU the
// library is loaded on and keeps until the process ends.  In host code the
// name `scratch` stands for the host-side shadow of that array, not a device
// address, so it is never passed to a kernel: the device address of each
// GPU's copy is looked up once, with that GPU current, and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"

namespace {

constexpr size_t SCRATCH_BYTES = FT_NOALLOC_SCRATCH_BYTES;
static_assert(SCRATCH_BYTES % 256 == 0, "scratch is a whole number of 256-byte units");

__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch_ptr[MAX_DEVICES];  // device address of `scratch` on each device

// Device address of the current device's copy of `scratch`; looked up on the
// first call on that device.
ft_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return ft::set_error(FT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES)
        return ft::set_error(FT_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return ft::set_error(FT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                 hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FT_OK;
}

}  // namespace

extern "C" ft_status ft_moe_ffn_noalloc(const ft_moe_weights* w, const void* x, ft_dtype act_dt, int T,
                                        int k, const int32_t* perm, const int32_t* offsets,
                                        const int32_t* slot_of_expert, void* y_perm, ft_dtype y_dt,
                                        void* stream) {
    ft::clear_error();
    FT_CHECK_ARG(w, "null weights");
    if (T == 0) return ft_moe_ffn(w, x, act_dt, T, k, perm, offsets, slot_of_expert, y_perm, y_dt,
                                  nullptr, 0, stream);
    const size_t need = ft_moe_ffn_workspace(w, T, k);
    if (need > SCRATCH_BYTES)
        return ft::set_error(FT_ERR_CAPACITY,
                             "ft_moe_ffn_noalloc: T=%d k=%d I=%d needs %zu bytes of workspace, the "
                             "static scratch holds %zu; use ft_moe_ffn with a caller workspace",
                             T, k, w->I, need, SCRATCH_BYTES);
    void* ws = nullptr;
    ft_status st = scratch_of_current_device(&ws);
    if (st != FT_OK) return st;
    return ft_moe_ffn(w, x, act_dt, T, k, perm, offsets, slot_of_expert, y_perm, y_dt, ws,
                      SCRATCH_BYTES, stream);
}
