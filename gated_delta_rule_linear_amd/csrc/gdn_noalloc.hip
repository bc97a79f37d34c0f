// gdn_prefill_noalloc: gdn_prefill with its scratch (the time split's segment
// maps and table) in a fixed device array instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable of GDN_NOALLOC_SCRATCH_BYTES.
// In host code its name is only a host-side stand-in, never a device address:
// the device address is looked up once per device with hipGetSymbolAddress (on
// the first call with that device current) and kept per device, and only that
// address reaches the kernels.  Every call on a GPU shares that GPU's array and
// finds there whatever the last call left; the kernels write every byte they
// later read (the segment table, then the maps, then the folded start states),
// so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_on_current_device(void** out) {
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int32_t gdn_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                                       const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                                       int64_t T_total, const float* initial_state, float* final_state, void* o,
                                       int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void* stream) {
    if (num_seqs < 0 || T_total < 0 || H < 1) return GDN_ERR_INVALID_ARG;
    // the same plan, and so the same scratch size, as gdn_prefill's (arguments only)
    const size_t need = gdn_prefill_workspace_bytes(T_total, num_seqs, H, d_k, d_v);
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0 && scratch_on_current_device(&ws) != hipSuccess) return GDN_ERR_HIP;
    return gdn_prefill(q, k, v, g, beta, cu_seqlens, num_seqs, T_total, initial_state, final_state, o, H, d_k, d_v,
                       dtype, ws, need > 0 ? (size_t)GDN_NOALLOC_SCRATCH_BYTES : 0, stream);
}
