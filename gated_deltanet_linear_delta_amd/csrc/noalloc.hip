// gdn_chunk_fwd_noalloc: gdn_chunk_fwd with its workspace in a fixed device array of the library
// instead of caller memory, for callers that cannot allocate device memory (code under stream
// capture, tight serving loops, harnesses that forbid allocation).  See include/gdn.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

namespace {

// The workspace of every gdn_chunk_fwd_noalloc call on a device.  Each device holds its own copy
// (at its own address) from the time the library's code is loaded on it until the process ends.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The device address of `scratch` on `dev`, looked up once per device with that device current.
// In host code the array's name is only a host-side stand-in, never a device address.
gdn_status_t scratch_on(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_NO_DEVICE;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return GDN_ERR_NO_DEVICE;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return GDN_ERR_LAUNCH;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" gdn_status_t gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                              const float* beta, const float* initial_state, float* final_state,
                                              void* o, int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                              gdn_dtype_t dtype, float scale, void* stream)
{
    // sizes the library does not take give 0 here; gdn_chunk_fwd reports them below
    const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need && B > 0 && T > 0) {
        int n = 0;
        if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return GDN_ERR_NO_DEVICE;
        // the device the work runs on: the stream's, or the current one for the null stream
        int dev = -1;
        if (stream) {
            hipDevice_t d = -1;
            if (hipStreamGetDevice((hipStream_t)stream, &d) != hipSuccess) return GDN_ERR_NO_DEVICE;
            dev = (int)d;
        } else if (hipGetDevice(&dev) != hipSuccess) {
            return GDN_ERR_NO_DEVICE;
        }
        const gdn_status_t s = scratch_on(dev, &ws);
        if (s != GDN_OK) return s;
    }
    return gdn_chunk_fwd(q, k, v, g, beta, initial_state, final_state, o, B, T, Hqk, Hv, dk, dv, chunk, dtype,
                         scale, ws, need, stream);
}
