// gdr2_noalloc.hip -- gdr2_forward_chunked_noalloc: the chunked forward with
// its workspace taken from a static device array of the library instead of
// the caller, for callers that cannot allocate device memory (code under
// stream capture, tight serving loops, hosts that forbid allocation).
//
// The array is `scratch` below, GDR2_NOALLOC_SCRATCH_BYTES bytes, one copy
// per device, held until the process ends.  In host code its name is only a
// host-side stand-in: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever passed to a kernel.  Calls on one device share the array, so calls
// that overlap in time on one device race; nothing in it needs to start at
// zero (every kernel writes what it later reads).
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr2.h"
#include "gdr2_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDR2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first
// call per device).  Returns hipSuccess and sets *out, or the HIP error.
hipError_t scratch_of_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" gdr2_status gdr2_forward_chunked_noalloc(const gdr2_fwd_args* a, void* stream)
{
    // every argument check first, on the host, before the device is touched
    const gdr2_status st = gdr2::check_forward_args(a);
    if (st != GDR2_OK)
        return st;
    gdr2_fwd_args x = *a;
    x.workspace = nullptr;
    x.workspace_bytes = 0;
    const size_t need = gdr2_forward_workspace_size(&x);
    if (need > (size_t)GDR2_NOALLOC_SCRATCH_BYTES)
        return gdr2::set_error(GDR2_ERR_WORKSPACE,
                               "gdr2_forward_chunked_noalloc: these arguments need %zu bytes of workspace; the "
                               "library's static scratch holds %zu (use gdr2_forward_chunked with a caller "
                               "workspace)",
                               need, (size_t)GDR2_NOALLOC_SCRATCH_BYTES);
    if (need > 0) {
        void* p = nullptr;
        const hipError_t e = scratch_of_current_device(&p);
        if (e != hipSuccess)
            return gdr2::set_error(GDR2_ERR_HIP, "gdr2_forward_chunked_noalloc: scratch address: %s",
                                   hipGetErrorString(e));
        x.workspace = p;
        x.workspace_bytes = GDR2_NOALLOC_SCRATCH_BYTES;
    }
    return gdr2_forward_chunked(&x, stream);
}
