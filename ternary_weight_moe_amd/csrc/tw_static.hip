// tw_static.hip -- the batch-1 decode with a library-owned scratch buffer instead of a caller's
// workspace, for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The buffer is a file-scope __device__ array, so each device the library runs on holds its own
// copy for the life of the process.  In host code the array's name is only a host-side stand-in;
// its device address is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is passed to kernels.  Every call on one device shares that
// device's copy: calls that overlap on one device race on it (keep these calls on one stream per
// device).  The decode kernels clear what must start at zero (their hand-off words, counters and
// health word) at the start of every call, so whatever the last call left there does not matter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tw_internal.h"

namespace tw {
namespace {

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    int status = 0;
};
constexpr int kMaxDevices = 64;
DeviceScratch g_scratch[kMaxDevices];

// The device address of the current device's copy of `scratch` (looked up on the first call on
// that device); returns 0 or a hipError_t value.
int current_scratch(void **out)
{
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return int(e);
    if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.status = int(r);
        d.ptr = r == hipSuccess ? p : nullptr;
    });
    *out = d.ptr;
    return d.ptr ? 0 : (d.status ? d.status : int(hipErrorInvalidSymbol));
}

__global__ void k_copy_health(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst)
{
    if (threadIdx.x == 0) dst[0] = src[0];
}

}  // namespace

int launch_decode_static(const Dims &dm, const LayerPtrs *layers, int n_layers, const void *x_in,
                         void *x_out, int io_bf16, uint32_t *health, void *stream)
{
    void *ws = nullptr;
    const int r = current_scratch(&ws);
    if (r != 0) return r;
    const int d = launch_decode(dm, layers, n_layers, x_in, x_out, io_bf16, ws, stream);
    if (d != 0) return d;
    if (health)
        k_copy_health<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(
            reinterpret_cast<const uint32_t *>(static_cast<uint8_t *>(ws) + decode_ws_layout(dm).err),
            health);
    return int(hipGetLastError());
}

}  // namespace tw
