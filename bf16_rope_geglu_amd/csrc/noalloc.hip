// rgg_selfcheck_noalloc (include/rgg.h): the device self-check over staging
// that the library holds itself, for callers that cannot allocate device
// memory.  The staging is a file-scope device array, one copy per GPU; its
// device address is looked up once per device (hipGetSymbolAddress) with the
// device current, and only that address is handed to the HIP runtime and the
// kernels.  Host images of the staging are static too, so a call allocates
// nothing.  Calls are serialized by a process-wide lock (they share the host
// images); calls on one GPU share its array, which keeps the last call's
// contents (every call overwrites the whole staged region first).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rgg.h"
#include "selfcheck.h"

namespace {

constexpr size_t kScratchBytes = RGG_SELFCHECK_WORKSPACE_BYTES;  // 1 MiB per GPU
static_assert(rgg::kSelfcheckBytes <= kScratchBytes, "self-check staging fits the scratch array");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
hipError_t g_lookup[kMaxDevices];
uint8_t *g_scratch[kMaxDevices];  // device address of `scratch` on each GPU

std::mutex g_lock;
alignas(256) uint8_t g_host_in[rgg::kSelfcheckBytes];
alignas(256) uint8_t g_host_out[rgg::kSelfcheckBytes];

}  // namespace

int rgg::noalloc_prepare(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return RGG_ERR_SHAPE;
    std::call_once(g_once[device], [device] {
        g_lookup[device] = hipGetSymbolAddress(reinterpret_cast<void **>(&g_scratch[device]),
                                               HIP_SYMBOL(scratch));
        if (g_lookup[device] == hipSuccess && g_scratch[device] == nullptr)
            g_lookup[device] = hipErrorInvalidSymbol;
    });
    return g_lookup[device] == hipSuccess ? RGG_OK : RGG_ERR_HIP;
}

extern "C" int rgg_selfcheck_noalloc(uint32_t checks, hipStream_t stream, uint32_t *failed)
{
    if (failed)
        *failed = 0;
    if (checks == 0 || (checks & ~(uint32_t)RGG_SELFCHECK_ALL))
        return RGG_ERR_SHAPE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return RGG_ERR_HIP;
    const int st = rgg::noalloc_prepare(dev);
    if (st != RGG_OK)
        return st;
    std::lock_guard<std::mutex> hold(g_lock);
    return rgg::selfcheck_run(g_scratch[dev], stream, checks, failed, g_host_in, g_host_out);
}
