// Device scratch owned by the library itself, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): mamba_selective_scan_fwd_noalloc runs the scan's
// kernels with their chunk carries in this array instead of a caller's
// workspace.
//
// The array is a file-scope device variable: every GPU that loads the library
// holds its own copy (kScratchBytes) until the process ends.  Host code never
// uses the array's name as a device address (on the host it names a shadow
// variable): the first use on a device looks up that device's copy with
// hipGetSymbolAddress, with the device current, and the pointer is kept per
// device.
//
// Every call on one GPU shares that GPU's copy and leaves its contents behind.
// Nothing in it needs to start at zero: each call writes every carry slot it
// reads before reading it.  Calls that overlap in time on one GPU (different
// streams, or host threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace mamba {

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};   // the array's address on each device, once looked up

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
    *ptr = nullptr;
    int current = 0;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    int dev = current;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        // The lookup happens with the stream's device current.
        if (dev != current && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != current) {
            const hipError_t r = hipSetDevice(current);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace mamba
