// Scratch memory of the allocation-free weight quantization: the per-column
// maxima of diag(s) W live in a file-scope device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy of the array
// (256 KB) until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so it
// is never passed to a kernel or a copy: its device address is taken once per
// device with hipGetSymbolAddress (that device current) and kept here.
#include <atomic>
#include <mutex>

#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

constexpr int64_t kScratchCols = 65536;

static __device__ __align__(256) uint32_t scratch[kScratchCols];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

int64_t noalloc_scratch_cols() { return kScratchCols; }

hipError_t noalloc_scratch(int device, void** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[device].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[device].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace sqk
