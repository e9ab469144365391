// The Muon step on a workspace the library holds itself, for callers that
// cannot allocate device memory (declared in include/muon.h as
// muon_momentum_ns5_batched_static).
//
// The workspace is `scratch`, a file-scope device array of
// MUON_STATIC_WORKSPACE_BYTES.  Each GPU holds its own copy from the moment
// the library's code is loaded on it until the process ends.  In host code
// the name `scratch` is only a host-side stand-in, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and that address is what the kernels receive.
//
// Nothing in the workspace has to start at zero: every region a call reads
// (the iterates, their zero padding, A, B, the norm partials) is written
// earlier in the same call, so the contents a previous call left behind do
// not matter.  Calls that overlap in time on one GPU share the array and
// race; the header states it.
#include <atomic>
#include <mutex>

#include "../../include/muon.h"
#include "internal.hpp"

namespace muon {

namespace {

static __device__ __align__(256) unsigned char scratch[MUON_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's `scratch`, looked up on the first call
// on the device.  Returns 0 or a MUON status (with the message set).
int scratch_of_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail_status(MUON_ERR_HIP, "hipGetDevice failed: no current device");
    }
    if (dev < 0 || dev >= kMaxDevices) return fail_status(MUON_ERR_UNSUPPORTED, "device index beyond 63");
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                (void)hipGetLastError();
                return fail_status(MUON_ERR_HIP, "hipGetSymbolAddress of the static workspace failed");
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return MUON_OK;
}

}  // namespace

}  // namespace muon

extern "C" int muon_momentum_ns5_batched_static(const float* const* g, float* const* buf, float* const* out,
                                                const int64_t* rows, const int64_t* cols, int64_t count, float mu,
                                                int steps, float eps, void* stream) {
    using namespace muon;
    return run_momentum_ns5_fixed_workspace(g, buf, out, rows, cols, count, mu, steps, eps,
                                            MUON_STATIC_WORKSPACE_BYTES, scratch_of_current_device,
                                            static_cast<hipStream_t>(stream));
}
