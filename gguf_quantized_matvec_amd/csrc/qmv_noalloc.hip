// Fixed activation scratch for qmv_launch_noalloc (include/qmv.h): a decode
// GEMV for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops or harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array per GPU, held from when the
// code object is loaded until the process ends.  In host code its name is a
// host-side stand-in, not a device address, so the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that pointer is ever handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/qmv.h"
#include "qmv_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QMV_NOALLOC_MAX_ACT_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_lookup_mu;                            // serialises first lookups
std::atomic<uint8_t*> g_scratch_ptr[MAX_DEVICES];  // device address per device, once found

}  // namespace

namespace qmv {

// Device address of the current device's scratch (QMV_NOALLOC_MAX_ACT_BYTES
// bytes, 256-byte aligned), or NULL with *err set to the HIP error.
uint8_t* noalloc_scratch(int* err) {
    *err = 0;
    int dev = 0;
    hipError_t rc = hipGetDevice(&dev);
    if (rc != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        *err = rc != hipSuccess ? (int)rc : (int)hipErrorInvalidDevice;
        return nullptr;
    }
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_lookup_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* addr = nullptr;
    rc = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (rc != hipSuccess || !addr) {
        *err = rc != hipSuccess ? (int)rc : (int)hipErrorInvalidSymbol;
        return nullptr;
    }
    p = static_cast<uint8_t*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace qmv
