// Scratch memory of gemm_bf16_noalloc, the entry point for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array of GEMM_NOALLOC_SCRATCH_BYTES:
// every GPU the library runs on holds its own copy from the time the library's
// code object is loaded on it until the process ends.  Host code never uses
// the array's name as an address (in host code it only names the symbol): the
// first call on a device looks its address up with hipGetSymbolAddress, with
// that device current, and keeps it; kernels receive that address.
#include <atomic>
#include <cstdint>
#include <mutex>

#include <hip/hip_runtime.h>

#include "gemm_problem.hpp"
#include "libgemm.h"

namespace libgemm {
namespace {

static __device__ __align__(256) char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mutex;

}  // namespace

hipError_t scratch_address(hipStream_t stream, void **ptr) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = 0;
            e = hipGetDevice(&cur);
            if (e != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return e;
            if (back != hipSuccess) return back;
            if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace libgemm
