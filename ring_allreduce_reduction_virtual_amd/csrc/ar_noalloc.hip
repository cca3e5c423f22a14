// The reduce-scatter entry point that allocates nothing: ar_reduce_scatter_noalloc.
//
// The ring's reduce-scatter keeps its partial sums between steps in a
// workspace, since its receive buffers hold one shard each.  Callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid it) get that workspace from a fixed array in
// device memory instead: `scratch` below, AR_NOALLOC_SCRATCH_BYTES bytes,
// which every device the library runs on holds from the first call there
// until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory.  Its
// device address is looked up once per device, with that device current,
// with hipGetSymbolAddress, and only that address is ever handed to a kernel.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "ar.h"
#include "ar_internal.h"

namespace {

static __device__ __align__(256) char scratch[AR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_lookup;

ar_result_t fail(ar_result_t code, const char* text) {
    arimpl::set_error_detail(text);
    return code;
}

// The current device's copy of `scratch`, looked up on the first call on that device.
ar_result_t device_scratch(char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(AR_ERR_HIP, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(AR_ERR_UNSUPPORTED, "device index beyond the scratch table");
    char* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || addr == nullptr) {
                char buf[160];
                std::snprintf(buf, sizeof(buf), "hipGetSymbolAddress(scratch): %s",
                              e != hipSuccess ? hipGetErrorString(e) : "null address");
                return fail(AR_ERR_HIP, buf);
            }
            p = static_cast<char*>(addr);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return AR_SUCCESS;
}

}  // namespace

extern "C" ar_result_t ar_reduce_scatter_noalloc(const void* const* sendbufs, void* const* recvbufs, size_t count,
                                                 ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo,
                                                 hipStream_t stream) {
    const size_t need = ar_workspace_bytes(AR_COLL_REDUCE_SCATTER, algo, count, dtype, nranks);
    const bool bad = sendbufs == nullptr || recvbufs == nullptr || op < AR_SUM || op > AR_AVG;
    if (need == 0 || need == static_cast<size_t>(-1) || bad) {
        // no partials to keep, or arguments the ordinary validation rejects
        // before anything touches the device
        return ar_reduce_scatter_ex(sendbufs, recvbufs, count, dtype, op, nranks, algo, nullptr, 0, stream);
    }
    if (need > AR_NOALLOC_SCRATCH_BYTES) {
        char buf[200];
        std::snprintf(buf, sizeof(buf),
                      "this call needs %zu bytes of scratch; the no-allocation entry point holds %llu", need,
                      static_cast<unsigned long long>(AR_NOALLOC_SCRATCH_BYTES));
        return fail(AR_ERR_INVALID_ARGUMENT, buf);
    }
    char* ws = nullptr;
    const ar_result_t rc = device_scratch(&ws);
    if (rc != AR_SUCCESS) return rc;
    return ar_reduce_scatter_ex(sendbufs, recvbufs, count, dtype, op, nranks, algo, ws, AR_NOALLOC_SCRATCH_BYTES,
                                stream);
}
