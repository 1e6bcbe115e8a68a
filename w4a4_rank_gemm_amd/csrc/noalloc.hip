// noalloc.hip -- twq_linear on memory the library owns, for callers that cannot allocate.
//
// twq_linear needs scratch memory for Q_X, s_X and T (or T's partial sums over K
// slices) between its two launches. twq_linear_noalloc takes that scratch from a
// file-scope device array instead of a caller workspace, so a call makes no
// allocation of any kind: code under stream capture, serving loops and harnesses
// that forbid hipMalloc can use it. Each GPU holds its own copy of the array (the
// code object's zero-initialized data) from the first use until the process ends.
//
// The array's name is only a host-side stand-in for the device symbol; its device
// address on a GPU comes from hipGetSymbolAddress with that GPU current, once per
// device, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "twq.h"
#include "twq_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // twq_linear_noalloc_max_bytes()
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};  // device address of `scratch` on each GPU, once taken

// The device address of the scratch array on the calling thread's current GPU.
hipError_t scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t twq_linear_noalloc_max_bytes(void) { return kScratchBytes; }

twq_status twq_linear_noalloc(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t,
                              int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *stream) {
    const int st = twq::linear_check(x, qw, sw, l1t, l2t, r, y, b, m, n);
    if (st != TWQ_OK) return (twq_status)st;
    if (b == 0 || n == 0) return TWQ_OK;
    const size_t need = twq::linear_workspace(b, m, n, r, 0, 0);
    if (need > kScratchBytes) return TWQ_ERR_WORKSPACE;  // before any HIP call
    void *ws = nullptr;
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) return (twq_status)twq::hip_error(e, "twq_linear_noalloc");
    return (twq_status)twq::linear_run(x, qw, sw, l1t, l2t, r, y, b, m, n, 0, ws, kScratchBytes, stream,
                                       "twq_linear_noalloc", 0, false);
}

}  // extern "C"
