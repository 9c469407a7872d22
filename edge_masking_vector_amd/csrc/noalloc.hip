// noalloc.hip -- tm_colsum_noalloc: the column sum of tm_colsum for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Its slab partials live in a file-scope device array instead of a caller workspace.
//
// `scratch` below is a host-side stand-in in host code: handing its name to a kernel would compile
// and then fault on the GPU.  Its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch; only that address is ever
// passed to a kernel.  Each device holds its own copy of the array until the process ends.
//
// Nothing in the array has to start at zero: pass 1 writes every partial pass 2 reads.  Calls on
// one device share the array, so calls that overlap on one device race (same stream: they are
// ordered and safe).  The call makes no allocation of any kind (no hipMalloc, no hipFree, no
// allocating library routine).
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "plan.h"

#define TM_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // TM_COLSUM_NOALLOC_MAX_BYTES in tilemap.h
static_assert(kScratchBytes == TM_COLSUM_NOALLOC_MAX_BYTES, "header and library agree on the limit");

__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once taken

// The device address of `scratch` on the device that runs `stream`.
hipError_t scratch_for(hipStream_t stream, void **p) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[dev] == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return e;
        if (back != hipSuccess)
            return back;
        g_scratch[dev] = q;
    }
    *p = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

TM_API int tm_colsum_noalloc(const float *x, int64_t ldx, float *out, int64_t M, int64_t N, int TM,
                             int TN, int aligned, int walk, void *stream) {
    // Argument checks first, before any HIP call: the planner sees a stand-in workspace address
    // (never launched with) of the array's size, so a call needing more partials than the array
    // holds is refused with TM_E_WORKSPACE here.
    tmp::ColPlan plan;
    float *const stand_in = reinterpret_cast<float *>(uintptr_t{256});
    int st = tmp::plan_cols(x, ldx, out, M, N, TM, TN, aligned, walk, stand_in, kScratchBytes, &plan);
    if (st != TM_OK || !plan.finish)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (scratch_for(s, &ws) != hipSuccess)
        return TM_E_HIP;
    st = tmp::plan_cols(x, ldx, out, M, N, TM, TN, aligned, walk, ws, kScratchBytes, &plan);
    if (st != TM_OK)
        return st;
    return tmk::launch_cols(plan, s) == hipSuccess ? TM_OK : TM_E_HIP;
}
