// jt_draft_verify_step_noalloc: the fused step with its scratch in a file-scope device
// array instead of a caller's workspace, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` holds what the workspace holds for jt_draft_verify_step (split-KV partial
// rows, the top-W partial lists, the arg-max partial keys, the per-sequence flags).  None
// of it needs initialising: every call writes what it later reads.  Each GPU that runs
// the call holds its own copy of the array until the process ends; calls that overlap in
// time on one GPU share it and race.
//
// In host code `scratch` names a host-side stand-in, not device memory.  Its device
// address is looked up once per device (hipGetSymbolAddress, with that device current)
// and kept; only that address is ever passed to a kernel.
#include <mutex>

#include "jt_internal.h"

namespace jt {

static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_at[kMaxDevices] = {};

// The device address of `scratch` on the device that `stream` runs on.
jt_status scratch_address(hipStream_t stream, void **out)
{
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess)
        return JT_ERR_LAUNCH;
    int dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess)
        return JT_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices)
        return JT_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_at[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return JT_ERR_LAUNCH;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur)
            (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return JT_ERR_LAUNCH;
        g_scratch_at[dev] = p;
    }
    *out = g_scratch_at[dev];
    return JT_OK;
}

} // namespace

jt_status launch_step_static(const StepLaunch &in, hipStream_t st)
{
    void *ws = nullptr;
    const jt_status e = scratch_address(st, &ws);
    if (e != JT_OK)
        return e;
    return launch_step(in, ws, st);
}

} // namespace jt
