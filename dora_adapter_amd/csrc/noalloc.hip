// noalloc.hip - dora_forward_noalloc: the module forward for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// It is dora_forward with the caller's workspace replaced by `scratch`, a
// file-scope device array of DORA_NOALLOC_SCRATCH_BYTES that every GPU the
// library runs on holds from module load until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept per device, and only that address is ever handed
// to dora_forward (and so to the kernels).
//
// Every call on a GPU shares that GPU's array.  No part of it needs to start
// at zero: each byte the forward's kernels read was written earlier in the
// same call (split-K slots, row-dot partials, the Gram pair, P).  Calls that
// overlap in time on one GPU (different streams, or threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dora.h"
#include "dora_internal.hpp"

namespace dora {
namespace {

constexpr size_t kScratchBytes = DORA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

// Device address of `scratch` on the device that owns `stream` (the current
// device for the null stream), looked up on first use with that device
// current.
int scratch_on(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return set_error(DORA_E_HIP, "dora_forward_noalloc: device of the stream: %s",
                         hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(DORA_E_HIP, "dora_forward_noalloc: device %d beyond the %d supported",
                         dev, kMaxDevices);
    std::lock_guard<std::mutex> hold(g_lock);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev)
            e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess)
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = (cur >= 0 && cur != dev) ? hipSetDevice(cur) : hipSuccess;
        if (e == hipSuccess)
            e = back;
        if (e != hipSuccess || p == nullptr)
            return set_error(DORA_E_HIP, "dora_forward_noalloc: scratch address on device %d: %s",
                             dev, e != hipSuccess ? hipGetErrorString(e) : "null");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DORA_OK;
}

}  // namespace
}  // namespace dora

extern "C" int dora_forward_noalloc(const void *x, const void *W, const void *A, const void *B,
                                    const float *m, float s, int64_t T, int64_t d_in,
                                    int64_t d_out, int64_t r, int dtype, void *y, float *n_out,
                                    void *P_out, const float *n_in, float *U_out, void *stream)
{
    using namespace dora;
    clear_error();
    // the size check comes first: it needs no device
    const size_t need = dora_forward_workspace(T, d_in, d_out, r, dtype);
    if (need > kScratchBytes)
        return set_error(DORA_E_WORKSPACE,
                         "dora_forward_noalloc: this module needs %zu bytes of scratch, above "
                         "the library's fixed %zu",
                         need, kScratchBytes);
    if (need == 0)  // invalid arguments: dora_forward reports which
        return dora_forward(x, W, A, B, m, s, T, d_in, d_out, r, dtype, y, n_out, P_out, n_in,
                            U_out, nullptr, 0, stream);
    void *ws = nullptr;
    const int rc = scratch_on(static_cast<hipStream_t>(stream), &ws);
    if (rc != DORA_OK)
        return rc;
    return dora_forward(x, W, A, B, m, s, T, d_in, d_out, r, dtype, y, n_out, P_out, n_in, U_out,
                        ws, kScratchBytes, stream);
}
