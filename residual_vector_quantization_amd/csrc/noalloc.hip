// rvq_encode_noalloc: the prepared-codebook encode with the prepared layout
// kept in a fixed device array of the library instead of a caller buffer,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: each GPU the library runs
// on holds its own copy (RVQ_NOALLOC_SCRATCH_BYTES) until the process ends.
// In host code its name is only a stand-in for the symbol, not a device
// address, so the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels. Every call on a GPU rewrites the whole part of the
// array that the encode reads (the preparation kernel writes every row,
// norm, maximum and exponent, padding rows included), so nothing has to
// start at zero; calls that overlap on one GPU (different streams, or
// another thread) race on the array.
#include <mutex>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rvq.h"
#include "rvq_internal.h"

namespace {

constexpr int64_t kScratchBytes = RVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// The device address of `scratch` on device `dev` (looked up on first use,
// with `dev` current; the caller's current device is restored).
hipError_t scratch_on(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

RVQ_API rvq_status rvq_encode_noalloc(const float *x, int64_t n_frames, int32_t dim, const float *codebooks,
                                      int32_t n_stages, int32_t n_codes, int32_t *codes, int32_t codes_ld,
                                      float *recon, float *residual, void *stream)
{
    if (n_frames < 0 || dim <= 0 || n_stages <= 0 || n_codes <= 0) return RVQ_ERR_INVALID_ARG;
    if (dim != rvq::kDim || n_stages > 65536) return RVQ_ERR_UNSUPPORTED;
    if (codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (rvq::prepared_bytes(n_stages, n_codes) > kScratchBytes) return RVQ_ERR_UNSUPPORTED;
    if (n_frames == 0) return RVQ_OK;
    if (!x || !codebooks || !codes) return RVQ_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(codebooks, 16) || !aligned(codes, 4) ||
        (recon && !aligned(recon, 16)) || (residual && !aligned(residual, 16)))
        return RVQ_ERR_INVALID_ARG;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return RVQ_ERR_DEVICE;
    void *prep = nullptr;
    if (scratch_on(dev, &prep) != hipSuccess) return RVQ_ERR_DEVICE;
    if (rvq::launch_prepare(codebooks, n_stages, n_codes, prep, s) != hipSuccess) return RVQ_ERR_DEVICE;
    return rvq::launch_encode_prepared(x, n_frames, codebooks, prep, n_stages, n_codes, codes, codes_ld, residual,
                                       recon, s) == hipSuccess
               ? RVQ_OK
               : RVQ_ERR_DEVICE;
}

}  // extern "C"
