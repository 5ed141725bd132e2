// Gather-sum residual vector quantization decode for gfx950 (CDNA4).
//
// out[n] = sum_{q=0}^{Q-1} C[q, codes[n, q]], float32, accumulator starting
// at +0 and adding stage 0 first: the per-codebook get_rows-and-accumulate
// decode graph of the "RVQ codec" section of the "Architecture" page
// (omnivoice.cpp), with identity output projections.
//
// Layout: 16 lanes per frame, each lane owns one float4 (4 of the 64 dims),
// so a wavefront covers 4 frames and every codeword gather and output store
// is a contiguous 256 B row. HBM traffic per frame is the Q codes and one
// output row; codebooks (2 MiB at Q=8) are re-read from L2 / MALL.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rvq_internal.h"

namespace rvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kDecodeThreads)
void decode_kernel(const int32_t *__restrict__ codes, int codes_ld, int64_t n_frames,
                   const float *__restrict__ books, int n_stages, int n_codes,
                   float *__restrict__ out)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kDecodeThreads + threadIdx.x;
    const int64_t frame = gid / kDecodeLanesPerFrame;
    const int part = static_cast<int>(gid % kDecodeLanesPerFrame);
    if (frame >= n_frames) return;

    const int32_t *row = codes + frame * codes_ld;
    const float *base = books + 4 * part;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    bool bad = false;
#pragma unroll 8
    for (int q = 0; q < n_stages; ++q) {
        int k = row[q];
        const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(n_codes);
        bad = bad || !ok;
        k = ok ? k : 0;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(
            base + (static_cast<int64_t>(q) * n_codes + k) * kDim);
        acc[0] = acc[0] + v[0];
        acc[1] = acc[1] + v[1];
        acc[2] = acc[2] + v[2];
        acc[3] = acc[3] + v[3];
    }
    if (bad) acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    *reinterpret_cast<f32x4 *>(out + frame * kDim + 4 * part) = acc;
}

}  // namespace

hipError_t launch_decode(const int32_t *codes, int codes_ld, int64_t n_frames,
                         const float *books, int n_stages, int n_codes, float *out,
                         hipStream_t stream)
{
    const int64_t threads = n_frames * kDecodeLanesPerFrame;
    const int64_t blocks = (threads + kDecodeThreads - 1) / kDecodeThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kDecodeThreads), 0,
                       stream, codes, codes_ld, n_frames, books, n_stages, n_codes, out);
    return hipGetLastError();
}

}  // namespace rvq
