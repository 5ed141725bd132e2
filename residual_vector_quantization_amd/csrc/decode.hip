// Gather-sum residual vector quantization decode for gfx950 (CDNA4).
//
// out[n] = sum_{q=0}^{Q-1} C[q, codes[n, q]], float32, accumulator starting
// at +0 and adding stage 0 first: the per-codebook get_rows-and-accumulate
// decode graph of the "RVQ codec" section of the "Architecture" page
// (omnivoice.cpp), with identity output projections.
//
// Layout: 16 lanes per frame, each lane owns one float4 (4 of the 64 dims),
// so every codeword gather and output store is a contiguous 256 B row. HBM
// traffic per frame is the Q codes and one output row; the codebook rows
// (Q x 256 B per frame) come from L2 / MALL, so the kernels are bound by the
// rate of 256 B row gathers out of cache rather than by HBM. Two kernels:
// frame-parallel (one frame per 16 lanes, stages in a loop) while the
// codebook is smaller than one XCD's L2, stage-ordered (below) from there on.
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

// Stage-ordered variant for codebooks of one XCD's L2 size and more (Q=32 x
// 1024 x 64 fp32 is 8 MiB against 4 MB). Each wavefront owns 32 frames
// with their accumulators in VGPRs and walks the stages in order, gathering
// stage q for all its frames before stage q+1. Every wavefront of the grid
// moves through the stages at about the same pace, so the rows being
// gathered at any moment come from a few stages that stay in L2 instead of
// the whole codebook. Each frame's sum is still +0 + C[0] + C[1] + ... in
// that order. Codes are staged per wavefront through LDS, 32 stages at a
// time, with a padded row (33 words) so the four frames read per
// instruction sit in different banks.
constexpr int kQChunk = 32;       // stages of codes staged in LDS at a time
constexpr int kCodeRow = kQChunk + 1;

template <int kTileFrames>        // frames per wavefront
__global__ __launch_bounds__(256)
void decode_tiled_kernel(const int32_t *__restrict__ codes, int codes_ld, int64_t n_frames,
                         const float *__restrict__ books, int n_stages, int n_codes,
                         float *__restrict__ out)
{
    constexpr int kG = kTileFrames / 4;   // frames per lane
    __shared__ int s_codes[4][kTileFrames * kCodeRow];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int part = lane & 15;   // float4 of the 64 dims
    const int sub = lane >> 4;    // frame within a group of 4
    const int64_t frame0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * kTileFrames;
    int *sc = s_codes[wave];

    f32x4 acc[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    unsigned bad = 0u;   // bit g: a code of frame 4g+sub is out of range

    for (int q0 = 0; q0 < n_stages; q0 += kQChunk) {
        const int qn = min(kQChunk, n_stages - q0);
        // codes of stages q0 .. q0+qn-1 for the wavefront's frames (0 past the batch)
        for (int i = lane; i < kTileFrames * kQChunk; i += 64) {
            const int f = i / kQChunk, j = i - f * kQChunk;
            const int64_t fr = frame0 + f;
            sc[f * kCodeRow + j] = (fr < n_frames && j < qn) ? codes[fr * codes_ld + q0 + j] : 0;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        for (int j = 0; j < qn; ++j) {
            const float *bq = books + static_cast<int64_t>(q0 + j) * n_codes * kDim + 4 * part;
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                int k = sc[(4 * g + sub) * kCodeRow + j];
                const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(n_codes);
                bad |= ok ? 0u : (1u << g);
                k = ok ? k : 0;
                const f32x4 v = *reinterpret_cast<const f32x4 *>(bq + static_cast<int64_t>(k) * kDim);
                acc[g][0] = acc[g][0] + v[0];
                acc[g][1] = acc[g][1] + v[1];
                acc[g][2] = acc[g][2] + v[2];
                acc[g][3] = acc[g][3] + v[3];
            }
        }
        // every lane is done reading this chunk of codes before it is overwritten
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
    }

#pragma unroll
    for (int g = 0; g < kG; ++g) {
        const int64_t fr = frame0 + 4 * g + sub;
        if (fr < n_frames) {
            const float nan = __builtin_nanf("");
            const f32x4 o = ((bad >> g) & 1u) ? f32x4{nan, nan, nan, nan} : acc[g];
            *reinterpret_cast<f32x4 *>(out + fr * kDim + 4 * part) = o;
        }
    }
}

}  // namespace

hipError_t launch_decode_tiled(const int32_t *codes, int codes_ld, int64_t n_frames, const float *books,
                               int n_stages, int n_codes, float *out, hipStream_t stream)
{
    constexpr int kTileFrames = 32;
    const int64_t blocks = (n_frames + 4 * kTileFrames - 1) / (4 * kTileFrames);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_tiled_kernel<kTileFrames>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       codes, codes_ld, n_frames, books, n_stages, n_codes, out);
    return hipGetLastError();
}

hipError_t launch_decode(const int32_t *codes, int codes_ld, int64_t n_frames,
                         const float *books, int n_stages, int n_codes, float *out,
                         hipStream_t stream)
{
    const int64_t book_bytes = static_cast<int64_t>(n_stages) * n_codes * kDim * sizeof(float);
    if (book_bytes >= kDecodeTiledMinBookBytes)
        return launch_decode_tiled(codes, codes_ld, n_frames, books, n_stages, n_codes, out, stream);
    const int64_t threads = n_frames * kDecodeLanesPerFrame;
    const int64_t blocks = (threads + kDecodeThreads - 1) / kDecodeThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kDecodeThreads), 0,
                       stream, codes, codes_ld, n_frames, books, n_stages, n_codes, out);
    return hipGetLastError();
}

}  // namespace rvq
