// Per-stage projected residual vector quantization for gfx950 (CDNA4).
//
// The codec quantizer of the "RVQ codec" section of the "Architecture" page
// (omnivoice.cpp): codebook q has its own project_in (hidden -> 64, with
// bias) and project_out (64 -> hidden, with bias), and the residual lives at
// the hidden width:
//
//   e = W_in[q] r + b_in[q];   k = argmin_i ||e - C[q,i]||^2;
//   r <- r - (W_out[q] C[q,k] + b_out[q]);
//   decode: out = sum_q (W_out[q] C[q,k_q] + b_out[q]), stage 0 first.
//
// The out-projection depends only on (q, k), so it is tabulated once per set
// of weights: P[q,k,:] = W_out[q] C[q,k] + b_out[q] (K x hidden floats per
// stage, 4 MiB at K = hidden = 1024), every entry a float64 sum over the
// codeword dims (64, or 8 for the normalized quantizer of cosine.hip) in
// ascending order with the bias added last, rounded once --
// the value a per-frame evaluation in that precision gives. The residual
// update and the decode are then gathers of table rows with no matrix work
// per frame: r <- fl32(r - P[q,k]) and out <- fl32(out + P[q,k]) from +0.
// The in-projection runs on the fp32 matrix cores (linear.hip) and the
// argmin is the exact single-stage encode on its output.
//
// Row kernels: one wavefront per frame, 64 lanes x float4 sweep the hidden
// row in 1 KiB steps, so every table gather and residual access is a
// contiguous, fully coalesced row.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rvq_internal.h"

namespace rvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTableCols = 256;   // output columns per workgroup (one per thread)
constexpr int kTableRows = 16;    // codewords per workgroup step
constexpr int kRowFrames = 4;     // frames per workgroup in the row kernels (one per wavefront)

// table[k, i] = fl32(sum_j C[k, j] W_out[i, j] (float64, j ascending) + b_out[i])
// for one stage, codeword dim kD; grid-strides over blocks of kTableRows codewords.
template <int kD>
__global__ __launch_bounds__(kTableCols)
void table_kernel(const float *__restrict__ book, const float *__restrict__ w_out,
                  const float *__restrict__ b_out, int n_codes, int hidden, float *__restrict__ table)
{
    __shared__ float s_c[kTableRows * kD];
    const int i = blockIdx.x * kTableCols + threadIdx.x;
    const bool active = i < hidden;
    float w[kD];
    const float *wi = w_out + static_cast<int64_t>(active ? i : 0) * kD;
#pragma unroll
    for (int t = 0; t < kD / 4; ++t) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(wi + 4 * t);
        w[4 * t] = v[0];
        w[4 * t + 1] = v[1];
        w[4 * t + 2] = v[2];
        w[4 * t + 3] = v[3];
    }
    const double bias = (b_out && active) ? static_cast<double>(b_out[i]) : 0.0;

    for (int k0 = blockIdx.y * kTableRows; k0 < n_codes; k0 += gridDim.y * kTableRows) {
        const int kn = min(kTableRows, n_codes - k0);
        __syncthreads();   // the previous block of rows is no longer read
        for (int t = threadIdx.x; t < kn * kD; t += kTableCols)
            s_c[t] = book[static_cast<int64_t>(k0) * kD + t];
        __syncthreads();
        if (!active) continue;
        for (int r = 0; r < kn; ++r) {
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < kD; ++j)
                s = __dadd_rn(s, __dmul_rn(static_cast<double>(s_c[r * kD + j]), static_cast<double>(w[j])));
            if (b_out) s = __dadd_rn(s, bias);
            table[static_cast<int64_t>(k0 + r) * hidden + i] = static_cast<float>(s);
        }
    }
}

// dst[n, :] = fl32(src[n, :] - table[codes[n * ld], :]) for one stage; src may
// be dst (each element is read, then written, by the same lane). A code
// outside [0, n_codes) gives a NaN row.
__global__ __launch_bounds__(64 * kRowFrames)
void update_kernel(const float *src, const int32_t *__restrict__ codes, int codes_ld, int64_t n_frames,
                   const float *__restrict__ table, int n_codes, int hidden, float *dst)
{
    const int lane = threadIdx.x & 63;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kRowFrames + (threadIdx.x >> 6);
    if (frame >= n_frames) return;
    int k = codes[frame * codes_ld];
    const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(n_codes);
    k = ok ? k : 0;
    const float *p = table + static_cast<int64_t>(k) * hidden;
    const float *s = src + frame * hidden;
    float *d = dst + frame * hidden;
    const float nan = __builtin_nanf("");
    for (int c = 4 * lane; c < hidden; c += 256) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(s + c);
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p + c);
        f32x4 o;
        o[0] = ok ? r[0] - v[0] : nan;
        o[1] = ok ? r[1] - v[1] : nan;
        o[2] = ok ? r[2] - v[2] : nan;
        o[3] = ok ? r[3] - v[3] : nan;
        *reinterpret_cast<f32x4 *>(d + c) = o;
    }
}

// out[n, :] = sum_q table[q, codes[n, q], :], float32 from +0, stage 0 first;
// a code outside [0, n_codes) gives a NaN row.
__global__ __launch_bounds__(64 * kRowFrames)
void projected_decode_kernel(const int32_t *__restrict__ codes, int codes_ld, int64_t n_frames,
                             const float *__restrict__ table, int n_stages, int n_codes, int hidden,
                             float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kRowFrames + (threadIdx.x >> 6);
    if (frame >= n_frames) return;
    const int32_t *row = codes + frame * codes_ld;
    const int64_t stage_floats = static_cast<int64_t>(n_codes) * hidden;
    bool bad = false;
    for (int q = 0; q < n_stages; ++q)
        bad = bad || static_cast<unsigned>(row[q]) >= static_cast<unsigned>(n_codes);
    float *o = out + frame * hidden;
    const float nan = __builtin_nanf("");
    for (int c = 4 * lane; c < hidden; c += 256) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!bad) {
            for (int q = 0; q < n_stages; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(
                    table + q * stage_floats + static_cast<int64_t>(row[q]) * hidden + c);
                acc[0] = acc[0] + v[0];
                acc[1] = acc[1] + v[1];
                acc[2] = acc[2] + v[2];
                acc[3] = acc[3] + v[3];
            }
        } else {
            acc = f32x4{nan, nan, nan, nan};
        }
        *reinterpret_cast<f32x4 *>(o + c) = acc;
    }
}

// Stage-ordered decode for tables larger than an XCD's L2: each wavefront
// owns kF frames with their hidden-width accumulators in VGPRs (hidden <=
// 1024) and adds stage q's rows for all of them before stage q+1, so the
// resident wavefronts sweep the stages together and gather from one or two
// stage tables at a time (4 MiB each at K = hidden = 1024) instead of the
// whole table. Per element the sum is the same: +0, stage 0 first. The
// wavefront's codes are staged through LDS 32 stages at a time, so a row
// address waits on an LDS read rather than on a global load per stage.
constexpr int kTiledFrames = 4;
constexpr int kTiledCols = 4;   // float4 columns per lane (hidden <= 1024)
constexpr int kCodeStages = 32;                 // stages of codes staged in LDS at a time
constexpr int kCodeRow = kCodeStages + 1;       // padded row per frame

__global__ __launch_bounds__(64 * kRowFrames)
void projected_decode_tiled_kernel(const int32_t *__restrict__ codes, int codes_ld, int64_t n_frames,
                                   const float *__restrict__ table, int n_stages, int n_codes, int hidden,
                                   float *__restrict__ out)
{
    __shared__ int s_codes[kRowFrames][kTiledFrames * kCodeRow];
    const int lane = threadIdx.x & 63;
    const int cols = hidden >> 2;
    const int64_t frame0 = (static_cast<int64_t>(blockIdx.x) * kRowFrames + (threadIdx.x >> 6)) * kTiledFrames;
    const int64_t stage_floats = static_cast<int64_t>(n_codes) * hidden;
    int *sc = s_codes[threadIdx.x >> 6];
    f32x4 acc[kTiledFrames][kTiledCols];
#pragma unroll
    for (int f = 0; f < kTiledFrames; ++f)
#pragma unroll
        for (int t = 0; t < kTiledCols; ++t) acc[f][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    unsigned bad = 0u;   // bit f: frame f has a code outside [0, n_codes)
    for (int q = 0; q < n_stages; ++q) {
        const int j = q % kCodeStages;
        if (j == 0) {
            // codes of stages q .. q+31 for the wavefront's frames (0 past the batch or the stages)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();   // the previous block of codes is read
            for (int i = lane; i < kTiledFrames * kCodeStages; i += 64) {
                const int f = i / kCodeStages, jj = i - f * kCodeStages;
                const int64_t fr = frame0 + f;
                sc[f * kCodeRow + jj] = (fr < n_frames && q + jj < n_stages) ? codes[fr * codes_ld + q + jj] : 0;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
        const float *tq = table + q * stage_floats;
#pragma unroll
        for (int f = 0; f < kTiledFrames; ++f) {
            int k = sc[f * kCodeRow + j];   // 0 for frames past the batch
            const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(n_codes);
            bad |= ok ? 0u : (1u << f);
            k = ok ? k : 0;
            const float *row = tq + static_cast<int64_t>(k) * hidden;
#pragma unroll
            for (int t = 0; t < kTiledCols; ++t) {
                const int col = lane + 64 * t;
                if (col < cols) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(row + 4 * col);
                    acc[f][t][0] = acc[f][t][0] + v[0];
                    acc[f][t][1] = acc[f][t][1] + v[1];
                    acc[f][t][2] = acc[f][t][2] + v[2];
                    acc[f][t][3] = acc[f][t][3] + v[3];
                }
            }
        }
    }
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int f = 0; f < kTiledFrames; ++f) {
        const int64_t fr = frame0 + f;
        if (fr >= n_frames) continue;
        float *o = out + fr * hidden;
#pragma unroll
        for (int t = 0; t < kTiledCols; ++t) {
            const int col = lane + 64 * t;
            if (col < cols)
                *reinterpret_cast<f32x4 *>(o + 4 * col) = ((bad >> f) & 1u) ? f32x4{nan, nan, nan, nan} : acc[f][t];
        }
    }
}

}  // namespace

hipError_t launch_projected_table(const float *books, int n_stages, int n_codes, int dim, const float *w_out,
                                  const float *b_out, int hidden, float *table, hipStream_t stream)
{
    if (dim != 8 && dim != kDim) return hipErrorInvalidValue;
    const unsigned gx = static_cast<unsigned>((hidden + kTableCols - 1) / kTableCols);
    const unsigned gy = static_cast<unsigned>(min((n_codes + kTableRows - 1) / kTableRows, 4096));
    for (int q = 0; q < n_stages; ++q) {
        const float *bq = books + static_cast<int64_t>(q) * n_codes * dim;
        const float *wq = w_out + static_cast<int64_t>(q) * hidden * dim;
        const float *biq = b_out ? b_out + static_cast<int64_t>(q) * hidden : nullptr;
        float *tq = table + static_cast<int64_t>(q) * n_codes * hidden;
        if (dim == 8)
            hipLaunchKernelGGL(table_kernel<8>, dim3(gx, gy), dim3(kTableCols), 0, stream, bq, wq, biq, n_codes,
                               hidden, tq);
        else
            hipLaunchKernelGGL(table_kernel<kDim>, dim3(gx, gy), dim3(kTableCols), 0, stream, bq, wq, biq, n_codes,
                               hidden, tq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_projected_update(const float *src, const int32_t *codes, int codes_ld, int64_t n_frames,
                                   const float *table, int n_codes, int hidden, float *dst, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kRowFrames - 1) / kRowFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(update_kernel, dim3(static_cast<unsigned>(blocks)), dim3(64 * kRowFrames), 0, stream,
                       src, codes, codes_ld, n_frames, table, n_codes, hidden, dst);
    return hipGetLastError();
}

hipError_t launch_projected_decode(const int32_t *codes, int codes_ld, int64_t n_frames, const float *table,
                                   int n_stages, int n_codes, int hidden, float *out, hipStream_t stream)
{
    const int64_t table_bytes = static_cast<int64_t>(n_stages) * n_codes * hidden * sizeof(float);
    if (table_bytes >= kDecodeTiledMinBookBytes && hidden <= 256 * kTiledCols) {
        const int64_t per_block = static_cast<int64_t>(kRowFrames) * kTiledFrames;
        const int64_t tb = (n_frames + per_block - 1) / per_block;
        if (tb > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL(projected_decode_tiled_kernel, dim3(static_cast<unsigned>(tb)), dim3(64 * kRowFrames), 0,
                           stream, codes, codes_ld, n_frames, table, n_stages, n_codes, hidden, out);
        return hipGetLastError();
    }
    const int64_t blocks = (n_frames + kRowFrames - 1) / kRowFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(projected_decode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(64 * kRowFrames), 0,
                       stream, codes, codes_ld, n_frames, table, n_stages, n_codes, hidden, out);
    return hipGetLastError();
}

}  // namespace rvq
