// Internal launch interface between the C ABI layer (rvq_api.hip) and the
// kernels (encode.hip, decode.hip). Not installed, not exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rvq {

// Latent / codeword dimension the kernels are built for.
constexpr int kDim = 64;

// fp32-scored encode: frames per workgroup (4 wavefronts x 32 frames).
constexpr int kEncodeFramesPerBlock = 128;
constexpr int kEncodeThreads = 256;

// Decode: 16 lanes per frame (one float4 each), 256 threads per workgroup.
constexpr int kDecodeLanesPerFrame = 16;
constexpr int kDecodeThreads = 256;
// Codebooks from this size on (one XCD's L2) take the stage-ordered decode.
constexpr int64_t kDecodeTiledMinBookBytes = int64_t(4) << 20;

// Launches the fused multi-stage encode. `residual` and `recon` may be null.
hipError_t launch_encode(const float *x, int64_t n_frames, const float *books,
                         int n_stages, int n_codes, int32_t *codes, int codes_ld,
                         float *residual, float *recon, hipStream_t stream);

// Same contract and results, scores on the bf16 matrix cores (split-bf16).
hipError_t launch_encode_bf16(const float *x, int64_t n_frames, const float *books,
                              int n_stages, int n_codes, int32_t *codes, int codes_ld,
                              float *residual, float *recon, hipStream_t stream);

// Bytes of the prepared-codebook buffer for n_stages x n_codes (dim 64).
int64_t prepared_bytes(int n_stages, int n_codes);

// Writes the prepared codebooks (layout in prepared.h).
hipError_t launch_prepare(const float *books, int n_stages, int n_codes, void *prepared, hipStream_t stream);

// Same contract and results, scores on the fp16 matrix cores from prepared
// codebooks: batches of up to 8,192 frames split each stage's codebook over
// a workgroup's wavefronts, larger ones tile the frames.
hipError_t launch_encode_prepared(const float *x, int64_t n_frames, const float *books, const void *prepared,
                                  int n_stages, int n_codes, int32_t *codes, int codes_ld,
                                  float *residual, float *recon, hipStream_t stream);

// Launches the gather-sum decode.
hipError_t launch_decode(const int32_t *codes, int codes_ld, int64_t n_frames,
                         const float *books, int n_stages, int n_codes, float *out,
                         hipStream_t stream);

// y[N, 64] = h[N, hidden] W[64, hidden]^T + bias (bias nullable); hidden % 64 == 0.
hipError_t launch_linear_in(const float *h, int64_t n_frames, int hidden, const float *w,
                            const float *bias, float *y, hipStream_t stream);

// linear_in on r = fl32(src - table[codes[n * ld]]) (the previous stage's
// residual update of a per-stage projected quantizer), also storing r to dst
// (dst may be src).
hipError_t launch_linear_in_update(const float *src, const int32_t *codes, int codes_ld, const float *table,
                                   int n_codes, float *dst, int64_t n_frames, int hidden, const float *w,
                                   const float *bias, float *y, hipStream_t stream);

// out[N, hidden] = x[N, 64] W[hidden, 64]^T + bias (bias nullable); hidden % 64 == 0.
hipError_t launch_linear_out(const float *x, int64_t n_frames, int hidden, const float *w,
                             const float *bias, float *out, hipStream_t stream);

// Per-stage projected RVQ (projected.hip). Table of projected codewords
// P[q, k, :] = W_out[q] C[q, k] + b_out[q] (float64 sums, rounded once);
// w_out [Q, hidden, dim], b_out [Q, hidden] (nullable), table [Q, K, hidden];
// dim 64 or 8.
hipError_t launch_projected_table(const float *books, int n_stages, int n_codes, int dim, const float *w_out,
                                  const float *b_out, int hidden, float *table, hipStream_t stream);

// dst[n] = src[n] - table[codes[n * ld]] for one stage (src may be dst).
hipError_t launch_projected_update(const float *src, const int32_t *codes, int codes_ld, int64_t n_frames,
                                   const float *table, int n_codes, int hidden, float *dst, hipStream_t stream);

// out[n] = sum_q table[q, codes[n, q]], float32 from +0, stage 0 first.
hipError_t launch_projected_decode(const int32_t *codes, int codes_ld, int64_t n_frames, const float *table,
                                   int n_stages, int n_codes, int hidden, float *out, hipStream_t stream);

// Normalized (cosine) quantizer, codebook dim 8 (cosine.hip).
// units[q, k, :] = C[q, k] / max(|C[q, k]|, 1e-12) in float64.
hipError_t launch_cosine_units(const float *books, int n_stages, int n_codes, double *units, hipStream_t stream);

// y[N, 8] = W r + bias with W [8, hidden], hidden <= 1024; with prev_codes
// set, r = fl32(src - prev_table[prev_codes[n * ld]]) is also stored to dst.
hipError_t launch_proj8(const float *src, const int32_t *prev_codes, int codes_ld, const float *prev_table,
                        int n_codes, float *dst, int64_t n_frames, int hidden, const float *w, const float *bias,
                        float *y, hipStream_t stream);

// All stages of the normalized quantizer in one kernel (residual rows kept
// in registers); supported for n_codes <= 1024 and hidden <= 1024.
bool cosine_fused_supported(int n_codes, int hidden);
hipError_t launch_cosine_fused(const float *h, int64_t n_frames, int hidden, const float *w_in, const float *b_in,
                               const double *units, const float *table, int n_stages, int n_codes, int32_t *codes,
                               int codes_ld, float *latent, float *residual, hipStream_t stream);

// codes[n * ld] = argmin_k |u_n - units[k]|^2 with u_n = lat[n] / max(|lat[n]|, 1e-12), exact.
hipError_t launch_cosine_argmin(const float *lat, int64_t n_frames, const double *units, int n_codes,
                                int32_t *codes, int codes_ld, hipStream_t stream);

}  // namespace rvq
