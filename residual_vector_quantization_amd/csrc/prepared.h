// Byte layout of the prepared codebooks (rvq_prepare_codebooks), shared by
// the kernel that writes them and the encode kernels that read them.
// Internal header.
//
// Per stage one block, kStageAlign-aligned, with Kp = n_codes rounded up to
// kChunk rows:
//   rows   [Kp][144 B]        128 B: fp16 of c' = 2^e c (round to nearest even), dims in
//                             order; then 16 B: 0.5*||c'||^2 (fp32 sum) as two fp16 parts
//                             hi | lo << 16 in the first word, zeros after it
//   max    [Kp/kChunk] u32    bits of the largest valid 0.5*||c'||^2 of each kChunk rows,
//                             or of +inf when the stage is out of the fp16 range
//   e      i32                the stage's power-of-two scale
// Rows k >= n_codes are zero.
#pragma once

#include <stdint.h>

namespace rvq {
namespace prep {

constexpr int kChunk = 256;
constexpr int64_t kStageAlign = 256;

__host__ __device__ inline int64_t padded_codes(int n_codes) { return (n_codes + kChunk - 1) / kChunk * kChunk; }
__host__ __device__ inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

constexpr int64_t kF16Row = 144;   // bytes of a row
__host__ __device__ inline int64_t f16_max(int64_t kp) { return kp * kF16Row; }
__host__ __device__ inline int64_t f16_exp(int64_t kp) { return f16_max(kp) + 4 * (kp / kChunk); }

__host__ __device__ inline int64_t stage_bytes(int n_codes)
{
    const int64_t kp = padded_codes(n_codes);
    return round_up(f16_exp(kp) + 4, kStageAlign);
}

// The stage scale e is chosen so that max |c'| lies in [1/2, 1), clamped to
// [kMinExp, kMaxExp] so that 2^-e is an fp16 value (normal or subnormal).
// A stage whose largest |c'| still exceeds kMaxScaled (entries beyond
// 2^20), or that holds a non-finite entry, is marked by an infinite max.
constexpr int kMinExp = -15;
constexpr int kMaxExp = 24;
constexpr float kMaxScaled = 32.0f;

}  // namespace prep
}  // namespace rvq
