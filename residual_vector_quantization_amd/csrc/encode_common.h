// Device helpers shared by the two encode kernels (fp32 and split-bf16
// scoring): packed keys and the exact float64 distance used to decide
// every pick. Internal header.
#pragma once

#include <float.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rvq_internal.h"

namespace rvq {
namespace enc {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kUnit = 5.9604644775390625e-08f;   // 2^-24
// gamma_n = n u / (1 - n u)
__host__ __device__ constexpr float gamma_n(int n) { return n * kUnit / (1.0f - n * kUnit); }

// A key is a score with its 6 low mantissa bits replaced by a codeword index
// local to a 64-codeword group; replacing them moves the value by less than
// 2^-17 of it.
constexpr unsigned kKeyMask = 0xFFFFFFC0u;
constexpr float kKeyError = 7.62939453125e-06f;
// Stands in for +inf in keys (an inf with index bits would be a NaN).
constexpr float kNoScore = FLT_MAX;
// Absolute slack for results in the fp32 subnormal range.
constexpr float kAbsSlack = 1e-35f;

__device__ __forceinline__ float make_key(float s, int lk)
{
    return __uint_as_float((__float_as_uint(s) & kKeyMask) | static_cast<unsigned>(lk));
}

// Float64 sum_j (r_j - c_j)^2 over this lane's 32 dims with n = -r,
// continuing from `acc`, one rounding per operation. fl(n + c) = -fl(r - c)
// exactly, so the squares equal those of the direct form.
__device__ inline double sq_dist_part(double acc, const float (&n)[32], const float *c)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(c + 4 * t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double d = __dadd_rn(static_cast<double>(n[4 * t + e]), static_cast<double>(v[e]));
            acc = __dadd_rn(acc, __dmul_rn(d, d));
        }
    }
    return acc;
}

// Float64 direct-form distance of codeword `k` (row pointer `book`, stage
// base) to the frame held by lane pair (l, l^32): half 0 sums dims 0..31
// from zero, half 1 continues with dims 32..63, so the sum runs j = 0..63
// in order. Every lane must call it (it shuffles); the result is valid on
// both lanes of each frame.
__device__ inline double pair_distance(const float (&n)[32], const float *book, int k, int half)
{
    const float *c = book + static_cast<int64_t>(k) * kDim + 32 * half;
    double s = 0.0;
    if (half == 0) s = sq_dist_part(0.0, n, c);
    const double p = __shfl_xor(s, 32);
    if (half == 1) s = sq_dist_part(p, n, c);
    const double x = __shfl_xor(s, 32);
    return half ? s : x;
}

// Full float64 rescan of frame f (lanes f, f+32) over all n_codes codewords
// of `book`, by the whole wavefront, two codewords per lane at a time;
// ties go to the lowest index. `row` is a 64-float LDS row owned by this
// wavefront. Returns the winner on every lane. Every lane must call it.
__device__ inline int rescan_frame(const float (&n)[32], float *row, const float *book, int n_codes,
                                   int f, int lane)
{
    const int col = lane & 31, half = lane >> 5;
    if (col == f) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            *reinterpret_cast<f32x4 *>(&row[32 * half + 4 * t]) =
                f32x4{n[4 * t], n[4 * t + 1], n[4 * t + 2], n[4 * t + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    double bd = INFINITY;
    int bk = 0x7fffffff;
    for (int k0 = lane; k0 < n_codes; k0 += 128) {
        const int k1 = k0 + 64;
        const bool has1 = k1 < n_codes;
        const float *c0 = book + static_cast<int64_t>(k0) * kDim;
        const float *c1 = book + static_cast<int64_t>(has1 ? k1 : k0) * kDim;
        double s0 = 0.0, s1 = 0.0;
#pragma unroll 4
        for (int t = 0; t < 16; ++t) {
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(c0 + 4 * t);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(c1 + 4 * t);
            const f32x4 rv = *reinterpret_cast<const f32x4 *>(row + 4 * t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double rj = static_cast<double>(rv[e]);
                const double d0 = __dadd_rn(rj, static_cast<double>(v0[e]));
                const double d1 = __dadd_rn(rj, static_cast<double>(v1[e]));
                s0 = __dadd_rn(s0, __dmul_rn(d0, d0));
                s1 = __dadd_rn(s1, __dmul_rn(d1, d1));
            }
        }
        // k0 < k1 and both ascend, so strict "<" keeps the lowest index on ties
        if (s0 < bd) {
            bd = s0;
            bk = k0;
        }
        if (has1 && s1 < bd) {
            bd = s1;
            bk = k1;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double od = __shfl_xor(bd, off);
        const int ok = __shfl_xor(bk, off);
        if (od < bd || (od == bd && ok < bk)) {
            bd = od;
            bk = ok;
        }
    }
    // all reads of `row` are done before a later call overwrites it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    return bk;
}

}  // namespace enc
}  // namespace rvq
