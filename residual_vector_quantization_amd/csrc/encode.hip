// Fused multi-stage residual vector quantization encode for gfx950 (CDNA4).
//
// Computes the residual loop of the "RVQ codec" section of the
// "Architecture" page (omnivoice.cpp): for q = 0..Q-1 pick
// argmin_k ||r - C[q,k]||^2 (lowest k on ties), emit k, r <- r - C[q,k].
//
// Work split
//   * One workgroup = 4 wavefronts = 128 frames; a wavefront owns 32 frames
//     for all Q stages, so a frame's argmin never leaves its wavefront.
//   * Residuals stay in VGPRs for the whole call. Lane l holds frame l%32;
//     lanes 0-31 keep dims 0..31, lanes 32-63 keep dims 32..63.
//   * Codebooks stream through LDS in chunks of 128 codewords (double
//     buffered, one barrier per chunk). While staging, each codeword is
//     negated and 0.5*||c||^2 is computed beside it.
//   * Scores on fp32 matrix cores: v_mfma_f32_32x32x2_f32 with codewords on
//     the M (row) side and frames on the N (column) side, accumulator
//     initialised with 0.5*||c||^2, so one 32-step chain yields
//         s_k = 0.5*||c_k||^2 - r.c_k  (= 0.5*(||r - c_k||^2 - ||r||^2)).
//     In the 32x32 output each lane holds 16 scores of one frame; the other
//     16 of that frame sit in lane l^32.
//   * Per lane: running best score/index and the second-best score.
//
// Exactness
//   The fp32 score of codeword k differs from the exact value by at most
//       e = gamma_{2D+2} * (0.5*||c_k||^2 + ||r||*||c_k||)
//   (norm and dot product each summed in fp32, any order). Every codeword
//   whose score lies within 2*kSafety*e_max of the best score is a candidate
//   for the true argmin, and nothing else can be. If the candidates are one
//   codeword it is the answer; if they are the two lane bests, both are
//   re-ranked with the float64 direct-form distance sum_j (r_j - c_j)^2,
//   j ascending, one rounding per operation; if a lane holds more than one
//   candidate, the wavefront rescans all K codewords of that frame with the
//   same float64 sum. The pick is therefore the argmin of that float64
//   distance, independent of fp32 rounding order.
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "rvq_internal.h"

namespace rvq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kFramesPerWave = 32;
constexpr int kChunk = 128;         // codewords per LDS chunk
constexpr int kRow = kDim + 4;      // padded LDS row (floats): 8 lanes of a b128 read hit 32 banks
constexpr int kBlocksPerChunk = kChunk / 32;

static_assert(kThreads == kEncodeThreads, "thread count");
static_assert(kWaves * kFramesPerWave == kEncodeFramesPerBlock, "frames per block");
static_assert(kThreads == 2 * kChunk, "staging maps 2 threads to a codeword row");

// gamma_n = n*u / (1 - n*u), u = 2^-24, n = 2D + 2 roundings bound one score.
constexpr float kUnit = 5.9604644775390625e-08f;
constexpr float kGamma = (2 * kDim + 2) * kUnit / (1.0f - (2 * kDim + 2) * kUnit);
// Margin for matrix-core rounding that is not round-to-nearest per step.
constexpr float kSafety = 4.0f;
// Absolute slack for results that land in the fp32 subnormal range.
constexpr float kAbsSlack = 1e-35f;

// Float64 sum_j (r_j - c_j)^2 over 32 dims, continuing from `acc`,
// one rounding per operation (no contraction into fma).
__device__ inline double sq_dist_part(double acc, const float (&r)[32], const float *c)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(c + 4 * t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double d = __dsub_rn(static_cast<double>(r[4 * t + e]), static_cast<double>(v[e]));
            acc = __dadd_rn(acc, __dmul_rn(d, d));
        }
    }
    return acc;
}

template <bool kRecon, bool kResidual>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void encode_kernel(const float *__restrict__ x, int64_t n_frames,
                   const float *__restrict__ books, int n_stages, int n_codes,
                   int32_t *__restrict__ codes, int codes_ld,
                   float *__restrict__ residual, float *__restrict__ recon)
{
    __shared__ __align__(16) float s_book[2][kChunk * kRow];
    __shared__ __align__(16) float s_norm[2][kChunk];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kEncodeFramesPerBlock +
                          wave * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    float r[32];
    float acc[32];
    if (valid) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(x + frame * kDim + 32 * half);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 v = src[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[4 * t + e] = v[e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) r[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.0f;

    const int n_chunks = (n_codes + kChunk - 1) / kChunk;
    const int total = n_stages * n_chunks;

    // Staging role: thread -> (codeword row, 32-float half of it).
    const int srow = tid >> 1;
    const int scol = (tid & 1) * 32;
    f32x4 stage[8];

    auto fetch = [&](int g) {
        const int q = g / n_chunks;
        const int k = (g - q * n_chunks) * kChunk + srow;
        if (k < n_codes) {
            const f32x4 *p = reinterpret_cast<const f32x4 *>(
                books + (static_cast<int64_t>(q) * n_codes + k) * kDim + scol);
#pragma unroll
            for (int i = 0; i < 8; ++i) stage[i] = p[i];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) stage[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    auto commit = [&](int buf) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s = s + stage[i][e] * stage[i][e];
        s = s + __shfl_xor(s, 1);
        float *dst = &s_book[buf][srow * kRow + scol];
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4 *>(dst + 4 * i) = -stage[i];
        if ((tid & 1) == 0) s_norm[buf][srow] = 0.5f * s;
    };

    fetch(0);
    commit(0);
    __syncthreads();

    float best = INFINITY, second = INFINITY;
    unsigned cmax = 0u;       // bits of max 0.5*||c||^2 seen by this lane in this stage
    int best_k = 0;

    for (int g = 0; g < total; ++g) {
        const int buf = g & 1;
        const int q = g / n_chunks;
        const int c = g - q * n_chunks;
        if (g + 1 < total) fetch(g + 1);

        // ---- scores of this chunk: two 32-codeword blocks, interleaved chains
        {
            const float *sb = s_book[buf];
            const float *sn = s_norm[buf];
            f32x16 d[kBlocksPerChunk];
#pragma unroll
            for (int b = 0; b < kBlocksPerChunk; ++b) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const f32x4 nv = *reinterpret_cast<const f32x4 *>(sn + b * 32 + 8 * m + 4 * half);
                    // norms are >= 0, so their bit patterns order like the values
                    cmax = max(cmax, max(max(__float_as_uint(nv[0]), __float_as_uint(nv[1])),
                                         max(__float_as_uint(nv[2]), __float_as_uint(nv[3]))));
#pragma unroll
                    for (int e = 0; e < 4; ++e) d[b][4 * m + e] = nv[e];
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x4 a[kBlocksPerChunk];
#pragma unroll
                for (int b = 0; b < kBlocksPerChunk; ++b)
                    a[b] = *reinterpret_cast<const f32x4 *>(sb + (b * 32 + col) * kRow + 32 * half + 4 * t);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int b = 0; b < kBlocksPerChunk; ++b)
                        d[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[b][e], r[4 * t + e], d[b], 0, 0, 0);
            }
            // Running best / second-best over this lane's scores. The index is
            // kept chunk-local (a compile-time constant per accumulator) and
            // folded into best_k once per chunk.
            auto update = [&](auto masked) {
                int loc = -1;
#pragma unroll
                for (int b = 0; b < kBlocksPerChunk; ++b) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        // accumulator v of this lane is codeword row 8*(v/4) + 4*half + v%4
                        const int lk = b * 32 + 8 * (v >> 2) + (v & 3);
                        float sc = d[b][v];
                        if (decltype(masked)::value && c * kChunk + lk + 4 * half >= n_codes) sc = INFINITY;
                        second = __builtin_amdgcn_fmed3f(sc, best, second);
                        const bool lt = sc < best;
                        loc = lt ? lk : loc;
                        best = lt ? sc : best;
                    }
                }
                if (loc >= 0) best_k = c * kChunk + 4 * half + loc;
            };
            if ((c + 1) * kChunk > n_codes)
                update(std::true_type{});
            else
                update(std::false_type{});
        }

        if (g + 1 < total) commit(buf ^ 1);

        if (c == n_chunks - 1) {
            // ---- stage q is scored for this wavefront's 32 frames: decide ----
            const float best_o = __shfl_xor(best, 32);
            const float second_o = __shfl_xor(second, 32);
            const int best_k_o = __shfl_xor(best_k, 32);
            const unsigned cmax_o = __shfl_xor(cmax, 32);
            float rn = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) rn = rn + r[j] * r[j];
            rn = rn + __shfl_xor(rn, 32);

            const float c2 = __uint_as_float(max(cmax, cmax_o));   // max_k 0.5*||c_k||^2
            const float bound = kSafety * kGamma * (c2 + sqrtf(rn) * sqrtf(2.0f * c2)) + kAbsSlack;
            const float m = fminf(best, best_o);
            const float lim = m + 2.0f * bound;
            const bool overflow = (second <= lim) || (second_o <= lim);
            const bool cand_me = best <= lim;
            const bool cand_o = best_o <= lim;
            int pick = cand_me ? best_k : best_k_o;

            // Two candidates, one per half: float64 re-rank.
            const bool rerank = valid && !overflow && cand_me && cand_o;
            if (__any(rerank)) {
                const int k_lo = half ? best_k_o : best_k;   // half 0's best
                const int k_hi = half ? best_k : best_k_o;   // half 1's best
                const float *ca = books + (static_cast<int64_t>(q) * n_codes + k_lo) * kDim + 32 * half;
                const float *cb = books + (static_cast<int64_t>(q) * n_codes + k_hi) * kDim + 32 * half;
                double sa = 0.0, sb = 0.0;
                if (half == 0) {          // dims 0..31, starting from zero
                    sa = sq_dist_part(0.0, r, ca);
                    sb = sq_dist_part(0.0, r, cb);
                }
                const double pa = __shfl_xor(sa, 32);
                const double pb = __shfl_xor(sb, 32);
                if (half == 1) {          // dims 32..63, continuing the same sum
                    sa = sq_dist_part(pa, r, ca);
                    sb = sq_dist_part(pb, r, cb);
                }
                // every lane runs both shuffles; half 0 takes half 1's finished sums
                const double xa = __shfl_xor(sa, 32);
                const double xb = __shfl_xor(sb, 32);
                const double fa = half ? sa : xa;
                const double fb = half ? sb : xb;
                const int winner = (fa < fb) ? k_lo : (fb < fa) ? k_hi : min(k_lo, k_hi);
                if (rerank) pick = winner;
            }

            // More than one candidate inside a lane: full float64 rescan.
            uint64_t pending = __ballot(valid && overflow && half == 0);
            while (pending) {
                const int f = __ffsll(static_cast<unsigned long long>(pending)) - 1;
                pending &= pending - 1;
                float rr[64];
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    rr[j] = __shfl(r[j], f);
                    rr[32 + j] = __shfl(r[j], f + 32);
                }
                double bd = INFINITY;
                int bk = 0x7fffffff;
                for (int k = lane; k < n_codes; k += 64) {
                    const float *cw = books + (static_cast<int64_t>(q) * n_codes + k) * kDim;
                    double s = 0.0;
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(cw + 4 * t);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const double dd = __dsub_rn(static_cast<double>(rr[4 * t + e]),
                                                        static_cast<double>(v[e]));
                            s = __dadd_rn(s, __dmul_rn(dd, dd));
                        }
                    }
                    if (s < bd) {
                        bd = s;
                        bk = k;
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
                if (col == f) pick = bk;
            }

            pick = min(max(pick, 0), n_codes - 1);
            if (valid && half == 0) codes[frame * codes_ld + q] = pick;
            const f32x4 *cw = reinterpret_cast<const f32x4 *>(
                books + (static_cast<int64_t>(q) * n_codes + pick) * kDim + 32 * half);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const f32x4 v = cw[t];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r[4 * t + e] = r[4 * t + e] - v[e];
                    if (kRecon) acc[4 * t + e] = acc[4 * t + e] + v[e];
                }
            }
            best = INFINITY;
            second = INFINITY;
            cmax = 0u;
            best_k = 0;
        }
        __syncthreads();
    }

    if (valid) {
        if (kResidual) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(residual + frame * kDim + 32 * half);
#pragma unroll
            for (int t = 0; t < 8; ++t) dst[t] = f32x4{r[4 * t], r[4 * t + 1], r[4 * t + 2], r[4 * t + 3]};
        }
        if (kRecon) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(recon + frame * kDim + 32 * half);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                dst[t] = f32x4{acc[4 * t], acc[4 * t + 1], acc[4 * t + 2], acc[4 * t + 3]};
        }
    }
}

}  // namespace

hipError_t launch_encode(const float *x, int64_t n_frames, const float *books,
                         int n_stages, int n_codes, int32_t *codes, int codes_ld,
                         float *residual, float *recon, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kEncodeFramesPerBlock - 1) / kEncodeFramesPerBlock;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    if (recon && residual)
        hipLaunchKernelGGL((encode_kernel<true, true>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (recon)
        hipLaunchKernelGGL((encode_kernel<true, false>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (residual)
        hipLaunchKernelGGL((encode_kernel<false, true>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    else
        hipLaunchKernelGGL((encode_kernel<false, false>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    return hipGetLastError();
}

}  // namespace rvq
