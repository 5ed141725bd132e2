// Fused multi-stage residual vector quantization encode for gfx950 (CDNA4).
//
// Computes the residual loop of the "RVQ codec" section of the
// "Architecture" page (omnivoice.cpp): for q = 0..Q-1 pick
// argmin_k ||r - C[q,k]||^2 (lowest k on ties), emit k, r <- r - C[q,k].
//
// Work split
//   * One workgroup = 4 wavefronts = 128 frames; a wavefront owns 32 frames
//     for all Q stages, so a frame's argmin never leaves its wavefront.
//   * Residuals stay in VGPRs for the whole call, stored negated (n = -r) so
//     that the matrix product yields -r.c directly. Lane l holds frame l%32;
//     lanes 0-31 keep dims 0..31, lanes 32-63 keep dims 32..63.
//   * Codebooks stream through LDS in chunks of 128 codewords (double
//     buffered, one barrier per chunk). The staging threads compute
//     0.5*||c||^2 of each row and, once per stage, the largest of them.
//   * Scores on fp32 matrix cores: v_mfma_f32_32x32x2_f32 with codewords on
//     the M (row) side and frames on the N (column) side, accumulator
//     initialised with 0.5*||c||^2, so one 32-step chain yields
//         s_k = 0.5*||c_k||^2 - r.c_k  (= 0.5*(||r - c_k||^2 - ||r||^2)).
//     In the 32x32 output each lane holds 16 scores of one frame; the other
//     16 of that frame sit in lane l^32.
//   * Per lane: running minimum and second minimum of packed keys. A key is
//     the score with its 6 low mantissa bits replaced by the codeword's
//     index inside its 64-codeword pair of blocks, so one float min tracks
//     value and index.
//     On gfx950 ordinary VALU work does not overlap fp32 MFMA execution, so
//     the scan is kept to three VALU operations per score.
//
// Exactness
//   The key of codeword k differs from the exact score by at most
//       e = (2 * gamma_{2D+4} + 2^-17) * (0.5*||c_k||^2 + ||r||*||c_k||)
//   (norm and dot product summed in fp32 in any order with at most 2u error
//   per operation, plus the 6 bits the index replaces). Every codeword whose key lies within 2*e_max of the
//   smallest key is a candidate for the true argmin, and nothing else can
//   be. One candidate is the answer; two candidates (the two lane minima of
//   the frame) are re-ranked with the float64 direct-form distance
//   sum_j (r_j - c_j)^2, j ascending, one rounding per operation; a lane
//   holding more than one candidate triggers a wavefront rescan of all K
//   codewords of that frame with the same float64 sum. The pick is
//   therefore the argmin of that float64 distance (lowest index on ties),
//   independent of the fp32 rounding order.
#include "encode_common.h"

namespace rvq {
namespace {

using namespace enc;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kFramesPerWave = 32;
constexpr int kChunk = 128;         // codewords per LDS chunk
constexpr int kRow = kDim + 4;      // padded LDS row (floats): 8 lanes of a b128 read hit 32 banks

static_assert(kThreads == kEncodeThreads, "thread count");
static_assert(kWaves * kFramesPerWave == kEncodeFramesPerBlock, "frames per block");
static_assert(kWaves * 32 == kChunk, "staging maps each wavefront to 32 codeword rows");

// A score is a D+1 term sum (norm plus D products, each product rounded)
// started from a norm that is itself a D-term fp32 sum: 2D + 4 roundings
// cover both.
constexpr float kGamma = gamma_n(2 * kDim + 4);
// Margin for matrix-core rounding that is not round-to-nearest: an error
// of up to 2u per operation (truncation) is still covered.
constexpr float kSafety = 2.0f;
constexpr float kBoundScale = kSafety * kGamma + kKeyError;

// Key scan of accumulators v0, v0+1 of both blocks of a pair. The
// pair-local codeword index of accumulator v of block b is
// b*32 + 8*(v/4) + v%4 (at most 59, an inline constant), plus this lane's
// 4*half row offset, added when the index is decoded.
template <int kV0>
__device__ __forceinline__ void scan_piece(const f32x16 (&d)[2], float &best, float &second)
{
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int v = kV0; v < kV0 + 2; ++v) {
            const float key = make_key(d[b][v], b * 32 + 8 * (v >> 2) + (v & 3));
            second = __builtin_amdgcn_fmed3f(key, best, second);
            best = __builtin_amdgcn_fmed3f(key, best, -FLT_MAX);   // min(key, best), no canonicalize
        }
    }
}

// Accumulators of a pair of 32-codeword blocks start at 0.5*||c||^2 of
// their rows (kNoScore for rows past n_codes).
__device__ __forceinline__ void init_pair(f32x16 (&d)[2], const float *sn, int pair, int half)
{
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 nv = *reinterpret_cast<const f32x4 *>(sn + pair * 64 + b * 32 + 8 * m + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) d[b][4 * m + e] = nv[e];
        }
    }
}

// Step t (dims 4t..4t+3 of this lane's half) of a pair's two MFMA chains,
// plus piece t of the previous pair's key scan.
template <int kPair, int kT>
__device__ __forceinline__ void pair_step(f32x16 (&d)[2], const f32x16 (&prev)[2], const float *sb,
                                          int col, int half, const float (&n)[32],
                                          float &best, float &second)
{
    f32x4 a[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
        a[b] = *reinterpret_cast<const f32x4 *>(sb + (kPair * 64 + b * 32 + col) * kRow + 32 * half + 4 * kT);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
            d[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[b][e], n[4 * kT + e], d[b], 0, 0, 0);
    }
    scan_piece<2 * kT>(prev, best, second);
}

template <int kPair>
__device__ __forceinline__ void pair_pass(f32x16 (&d)[2], const f32x16 (&prev)[2], const float *sb,
                                          const float *sn, int col, int half, const float (&n)[32],
                                          float &best, float &second)
{
    init_pair(d, sn, kPair, half);
    pair_step<kPair, 0>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 1>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 2>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 3>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 4>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 5>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 6>(d, prev, sb, col, half, n, best, second);
    pair_step<kPair, 7>(d, prev, sb, col, half, n, best, second);
}

// If `best` changed since `before`, its low bits name a codeword of the
// pair of blocks that starts at codeword `base`.
__device__ __forceinline__ void fold_index(float best, unsigned before, int base, int half, int &best_k)
{
    const unsigned bits = __float_as_uint(best);
    if (bits != before) best_k = base + 4 * half + static_cast<int>(bits & ~kKeyMask);
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
    __shared__ __align__(16) unsigned s_cmax[2][kWaves];   // per stage parity, per wavefront
    __shared__ __align__(16) float s_frame[kWaves][kDim];  // rescan: one frame's residual

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kEncodeFramesPerBlock +
                          wave * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    float n[32];     // negated residual
    float acc[32];   // reconstruction (kRecon)
    if (valid) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(x + frame * kDim + 32 * half);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 v = src[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) n[4 * t + e] = -v[e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) n[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.0f;

    const int n_chunks = (n_codes + kChunk - 1) / kChunk;
    const int total = n_stages * n_chunks;

    // Staging role: wavefront w stages rows 32w..32w+31; lane l takes row
    // 32w + l%32 and its half l/32, so 8 consecutive lanes write 8 rows of
    // the same half (row stride 68 floats: distinct LDS banks).
    const int srow = wave * 32 + col;
    const int scol = half * 32;
    f32x4 stage[8];
    bool stage_valid = false;
    unsigned stage_max = 0u;   // bits of the largest valid 0.5*||c||^2 staged in this stage

    auto fetch = [&](int g) {
        const int q = g / n_chunks;
        const int c = g - q * n_chunks;
        const int k = c * kChunk + srow;
        if (c == 0) stage_max = 0u;
        // Rows past n_codes load the last row again; their norm is replaced
        // by kNoScore on commit, so their scores never win.
        stage_valid = k < n_codes;
        const f32x4 *p = reinterpret_cast<const f32x4 *>(
            books + (static_cast<int64_t>(q) * n_codes + min(k, n_codes - 1)) * kDim + scol);
#pragma unroll
        for (int i = 0; i < 8; ++i) stage[i] = p[i];
    };
    // Writes chunk g's rows and 0.5*||c||^2 into buffer g&1. After the last
    // chunk of a stage, publishes each wavefront's largest half-norm of the
    // stage in s_cmax[stage & 1].
    auto commit = [&](int g) {
        const int buf = g & 1;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_fmaf(stage[i][e], stage[i][e], s);
        s = s + __shfl_xor(s, 32);
        const float hn = 0.5f * s;
        float *dst = &s_book[buf][srow * kRow + scol];
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4 *>(dst + 4 * i) = stage[i];
        if (half == 0) s_norm[buf][srow] = stage_valid ? hn : kNoScore;
        if (stage_valid) stage_max = max(stage_max, __float_as_uint(hn));   // hn >= 0: bits order like values
        const int q = g / n_chunks;
        if (g - q * n_chunks == n_chunks - 1) {
            unsigned m = stage_max;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1)
                m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), off)));
            if (lane == 0) s_cmax[q & 1][wave] = m;
        }
    };

    fetch(0);
    commit(0);
    __syncthreads();

    float best = kNoScore, second = kNoScore;
    int best_k = 0;
    f32x16 dA[2], dB[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) dB[b][v] = kNoScore;

    for (int g = 0; g < total; ++g) {
        const int buf = g & 1;
        const int q = g / n_chunks;
        const int c = g - q * n_chunks;
        if (g + 1 < total) fetch(g + 1);

        const float *sb = s_book[buf];
        const float *sn = s_norm[buf];
        // Pair 0 of this chunk on the matrix cores; the key scan of the
        // previous chunk's pair 1 (all kNoScore at a stage start) rides along.
        unsigned before = __float_as_uint(best);
        pair_pass<0>(dA, dB, sb, sn, col, half, n, best, second);
        fold_index(best, before, (c - 1) * kChunk + 64, half, best_k);
        // Pair 1 on the matrix cores, scan of pair 0.
        before = __float_as_uint(best);
        pair_pass<1>(dB, dA, sb, sn, col, half, n, best, second);
        fold_index(best, before, c * kChunk, half, best_k);

        if (g + 1 < total) commit(g + 1);

        if (c == n_chunks - 1) {
            // Drain: scan the stage's last pair, then mark it consumed.
            before = __float_as_uint(best);
            scan_piece<0>(dB, best, second);
            scan_piece<2>(dB, best, second);
            scan_piece<4>(dB, best, second);
            scan_piece<6>(dB, best, second);
            scan_piece<8>(dB, best, second);
            scan_piece<10>(dB, best, second);
            scan_piece<12>(dB, best, second);
            scan_piece<14>(dB, best, second);
            fold_index(best, before, c * kChunk + 64, half, best_k);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) dB[b][v] = kNoScore;

            // ---- stage q is scored for this wavefront's 32 frames: decide ----
            // A key decodes to a real codeword whenever the frame's scores are
            // finite; a non-finite frame (its code is then unspecified) can
            // decode a padding slot, so the index is clamped before any row load.
            best_k = min(max(best_k, 0), n_codes - 1);
            const float best_o = __shfl_xor(best, 32);
            const float second_o = __shfl_xor(second, 32);
            const int best_k_o = __shfl_xor(best_k, 32);
            float rn = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) rn = __builtin_fmaf(n[j], n[j], rn);
            rn = rn + __shfl_xor(rn, 32);

            const uint4 cm = *reinterpret_cast<const uint4 *>(s_cmax[q & 1]);
            const float c2 = __uint_as_float(max(max(cm.x, cm.y), max(cm.z, cm.w)));   // max_k 0.5||c_k||^2
            const float bound = kBoundScale * (c2 + sqrtf(rn) * sqrtf(2.0f * c2)) + kAbsSlack;
            const float m = fminf(best, best_o);
            const float lim = m + 2.0f * bound;
            const bool overflow = (second <= lim) || (second_o <= lim);
            const bool cand_me = best <= lim;
            const bool cand_o = best_o <= lim;
            const int k_lo = half ? best_k_o : best_k;   // half 0's best
            const int k_hi = half ? best_k : best_k_o;   // half 1's best
            // the same choice on both lanes of the frame, also when no key is a
            // candidate (non-finite scores)
            int pick = (half ? cand_o : cand_me) ? k_lo : k_hi;

            // Two candidates, one per half: float64 re-rank.
            const bool rerank = valid && !overflow && cand_me && cand_o;
            if (__any(rerank)) {
                const float *ca = books + (static_cast<int64_t>(q) * n_codes + k_lo) * kDim + 32 * half;
                const float *cb = books + (static_cast<int64_t>(q) * n_codes + k_hi) * kDim + 32 * half;
                double sa = 0.0, sb2 = 0.0;
                if (half == 0) {          // dims 0..31, starting from zero
                    sa = sq_dist_part(0.0, n, ca);
                    sb2 = sq_dist_part(0.0, n, cb);
                }
                const double pa = __shfl_xor(sa, 32);
                const double pb = __shfl_xor(sb2, 32);
                if (half == 1) {          // dims 32..63, continuing the same sum
                    sa = sq_dist_part(pa, n, ca);
                    sb2 = sq_dist_part(pb, n, cb);
                }
                // every lane runs both shuffles; half 0 takes half 1's finished sums
                const double xa = __shfl_xor(sa, 32);
                const double xb = __shfl_xor(sb2, 32);
                const double fa = half ? sa : xa;
                const double fb = half ? sb2 : xb;
                const int winner = (fa < fb) ? k_lo : (fb < fa) ? k_hi : min(k_lo, k_hi);
                if (rerank) pick = winner;
            }

            // More than one candidate inside a lane: full float64 rescan of the
            // frame by the whole wavefront, two codewords per lane at a time.
            uint64_t pending = __ballot(valid && overflow && half == 0);
            while (pending) {
                const int f = __ffsll(static_cast<unsigned long long>(pending)) - 1;
                pending &= pending - 1;
                const int w = rescan_frame(n, s_frame[wave], books + static_cast<int64_t>(q) * n_codes * kDim,
                                           n_codes, f, lane);
                if (col == f) pick = w;
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
                    n[4 * t + e] = n[4 * t + e] + v[e];   // = -(r - c), exactly
                    if (kRecon) acc[4 * t + e] = acc[4 * t + e] + v[e];
                }
            }
            best = kNoScore;
            second = kNoScore;
            best_k = 0;
        }
        __syncthreads();
    }

    if (valid) {
        if (kResidual) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(residual + frame * kDim + 32 * half);
#pragma unroll
            for (int t = 0; t < 8; ++t) dst[t] = f32x4{-n[4 * t], -n[4 * t + 1], -n[4 * t + 2], -n[4 * t + 3]};
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
