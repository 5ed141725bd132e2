// Fused multi-stage residual vector quantization encode for gfx950 (CDNA4)
// with split-bf16 scoring on the bf16 matrix cores.
//
// Computes the residual loop of the "RVQ codec" section of the
// "Architecture" page (omnivoice.cpp): for q = 0..Q-1 pick
// argmin_k ||r - C[q,k]||^2 (lowest k on ties), emit k, r <- r - C[q,k].
// The pick is the same as the fp32-scored kernel's (encode.hip): both end
// in the float64 direct form for every codeword that the fp32 or split-bf16
// scores cannot separate from the best. This kernel only scores faster:
// one v_mfma_f32_32x32x16_bf16 does the work of eight fp32 32x32x2 steps.
//
// Scoring: every fp32 value v is split as v = hi + lo + e with hi = bf16(v)
// and lo = bf16(v - hi) (round to nearest even; v - hi is exact in fp32),
// |e| <= 2^-16 |v|. The dot product n.c (n = -r) is computed as
//     n_hi.c_lo + n_lo.c_hi + n_hi.c_hi
// on the matrix cores (bf16 x bf16 products are exact in fp32), added to an
// accumulator that starts at 0.5*||c||^2 (fp32, from the fp32 codeword).
// The dropped terms n_lo.c_lo and the split remainders are at most
// 3.2 * 2^-16 * |n_j c_j| per dimension; the fp32 accumulation of 3D + 1
// terms plus the norm's own D-term sum adds at most 2*gamma_{3D+8} (2u per
// operation) of 0.5*||c||^2 + sum_j |n_j c_j|; the packed key adds 2^-17 of
// the score. So every key is within
//     e = (3.2 * 2^-16 + 2*gamma_{3D+8} + 2^-17) * (0.5*||c||^2 + ||r|| ||c||)
// of the exact score, and every codeword within 2*e_max of the smallest key
// is a candidate for the true argmin.
//
// Work split: 8 wavefronts x 32 frames per workgroup, residual in VGPRs
// (negated, plus its bf16 split), codebooks streamed through LDS in
// 256-codeword chunks (stored as hi/lo bf16, 8-dim groups; 140 KB double
// buffered, one workgroup per CU, two wavefronts per SIMD), each chunk
// scored as four 64-codeword groups of two interleaved MFMA chains. The
// larger chunk halves the barriers and per-wave staging per codeword
// against 4 wavefronts with 128-codeword chunks (7% faster at Q=32).
// Because candidate sets are wider than with fp32 scores, each lane keeps
// its best, second and third keys and the indices of the first two: a
// frame resolves from up to four candidates (two per half) with the float64
// re-rank, and only a third candidate inside one lane sends it to the full
// float64 rescan. This file holds the encodes of codebooks given as fp32
// (split in every workgroup) and the preparation of codebooks for the fp16
// kernels (encode_f16.hip), which take every prepared encode.
#include "encode_common.h"
#include "prepared.h"

namespace rvq {
namespace {

using namespace enc;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kFramesPerWave = 32;
constexpr int kBlockFrames = kWaves * kFramesPerWave;
constexpr int kChunk = 256;              // codewords per LDS chunk (4 groups of 64)
constexpr int kRowH = 2 * kDim + 8;      // bf16 per LDS row: 8 groups of (8 hi, 8 lo) + 16 B pad
constexpr float kSplitError = 3.2f * 1.52587890625e-05f;   // 3.2 * 2^-16
constexpr float kBoundScale = kSplitError + 2.0f * gamma_n(3 * kDim + 8) + kKeyError;

static_assert(kWaves * 32 == kChunk, "staging maps each wavefront to 32 codeword rows");

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// hi = bf16(v), lo = bf16(v - hi), both round to nearest even, converted in
// pairs (one v_cvt_pk_bf16_f32 per two values); hi is widened back to fp32 by
// placing its 16 bits at the top of a word, and v - hi is exact in fp32.
__device__ __forceinline__ void split8(const float *v, bf16x8 &hi, bf16x8 &lo)
{
    u32x4 hp, lp;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{v[2 * p], v[2 * p + 1]}, bf16x2));
        const float r0 = v[2 * p] - __uint_as_float(h << 16);
        const float r1 = v[2 * p + 1] - __uint_as_float(h & 0xFFFF0000u);
        hp[p] = h;
        lp[p] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
    }
    hi = __builtin_bit_cast(bf16x8, hp);
    lo = __builtin_bit_cast(bf16x8, lp);
}

// Key scan of a 64-codeword group (two blocks): running best, second and
// third key of this lane. Local index of accumulator v of block b:
// b*32 + 8*(v/4) + v%4, plus the lane's 4*half row offset.
__device__ __forceinline__ void scan_block(const f32x16 &d, int b, float &best, float &second, float &third)
{
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float key = make_key(d[v], b * 32 + 8 * (v >> 2) + (v & 3));
        third = __builtin_amdgcn_fmed3f(key, second, third);
        second = __builtin_amdgcn_fmed3f(key, best, second);
        best = __builtin_amdgcn_fmed3f(key, best, -FLT_MAX);
    }
}

__device__ __forceinline__ void scan_group(const f32x16 (&d)[2], float &best, float &second, float &third)
{
    scan_block(d[0], 0, best, second, third);
    scan_block(d[1], 1, best, second, third);
}

// Index bookkeeping after scanning the group that starts at codeword `base`.
// A changed second key is either the previous best (demoted) or a key of this
// group; equal bit patterns from different groups also leave a third key with
// the same value, which the decision treats as an unresolved candidate.
__device__ __forceinline__ void fold_group(float best, float second, unsigned best_before,
                                           unsigned second_before, int base, int half,
                                           int &best_k, int &second_k)
{
    const unsigned bb = __float_as_uint(best), sb = __float_as_uint(second);
    if (sb != second_before)
        second_k = (bb != best_before && sb == best_before) ? best_k
                                                            : base + 4 * half + static_cast<int>(sb & ~kKeyMask);
    if (bb != best_before) best_k = base + 4 * half + static_cast<int>(bb & ~kKeyMask);
}

// Scores codewords 64*kG .. 64*kG+63 of the chunk in LDS (two 32-codeword
// blocks, two interleaved MFMA chains of 12 steps) and folds them into this
// lane's best / second / third keys.
__device__ __forceinline__ void score_group(int kG, const __bf16 *sb, const float *sn, int col, int half,
                                            const bf16x8 (&nh)[4], const bf16x8 (&nl)[4], int base,
                                            float &best, float &second, float &third,
                                            int &best_k, int &second_k)
{
    f32x16 d[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 nv = *reinterpret_cast<const f32x4 *>(sn + kG * 64 + b * 32 + 8 * m + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) d[b][4 * m + e] = nv[e];
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8 ah[2], al[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const __bf16 *row = sb + (kG * 64 + b * 32 + col) * kRowH + 16 * (4 * half + s);
            ah[b] = *reinterpret_cast<const bf16x8 *>(row);
            al[b] = *reinterpret_cast<const bf16x8 *>(row + 8);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) d[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[b], nl[s], d[b], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b) d[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[b], nh[s], d[b], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b) d[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[b], nh[s], d[b], 0, 0, 0);
    }
    const unsigned bb = __float_as_uint(best), sb0 = __float_as_uint(second);
    scan_group(d, best, second, third);
    fold_group(best, second, bb, sb0, base, half, best_k, second_k);
}

using prep::padded_codes;
using prep::stage_bytes;

// An upper bound of sqrt(x) for x >= 0: the hardware square root (within a
// few ulp) of max(x, FLT_MIN), raised by 2^-20 of itself.
__device__ __forceinline__ float sqrt_up(float x)
{
    return __builtin_amdgcn_sqrtf(fmaxf(x, FLT_MIN)) * (1.0f + 9.5367431640625e-07f);
}

// The decision for one stage, from this lane's best / second / third keys
// and the indices of the first two (codeword slots of one half of a frame;
// lanes l and l^32 hold the two halves): every codeword within twice the
// error bound of the frame's smallest key is a candidate; two to four
// candidates are re-ranked in float64, a third candidate inside one lane
// (or ambiguous bookkeeping) sends the frame to the full float64 rescan.
// Then the pick is stored (code_out, when not null) and subtracted from the
// negated residual n (and added to acc for kRecon). Every lane must call it.
template <bool kRecon>
__device__ __forceinline__ void decide_stage(float (&n)[32], float (&acc)[32], float best, float second, float third,
                                             int best_k, int second_k, const float *book, int n_codes, float c2,
                                             bool valid, int half, int col, int lane, float *frame_row,
                                             int32_t *code_out)
{
    // Keys decode to real codewords whenever the frame's scores are finite;
    // a non-finite frame (its code is then unspecified) can decode padding
    // slots, so the indices are clamped before any row load.
    best_k = min(max(best_k, 0), n_codes - 1);
    second_k = min(max(second_k, 0), n_codes - 1);
    const float best_o = __shfl_xor(best, 32);
    const float second_o = __shfl_xor(second, 32);
    const float third_o = __shfl_xor(third, 32);
    const int best_k_o = __shfl_xor(best_k, 32);
    const int second_k_o = __shfl_xor(second_k, 32);
    float rn = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) rn = __builtin_fmaf(n[j], n[j], rn);
    rn = rn + __shfl_xor(rn, 32);

    const float bound = kBoundScale * (c2 + sqrt_up(rn) * sqrt_up(2.0f * c2)) + kAbsSlack;
    const float lim = fminf(best, best_o) + 2.0f * bound;
    const bool overflow = third <= lim || third_o <= lim ||
                          (second <= lim && second_k == best_k) ||
                          (second_o <= lim && second_k_o == best_k_o);
    // candidate slots in frame order: half 0's best and second, then half 1's
    const float sv[4] = {half ? best_o : best, half ? second_o : second,
                         half ? best : best_o, half ? second : second_o};
    const int sk[4] = {half ? best_k_o : best_k, half ? second_k_o : second_k,
                       half ? best_k : best_k_o, half ? second_k : second_k_o};
    bool cf[4];
    int ncand = 0, pick = sk[0];
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        cf[i] = sv[i] <= lim;
        ncand += cf[i];
        if (cf[i]) pick = sk[i];
    }

    // Two to four candidates: float64 re-rank (slot 0 is always a valid index).
    const bool rerank = valid && !overflow && ncand >= 2;
    if (__any(rerank)) {
        double bd = INFINITY;
        int bk = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool use = rerank && cf[i];
            if (__any(use)) {
                const int k = use ? sk[i] : sk[0];
                const double dist = pair_distance(n, book, k, half);
                if (use && (dist < bd || (dist == bd && k < bk))) {
                    bd = dist;
                    bk = k;
                }
            }
        }
        if (rerank) pick = bk;
    }

    // A third candidate inside one lane (or ambiguous bookkeeping): full rescan.
    uint64_t pending = __ballot(valid && overflow && half == 0);
    while (pending) {
        const int f = __ffsll(static_cast<unsigned long long>(pending)) - 1;
        pending &= pending - 1;
        const int w = rescan_frame(n, frame_row, book, n_codes, f, lane);
        if (col == f) pick = w;
    }

    pick = min(max(pick, 0), n_codes - 1);
    if (code_out) *code_out = pick;
    const f32x4 *cw = reinterpret_cast<const f32x4 *>(book + static_cast<int64_t>(pick) * kDim + 32 * half);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const f32x4 v = cw[t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            n[4 * t + e] = n[4 * t + e] + v[e];   // = -(r - c), exactly
            if (kRecon) acc[4 * t + e] = acc[4 * t + e] + v[e];
        }
    }
}

// Codebooks as given (fp32): every workgroup splits each chunk and sums its
// half-norms while staging it.
template <bool kRecon, bool kResidual>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void encode_bf16_kernel(const float *__restrict__ x, int64_t n_frames,
                        const float *__restrict__ books,
                        int n_stages, int n_codes,
                        int32_t *__restrict__ codes, int codes_ld,
                        float *__restrict__ residual, float *__restrict__ recon)
{
    __shared__ __align__(16) __bf16 s_book[2][kChunk * kRowH];
    __shared__ __align__(16) float s_norm[2][kChunk];
    __shared__ __align__(16) unsigned s_cmax[2][kWaves];   // per stage parity, per wavefront
    __shared__ __align__(16) float s_frame[kWaves][kDim];  // rescan: one frame's residual

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kBlockFrames +
                          wave * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    float n[32];     // negated residual, dims 32*half .. 32*half+31
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
    bf16x8 nh[4], nl[4];   // split of n: step s holds dims 32*half + 8s .. +7

    const int n_chunks = (n_codes + kChunk - 1) / kChunk;
    const int total = n_stages * n_chunks;

    // Staging: wavefront w stages rows 32w..32w+31, lane -> (row 32w + l%32, half l/32).
    const int srow = wave * 32 + col;
    f32x4 stage[8];
    bool stage_valid = false;
    unsigned stage_max = 0u;

    auto fetch = [&](int g) {
        const int q = g / n_chunks;
        const int c = g - q * n_chunks;
        const int k = c * kChunk + srow;
        if (c == 0) stage_max = 0u;
        // rows past n_codes load the last row again; their norm becomes kNoScore
        stage_valid = k < n_codes;
        const f32x4 *p = reinterpret_cast<const f32x4 *>(
            books + (static_cast<int64_t>(q) * n_codes + min(k, n_codes - 1)) * kDim + 32 * half);
#pragma unroll
        for (int i = 0; i < 8; ++i) stage[i] = p[i];
    };
    auto commit = [&](int g) {
        const int buf = g & 1;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_fmaf(stage[i][e], stage[i][e], s);
        s = s + __shfl_xor(s, 32);
        const float hn = 0.5f * s;
        __bf16 *dst = &s_book[buf][srow * kRowH];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = stage[2 * t][e];
                v[4 + e] = stage[2 * t + 1][e];
            }
            bf16x8 hi, lo;
            split8(v, hi, lo);
            const int grp = 4 * half + t;
            *reinterpret_cast<bf16x8 *>(dst + 16 * grp) = hi;
            *reinterpret_cast<bf16x8 *>(dst + 16 * grp + 8) = lo;
        }
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

    float best = kNoScore, second = kNoScore, third = kNoScore;
    int best_k = 0, second_k = 0;

    for (int g = 0; g < total; ++g) {
        const int buf = g & 1;
        const int q = g / n_chunks;
        const int c = g - q * n_chunks;
        if (g + 1 < total) fetch(g + 1);
        if (c == 0) {
#pragma unroll
            for (int s = 0; s < 4; ++s) split8(&n[8 * s], nh[s], nl[s]);
        }

        {
            const __bf16 *sb = s_book[buf];
            const float *sn = s_norm[buf];
            // a rolled loop keeps one group's operands live at a time (no spills)
#pragma unroll 1
            for (int gg = 0; gg < kChunk / 64; ++gg)
                score_group(gg, sb, sn, col, half, nh, nl, c * kChunk + 64 * gg, best, second, third, best_k,
                            second_k);
        }

        if (g + 1 < total) commit(g + 1);

        if (c == n_chunks - 1) {
            // ---- stage q is scored for this wavefront's 32 frames: decide ----
            const float *book = books + static_cast<int64_t>(q) * n_codes * kDim;
            unsigned m = 0u;   // max_k 0.5||c_k||^2 over the stage
#pragma unroll
            for (int w = 0; w < kWaves; ++w) m = max(m, s_cmax[q & 1][w]);
            const float c2 = __uint_as_float(m);
            decide_stage<kRecon>(n, acc, best, second, third, best_k, second_k, book, n_codes, c2, valid, half, col,
                                 lane, s_frame[wave], (valid && half == 0) ? codes + frame * codes_ld + q : nullptr);
            best = kNoScore;
            second = kNoScore;
            third = kNoScore;
            best_k = 0;
            second_k = 0;
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

// ---- small batches: the codebook split over the wavefronts ----------------
//
// With few frames the kernel above fills few workgroups, and each
// wavefront walks all K codewords of every stage alone. Here the 8
// wavefronts of a workgroup share one tile of 32 frames (each holds the
// tile's residual) and split every stage's codebook: wavefront w scores
// 64-codeword groups w, w + 8, ..., each staged into its own LDS buffer
// (no workgroup barrier while scoring). The per-lane best / second / third
// keys with the first two indices are then merged over the 8 wavefronts
// through LDS in a fixed order by wavefront 0, which takes the decision
// (decide_stage) on the residual it holds, writes the codes and publishes
// the bf16 split of the updated residual through LDS for the other
// wavefronts (which hold only the split); it writes the outputs at the end.
constexpr int kSplitWaves = 8;
constexpr int kSplitGroup = 64;
// up to this many frames the split kernel runs: two rounds of one-tile
// workgroups on 256 CUs are still faster than the wide kernel's 256-frame tiles
constexpr int64_t kSplitMaxFrames = 16384;

// top-3 of keys from disjoint codeword sets; k < 0 marks an unknown index,
// which orders after known ones on equal keys
struct Top3 {
    float b, s, t;
    int bk, sk;
};

__device__ __forceinline__ bool key_before(float v1, int k1, float v2, int k2)
{
    return v1 < v2 || (v1 == v2 && static_cast<unsigned>(k1) < static_cast<unsigned>(k2));
}

__device__ __forceinline__ void top3_insert(Top3 &m, float v, int k)
{
    if (key_before(v, k, m.b, m.bk)) {
        m.t = m.s;
        m.s = m.b;
        m.sk = m.bk;
        m.b = v;
        m.bk = k;
    } else if (key_before(v, k, m.s, m.sk)) {
        m.t = m.s;
        m.s = v;
        m.sk = k;
    } else {
        m.t = fminf(m.t, v);
    }
}

template <bool kRecon, bool kResidual>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kSplitWaves, 64 * kSplitWaves), amdgpu_waves_per_eu(2)))
void encode_bf16_ksplit_kernel(const float *__restrict__ x, int64_t n_frames,
                               const float *__restrict__ books, int n_stages, int n_codes,
                               int32_t *__restrict__ codes, int codes_ld,
                               float *__restrict__ residual, float *__restrict__ recon)
{
    __shared__ __align__(16) __bf16 s_rows[kSplitWaves][kSplitGroup * kRowH];
    __shared__ __align__(16) float s_gnorm[kSplitWaves][kSplitGroup];
    __shared__ __align__(16) float s_part[kSplitWaves][5][64];   // best, second, third, best_k, second_k
    __shared__ unsigned s_wmax[kSplitWaves];
    __shared__ __align__(16) float s_frame[kSplitWaves][kDim];
    __shared__ __align__(16) bf16x8 s_split[64][8];   // the tile's next-stage operand split, per lane

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    float n[32];
    float acc[32];
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
    bf16x8 nh[4], nl[4];

    const int n_groups = (n_codes + kSplitGroup - 1) / kSplitGroup;
    __bf16 *rows = s_rows[wave];
    float *gnorm = s_gnorm[wave];

#pragma unroll
    for (int s = 0; s < 4; ++s) split8(&n[8 * s], nh[s], nl[s]);

    for (int q = 0; q < n_stages; ++q) {
        if (q > 0 && wave != 0) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                nh[s] = s_split[lane][s];
                nl[s] = s_split[lane][4 + s];
            }
        }
        float best = kNoScore, second = kNoScore, third = kNoScore;
        int best_k = 0, second_k = 0;
        unsigned wmax = 0u;

        for (int g = wave; g < n_groups; g += kSplitWaves) {
            // lane l stages row 64 g + l of the stage (rows past n_codes:
            // the last row again with norm kNoScore)
            const int k = g * kSplitGroup + lane;
            __bf16 *dst = rows + lane * kRowH;
            const f32x4 *p = reinterpret_cast<const f32x4 *>(
                books + (static_cast<int64_t>(q) * n_codes + min(k, n_codes - 1)) * kDim);
            float hn = 0.0f;
#pragma unroll
            for (int grp = 0; grp < 8; ++grp) {
                const f32x4 a = p[2 * grp], b = p[2 * grp + 1];
                const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
                for (int e = 0; e < 8; ++e) hn = __builtin_fmaf(v[e], v[e], hn);
                bf16x8 hi, lo;
                split8(v, hi, lo);
                *reinterpret_cast<bf16x8 *>(dst + 16 * grp) = hi;
                *reinterpret_cast<bf16x8 *>(dst + 16 * grp + 8) = lo;
            }
            hn = 0.5f * hn;
            gnorm[lane] = k < n_codes ? hn : kNoScore;
            if (k < n_codes) wmax = max(wmax, __float_as_uint(hn));
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            score_group(0, rows, gnorm, col, half, nh, nl, g * kSplitGroup, best, second, third, best_k,
                        second_k);
            // the buffer is read before the next group overwrites it
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
        }

        s_part[wave][0][lane] = best;
        s_part[wave][1][lane] = second;
        s_part[wave][2][lane] = third;
        s_part[wave][3][lane] = __int_as_float(best_k);
        s_part[wave][4][lane] = __int_as_float(second_k);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1)
            wmax = max(wmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(wmax), off)));
        if (lane == 0) s_wmax[wave] = wmax;
        __syncthreads();
        if (wave == 0) {
            // wavefront 0 merges the parts, decides, and publishes the split
            // of the updated residual for the other wavefronts
            Top3 m = {kNoScore, kNoScore, kNoScore, 0, 0};   // the scan's own initial state
#pragma unroll
            for (int w = 0; w < kSplitWaves; ++w) {
                top3_insert(m, s_part[w][0][lane], __float_as_int(s_part[w][3][lane]));
                top3_insert(m, s_part[w][1][lane], __float_as_int(s_part[w][4][lane]));
                top3_insert(m, s_part[w][2][lane], -1);
            }
            unsigned mm = 0u;
#pragma unroll
            for (int w = 0; w < kSplitWaves; ++w) mm = max(mm, s_wmax[w]);
            const float c2 = __uint_as_float(mm);   // max_k 0.5||c_k||^2 over the stage
            const float *book = books + static_cast<int64_t>(q) * n_codes * kDim;
            decide_stage<kRecon>(n, acc, m.b, m.s, m.t, m.bk, m.sk, book, n_codes, c2, valid, half, col, lane,
                                 s_frame[0], (valid && half == 0) ? codes + frame * codes_ld + q : nullptr);
            if (q + 1 < n_stages) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    split8(&n[8 * s], nh[s], nl[s]);
                    s_split[lane][s] = nh[s];
                    s_split[lane][4 + s] = nl[s];
                }
            }
        }
        __syncthreads();   // the split is published; s_part and s_wmax are free again
    }

    if (wave == 0 && valid) {
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

// One workgroup per kChunk padded rows of a stage, 8 lanes per row (one
// 8-dim group each, so a wavefront reads and writes 8 whole rows). Every
// workgroup first finds the stage's largest |c| itself, so all of a stage's
// workgroups reach the same scale e. Then per row: fp16 of c' = 2^e c and
// the fp16 parts of 0.5*||c'||^2; and the largest valid half-norm of the
// workgroup's rows.
constexpr int kPrepThreads = 512;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ unsigned block_max_bits(unsigned m, unsigned *s_m)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), off)));
    __syncthreads();   // s_m is free (a previous call's readers are done)
    if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
    __syncthreads();
    unsigned mm = 0u;
#pragma unroll
    for (int w = 0; w < kPrepThreads / 64; ++w) mm = max(mm, s_m[w]);
    return mm;
}

__global__ __launch_bounds__(kPrepThreads)
void prepare_kernel(const float *__restrict__ books, int n_codes, uint8_t *__restrict__ prepared)
{
    __shared__ unsigned s_m[kPrepThreads / 64];
    const int c = blockIdx.x;
    const int q = blockIdx.y;
    const int64_t kp = padded_codes(n_codes);
    uint8_t *blk = prepared + q * stage_bytes(n_codes);
    const float *stage = books + static_cast<int64_t>(q) * n_codes * kDim;

    // the stage's largest |c|: bits of non-negative floats order like the
    // values, and a NaN's bits lie above those of +inf
    unsigned a = 0u;
    {
        const f32x4 *sv = reinterpret_cast<const f32x4 *>(stage);
        const int64_t n4 = static_cast<int64_t>(n_codes) * (kDim / 4);
#pragma unroll 4
        for (int64_t i = threadIdx.x; i < n4; i += kPrepThreads) {
            const f32x4 v = sv[i];
#pragma unroll
            for (int t = 0; t < 4; ++t) a = max(a, __float_as_uint(fabsf(v[t])));
        }
    }
    const unsigned amax_bits = block_max_bits(a, s_m);
    const float amax = __uint_as_float(amax_bits);
    int e = 0;
    if (amax_bits != 0u && amax_bits < 0x7F800000u) {
        int x;
        (void)frexpf(amax, &x);   // amax = f * 2^x, f in [1/2, 1)
        e = min(max(-x, prep::kMinExp), prep::kMaxExp);
    }
    const bool in_range = amax_bits < 0x7F800000u && ldexpf(amax, e) <= prep::kMaxScaled;

    const int grp = threadIdx.x & 7;
    unsigned m16 = 0u;
    for (int k = c * kChunk + (threadIdx.x >> 3); k < (c + 1) * kChunk; k += kPrepThreads / 8) {
        u32x4 *row16 = reinterpret_cast<u32x4 *>(blk + static_cast<int64_t>(k) * prep::kF16Row);
        if (k >= n_codes) {   // the 8 lanes of a row take the same branch
            row16[grp] = u32x4{0u, 0u, 0u, 0u};
            if (grp == 0) row16[8] = u32x4{0u, 0u, 0u, 0u};
            continue;
        }
        const f32x4 *src = reinterpret_cast<const f32x4 *>(stage + static_cast<int64_t>(k) * kDim + 8 * grp);
        const f32x4 va = src[0], vb = src[1];
        const float v[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
        float s16 = 0.0f;
        f16x8 h16;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float w = ldexpf(v[t], e);   // exact unless it falls below the fp32 normal range
            s16 = __builtin_fmaf(w, w, s16);
            h16[t] = static_cast<_Float16>(w);   // round to nearest even
        }
        row16[grp] = __builtin_bit_cast(u32x4, h16);
        s16 += __shfl_xor(s16, 1);
        s16 += __shfl_xor(s16, 2);
        s16 += __shfl_xor(s16, 4);
        const float hn16 = 0.5f * s16;
        if (grp == 0) {
            // two fp16 parts: hn16 - hi is exact in fp32
            const _Float16 p_hi = static_cast<_Float16>(hn16);
            const _Float16 p_lo = static_cast<_Float16>(hn16 - static_cast<float>(p_hi));
            row16[8] = u32x4{static_cast<unsigned>(__builtin_bit_cast(unsigned short, p_hi)) |
                                 (static_cast<unsigned>(__builtin_bit_cast(unsigned short, p_lo)) << 16),
                             0u, 0u, 0u};
        }
        m16 = max(m16, __float_as_uint(hn16));   // hn16 >= 0: bits order like values
    }
    const unsigned mm16 = block_max_bits(m16, s_m);
    if (threadIdx.x == 0) {
        reinterpret_cast<unsigned *>(blk + prep::f16_max(kp))[c] = in_range ? mm16 : 0x7F800000u;
        if (c == 0) *reinterpret_cast<int *>(blk + prep::f16_exp(kp)) = e;
    }
}

}  // namespace

int64_t prepared_bytes(int n_stages, int n_codes) { return stage_bytes(n_codes) * n_stages; }

hipError_t launch_prepare(const float *books, int n_stages, int n_codes, void *prepared, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(padded_codes(n_codes) / kChunk), static_cast<unsigned>(n_stages));
    hipLaunchKernelGGL(prepare_kernel, grid, dim3(kPrepThreads), 0, stream, books, n_codes,
                       static_cast<uint8_t *>(prepared));
    return hipGetLastError();
}

hipError_t launch_encode_bf16(const float *x, int64_t n_frames, const float *books,
                              int n_stages, int n_codes, int32_t *codes, int codes_ld,
                              float *residual, float *recon, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kBlockFrames - 1) / kBlockFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (n_frames <= kSplitMaxFrames) {
        // few frames: one 32-frame tile per workgroup, the codebook split over its wavefronts
        const dim3 sgrid(static_cast<unsigned>((n_frames + kFramesPerWave - 1) / kFramesPerWave));
        const dim3 sblock(64 * kSplitWaves);
        if (recon && residual)
            hipLaunchKernelGGL((encode_bf16_ksplit_kernel<true, true>), sgrid, sblock, 0, stream,
                               x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
        else if (recon)
            hipLaunchKernelGGL((encode_bf16_ksplit_kernel<true, false>), sgrid, sblock, 0, stream,
                               x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
        else if (residual)
            hipLaunchKernelGGL((encode_bf16_ksplit_kernel<false, true>), sgrid, sblock, 0, stream,
                               x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
        else
            hipLaunchKernelGGL((encode_bf16_ksplit_kernel<false, false>), sgrid, sblock, 0, stream,
                               x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    if (recon && residual)
        hipLaunchKernelGGL((encode_bf16_kernel<true, true>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (recon)
        hipLaunchKernelGGL((encode_bf16_kernel<true, false>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (residual)
        hipLaunchKernelGGL((encode_bf16_kernel<false, true>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    else
        hipLaunchKernelGGL((encode_bf16_kernel<false, false>), grid, block, 0, stream,
                           x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon);
    return hipGetLastError();
}

}  // namespace rvq
