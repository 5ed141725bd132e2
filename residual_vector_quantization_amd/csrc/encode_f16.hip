// Fused multi-stage residual vector quantization encode for gfx950 (CDNA4)
// that scores with one fp16 product per dimension on the matrix cores and
// decides every stage exactly.
//
// Computes the residual loop of the "RVQ codec" section of the
// "Architecture" page (omnivoice.cpp): for q = 0..Q-1 pick
// argmin_k ||r - C[q,k]||^2 (lowest k on ties), emit k, r <- r - C[q,k].
// The picks, residuals and reconstructions are those of the other encode
// kernels: a pick is made from fast scores only when no other codeword can
// be within the scores' proven error of it, and otherwise by the float64
// direct form that the oracle uses.
//
// Scores: with a per-stage power of two 2^e that brings the stage's
// largest |c| into [1/2, 1), c' = 2^e c, n = -r and the key
//     s'_k = 2^-e * 0.5*||c'_k||^2 + n . c'_k  =  2^e * (0.5*||c_k||^2 - r . c_k)
// orders the codewords like the distance. One v_mfma_f32_32x32x16_f16 per
// 16 dims multiplies fp16(n_j) by fp16(c'_j) (exact products in fp32), and
// a fifth step adds the half-norm: its two fp16 parts times 2^-e. With
// u = 2^-11 (fp16 rounding), the stage maxima T = 2^-e max 0.5*||c'||^2
// and C = max ||c'||, every key is within
//     E = (2u + u^2 + 2 gamma_{D+8} + 2^-15 + u^2 + gamma_64) (T + ||n|| C)
//         + 2^-21 ||n|| + 2^-22 C + 2^-(e+25) + 2^-43                 (1)
// of the exact scaled score: the products lose at most (2u + u^2)|n_j c'_j|
// plus 2^-24 |n_j| + 2^-25 |c'_j| in the fp16 subnormal range (D = 64
// dims, so the 1-norms are at most 8 times the 2-norms); the half-norm's
// fp32 sum and its two fp16 parts lose gamma_64 + u^2 of it plus 2^-25;
// the fp32 accumulation 2 gamma_{D+8} and the packed key 2^-15 of the sum.
// Every codeword whose key is within 2E of the frame's smallest key is a
// candidate for the true argmin. fp16 keeps its range only while every
// |n_j| < 2^15: a frame whose residual leaves that range, or a stage whose
// codebook does (marked by an infinite maximum when it was prepared), goes
// to the full float64 rescan instead.
//
// The fp16 scores are about 20 times coarser than split-bf16 ones, so
// candidate sets are wider: each lane keeps two sets of keys (even and odd
// 64-codeword groups), best and second key, a lower bound of the third, and
// the indices of the first two, updated two scores at a time (five
// instructions per pair besides the keys). A key carries the codeword's
// index inside a span of 1024 codewords, so index bookkeeping runs once per
// span and set instead of once per group. The smallest key's codeword is fetched as the decision
// starts (it is the pick of a frame with one candidate, and serves the
// update); two to eight candidates (two per set and lane) are compared by
// a float32 direct form, and only near ties by the float64 one; a third
// candidate inside a set makes the wavefront sweep that set's K/4
// codewords with the other sets' candidates, float32 first and float64 for
// near ties.
//
// Work split: 4 wavefronts x 32 frames per workgroup and two workgroups per
// CU (74.8 KB of LDS each), residual in VGPRs, prepared fp16 rows (64 dims
// and the half-norm parts, 144 bytes) copied straight into LDS in
// 256-codeword chunks (double buffered), each chunk scored as four
// 64-codeword groups of two interleaved matrix-core chains, with the key
// scan of one group issued between the matrix-core steps of the next.
// Batches too small to fill the CUs that way (up to 8,192 frames) take a
// second kernel, at the end of this file, that splits every stage's
// codebook over the wavefronts of a workgroup instead.
#include "encode_common.h"
#include "prepared.h"

namespace rvq {
namespace {

using namespace enc;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kFramesPerWave = 32;
constexpr int kBlockFrames = kWaves * kFramesPerWave;
constexpr int kChunk = prep::kChunk;                         // codewords per LDS chunk (4 groups of 64)
constexpr int kGroups = kChunk / 64;
constexpr int kRowSlots = 9;                                 // 16-byte slots per row: 8 of dims, 1 of half-norm
constexpr int kRowHalfs = 8 * kRowSlots;                     // fp16 per LDS row
constexpr int kWaveRows = kChunk / kWaves;                   // rows each wavefront copies per chunk
constexpr int kWaveLoads = kWaveRows * kRowSlots / 64;       // wavefront-wide row copies per chunk
static_assert(kWaveRows * kRowSlots % 64 == 0, "whole wavefront-wide copies");
static_assert(kGroups == 4, "two group pairs per chunk");
static_assert(prep::kF16Row == 16 * kRowSlots, "LDS rows mirror the prepared rows");

// Relative and absolute coefficients of (1), rounded up.
constexpr float kRel = 1.021e-3f;      // 2u + u^2 + 2 gamma_72 + 2^-15 + u^2 + gamma_64 = 1.01996e-3
constexpr float kAbsN = 4.8e-7f;       // 2^-21 (1 + u) with the accumulation factor
constexpr float kAbsC = 2.4e-7f;       // 2^-22 (1 + u) with the accumulation factor
constexpr float kAbsNorm = 3.0e-8f;    // 2^-25, times 2^-e
constexpr float kAbsConst = 1.2e-13f;  // 64 * 2^-49

// One wavefront-wide direct load from global memory into LDS: active lane i
// copies 16 bytes from src into dst + 16 i (dst wave-uniform, in LDS).
// Issued as inline assembly so that the compiler does not order every LDS
// read behind it; the caller waits with the vector-memory counter.
__device__ __forceinline__ void dma16(const void *src, void *dst)
{
    const unsigned m0 = static_cast<unsigned>(reinterpret_cast<size_t>((lds_void *)dst));
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// fp16 (round to nearest even) of 8 consecutive floats, one v_cvt_pk_f16_f32 per pair.
__device__ __forceinline__ f16x8 to_f16x8(const float *v)
{
    f16x8 h;
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = static_cast<_Float16>(v[t]);
    return h;
}

// Keys of this kernel: a score with its 8 low mantissa bits replaced by the
// codeword's index inside a span of 1024 codewords of one key set and lane
// half (256 codewords), which moves the value by less than 2^-15 of it. The
// index bits of the score v (0..31, block v >> 4, accumulator v & 15) of the
// group that starts at codeword g (a multiple of 64) are
//   ((g >> 8) & 3) << 6  |  ((g >> 7) & 1) << 5  |  v
// (chunk within the span, group pair within the chunk, score), and the
// codeword is
//   span + 64 * set + 4 * half + ((bits & 0xE0) << 2) + ((bits & 0x1C) << 1) + (bits & 3).
constexpr int kSpan = 1024;              // codewords whose keys share one index space
constexpr unsigned kKeyMask8 = 0xFFFFFF00u;

// Index bits of the group starting at codeword g, before the score's own 5.
__device__ __forceinline__ int group_bits(int g) { return (g >> 2) & 0xE0; }

// base | c as an opaque scalar register (c a small constant), so that the key
// of each score is one v_and_or_b32 with the mask in a vector register.
__device__ __forceinline__ int sgpr_or(int base, int c)
{
    int r;
    asm("s_or_b32 %0, %1, %2" : "=s"(r) : "s"(base), "i"(c));
    return r;
}

__device__ __forceinline__ float key8(float s, unsigned mask, int bits)
{
    return __uint_as_float((__float_as_uint(s) & mask) | static_cast<unsigned>(bits));
}

// Running best and second key of one set, the indices of both, and a lower
// bound of the third smallest key (exact in all but rare orders).
struct KeySet {
    float best, second, third;
    int best_k, second_k;
};

__device__ __forceinline__ void reset(KeySet &s)
{
    s.best = s.second = s.third = kNoScore;
    s.best_k = s.second_k = 0;
}

// Keys a, b of scores v and v+1 (same block) into set s. With the old best
// B <= second S, the two smallest keys of {B, S, a, b} are min(B, a, b) and
// min(S, med3(B, a, b)); and med3(S, a, b), the second smallest of the same
// keys without B, is at most their third smallest, so third <- min(third,
// med3(S, a, b)) keeps a lower bound of the third smallest key seen (equal
// to it unless both a and b fall below B; a lower bound is all the decision
// needs to find a set that may hold a third candidate). Five instructions
// per two scores besides the keys, with consecutive second and third
// updates merged into v_min3 by the compiler.
__device__ __forceinline__ void scan_pair(const f32x16 (&d)[2], int v, int gbits, unsigned mask, KeySet &s)
{
    const int b = v >> 4, a = v & 15;
    const float k0 = key8(d[b][a], mask, sgpr_or(gbits, v));
    const float k1 = key8(d[b][a + 1], mask, sgpr_or(gbits, v + 1));
    const float t = __builtin_amdgcn_fmed3f(s.best, k0, k1);
    const float u = __builtin_amdgcn_fmed3f(s.second, k0, k1);
    s.best = __builtin_fminf(__builtin_fminf(s.best, k0), k1);
    s.second = __builtin_fminf(s.second, t);
    s.third = __builtin_fminf(s.third, u);
}

// Index bookkeeping of set `set` after the span that starts at codeword
// `span` (best / second bits before it: bb0, sb0). A changed second key is
// either the previous best (demoted) or a key of this span; equal bit
// patterns from different spans leave a second key equal to the best, which
// the decision treats as an unresolved candidate.
__device__ __forceinline__ void fold(KeySet &s, unsigned bb0, unsigned sb0, int span, int set, int half)
{
    const unsigned bb = __float_as_uint(s.best), sbits = __float_as_uint(s.second);
    const int base = span + 64 * set + 4 * half;
    const int k_of_best = base + static_cast<int>(((bb & 0xE0u) << 2) + ((bb & 0x1Cu) << 1) + (bb & 3u));
    const int k_of_second = base + static_cast<int>(((sbits & 0xE0u) << 2) + ((sbits & 0x1Cu) << 1) + (sbits & 3u));
    const bool best_moved = bb != bb0;
    const int demoted = (best_moved && sbits == bb0) ? s.best_k : k_of_second;
    s.second_k = sbits != sb0 ? demoted : s.second_k;
    s.best_k = best_moved ? k_of_best : s.best_k;
}

// How many pairs of the previous group's 32 scores are scanned after each of
// a group's ten matrix-core steps (half-norm of block 0 and of block 1, then
// each 16-dim step of block 0 and block 1).
constexpr int kPairsAfter[10] = {2, 2, 2, 2, 2, 2, 1, 1, 1, 1};

// Matrix-core steps of group kG of the chunk in LDS (rows sb) into dn: two
// 32-codeword blocks, each a chain of the half-norm step and four 16-dim
// steps. When kScan, the key scan of the previous group dp (index bits
// gbits) into set `ks` is placed between them in a fixed order, and the
// operands of the next step are read from LDS before the current step's
// products are issued.
template <bool kScan>
__device__ __forceinline__ void step_group(f32x16 (&dn)[2], const f32x16 (&dp)[2], int kG, const _Float16 *sb,
                                           int col, int half, const f16x8 (&nb)[4],
                                           const f16x8 &nnorm, int gbits, unsigned mask, KeySet &ks)
{
    f16x8 a[2][2];   // [step parity][block]
    auto load_ops = [&](int s) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
            a[s & 1][b] = *reinterpret_cast<const f16x8 *>(sb + (kG * 64 + b * 32 + col) * kRowHalfs +
                                                          8 * (4 * half + s));
    };
    // the half-norm step's operand: the row's last slot (its two fp16 parts
    // first, then zeros; only half 0's first two products are nonzero)
    f16x8 an[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
        an[b] = *reinterpret_cast<const f16x8 *>(sb + (kG * 64 + b * 32 + col) * kRowHalfs + 64);
    load_ops(0);
    int v = 0;   // next score of dp
    auto scan_some = [&](int pairs) {
        if (kScan) {
#pragma unroll
            for (int i = 0; i < pairs; ++i) {
                scan_pair(dp, v + 2 * i, gbits, mask, ks);
                // keep the updates here, between the matrix steps (the
                // compiler would otherwise sink the second and third chains
                // past the group), after every second pair so that the
                // third's updates still merge into v_min3; the second key
                // feeds the third's update, so it stays in place unpinned
                // (a pinned value is opaque to the compiler, which then
                // canonicalizes it before every minimum: one more
                // instruction per pair)
                if (((v >> 1) + i) & 1) asm volatile("" : "+v"(ks.best), "+v"(ks.third));
            }
        }
        v += 2 * pairs;
    };
    const f32x16 zero = {};
    dn[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(an[0], nnorm, zero, 0, 0, 0);
    scan_some(kPairsAfter[0]);
    __builtin_amdgcn_sched_barrier(0);
    dn[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(an[1], nnorm, zero, 0, 0, 0);
    scan_some(kPairsAfter[1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (s < 3) load_ops(s + 1);
        __builtin_amdgcn_sched_barrier(0);
        dn[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s & 1][0], nb[s], dn[0], 0, 0, 0);
        scan_some(kPairsAfter[2 + 2 * s]);
        __builtin_amdgcn_sched_barrier(0);
        dn[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s & 1][1], nb[s], dn[1], 0, 0, 0);
        scan_some(kPairsAfter[3 + 2 * s]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The key scan of the last group of a stage, alone.
__device__ __forceinline__ void scan_last(const f32x16 (&d)[2], int gbits, unsigned mask, KeySet &ks)
{
#pragma unroll
    for (int v = 0; v < 32; v += 2) scan_pair(d, v, gbits, mask, ks);
}

// The group at `base` that holds codeword n_codes - 1 when n_codes is not a
// multiple of 64: its rows at or past n_codes (zero rows of the prepared
// block) get kNoScore before the scan, so they are never candidates.
__device__ __forceinline__ void mask_tail(f32x16 (&d)[2], int base, int half, int n_codes)
{
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 16; ++a)
            if (base + b * 32 + 8 * (a >> 2) + 4 * half + (a & 3) >= n_codes) d[b][a] = kNoScore;
}

// The largest 0.5*||c'||^2 of a prepared stage: the maximum of its Kp/kChunk
// fp16-section words (loaded early by stage_max_part, reduced over the
// wavefront by wave_max_bits at the decision). Values are >= 0 (or +inf), so
// their bits order like the values.
__device__ __forceinline__ unsigned stage_max_part(const uint8_t *blk, int64_t kp, int lane)
{
    const unsigned *words = reinterpret_cast<const unsigned *>(blk + prep::f16_max(kp));
    const int n_words = static_cast<int>(kp / kChunk);
    unsigned m = lane < n_words ? words[lane] : 0u;
    for (int c = lane + 64; c < n_words; c += 64) m = max(m, words[c]);
    return m;
}

__device__ __forceinline__ float wave_max_bits(unsigned m)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), off)));
    return __uint_as_float(m);
}

// An upper bound of sqrt(x) for x >= 0: the hardware square root (within a
// few ulp) of max(x, FLT_MIN), raised by 2^-20 of itself.
__device__ __forceinline__ float sqrt_up(float x)
{
    return __builtin_amdgcn_sqrtf(fmaxf(x, FLT_MIN)) * (1.0f + 9.5367431640625e-07f);
}

// The value held by lane l ^ 32, the other half of this lane's frame: one
// v_permlane32_swap (a VALU op, no LDS round trip). Every lane must be
// active.
__device__ __forceinline__ unsigned other_half(unsigned x, int half)
{
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return half ? r[0] : r[1];
}
__device__ __forceinline__ float other_half(float x, int half)
{
    return __uint_as_float(other_half(__float_as_uint(x), half));
}
__device__ __forceinline__ int other_half(int x, int half)
{
    return static_cast<int>(other_half(static_cast<unsigned>(x), half));
}

// This lane's half (32 dims) of codeword k's fp32 row.
__device__ __forceinline__ void load_row(f32x4 (&row)[8], const float *book, int k, int half)
{
    const f32x4 *src = reinterpret_cast<const f32x4 *>(book + static_cast<int64_t>(k) * kDim + 32 * half);
#pragma unroll
    for (int t = 0; t < 8; ++t) row[t] = src[t];
}

// Float32 direct-form distance sum_j fl(n_j + c_j)^2 of a codeword (this
// lane's half of its row in registers) to the frame held by lanes
// (l, l^32), fused multiply-adds in four chains per lane; the same value on
// both lanes. Every lane must call it.
__device__ __forceinline__ float pair_distance_f32_row(const float (&n)[32], const f32x4 (&row)[8], int half)
{
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = n[4 * t + i] + row[t][i];
            a[i] = __builtin_fmaf(d, d, a[i]);
        }
    const float s = (a[0] + a[1]) + (a[2] + a[3]);
    return s + other_half(s, half);
}


// Entry i (0..3) of a four-entry list, selected without indexing registers.
__device__ __forceinline__ int pick4(const int (&l)[4], int i)
{
    return i == 0 ? l[0] : i == 1 ? l[1] : i == 2 ? l[2] : l[3];
}

// Codeword i of key set (h, s) in ascending order: lane half h holds rows
// with bit 2 equal to h, set s the 64-codeword groups with bit 6 equal to s.
__device__ __forceinline__ int subset_code(int i, int h, int s)
{
    return ((i >> 5) << 7) | (s << 6) | (((i >> 2) & 7) << 3) | (h << 2) | (i & 3);
}

// Float32 direct form sum_j fl(r_j + c_j)^2 over all 64 dims of codeword k
// (frame row r in LDS), four fused multiply-add chains; within
// (2u + u^2 + gamma_64) of the exact distance, as pair_distance_f32_row.
__device__ __forceinline__ float row_distance_f32(const float *row, const float *book, int k)
{
    const f32x4 *r4 = reinterpret_cast<const f32x4 *>(row);
    const f32x4 *c4 = reinterpret_cast<const f32x4 *>(book + static_cast<int64_t>(k) * kDim);
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const f32x4 rv = r4[t], cv = c4[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = rv[i] + cv[i];
            a[i] = __builtin_fmaf(d, d, a[i]);
        }
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// Float64 direct form in the oracle's order (j = 0..63, one rounding per
// operation) of codeword k against the frame row in LDS.
__device__ __forceinline__ double row_distance_f64(const float *row, const float *book, int k)
{
    const f32x4 *r4 = reinterpret_cast<const f32x4 *>(row);
    const f32x4 *c4 = reinterpret_cast<const f32x4 *>(book + static_cast<int64_t>(k) * kDim);
    double acc = 0.0;
#pragma unroll 4
    for (int t = 0; t < 16; ++t) {
        const f32x4 rv = r4[t], cv = c4[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double d = __dadd_rn(static_cast<double>(rv[i]), static_cast<double>(cv[i]));
            acc = __dadd_rn(acc, __dmul_rn(d, d));
        }
    }
    return acc;
}

// kParts wavefronts of a workgroup that resolve the same frame each take
// every kParts-th codeword and then combine their results through LDS
// (`xch`, 4 words per wavefront), all in wavefront order, so that every one
// of them ends with the same values. Every wavefront of the workgroup must
// call these, equally often; the first barrier keeps a previous exchange's
// readers ahead of this one's writers.
template <int kParts>
__device__ __forceinline__ void exchange_f32(float &f1, float &f2, int &k1, unsigned *xch, int part, int lane)
{
    __syncthreads();
    if (lane == 0) {
        xch[4 * part] = __float_as_uint(f1);
        xch[4 * part + 1] = __float_as_uint(f2);
        xch[4 * part + 2] = static_cast<unsigned>(k1);
    }
    __syncthreads();
    float a1 = __uint_as_float(xch[0]), a2 = __uint_as_float(xch[1]);
    int ak = static_cast<int>(xch[2]);
#pragma unroll
    for (int p = 1; p < kParts; ++p) {
        const float b1 = __uint_as_float(xch[4 * p]), b2 = __uint_as_float(xch[4 * p + 1]);
        const int bk = static_cast<int>(xch[4 * p + 2]);
        const float lo = fminf(a1, b1), hi = fmaxf(a1, b1);
        ak = a1 < b1 ? ak : (b1 < a1 ? bk : min(ak, bk));
        a2 = fminf(fminf(a2, b2), hi);
        a1 = lo;
    }
    f1 = a1;
    f2 = a2;
    k1 = ak;
}

template <int kParts>
__device__ __forceinline__ void exchange_f64(double &bd, int &bk, unsigned *xch, int part, int lane)
{
    __syncthreads();
    if (lane == 0) {
        const unsigned long long u = __double_as_longlong(bd);
        xch[4 * part] = static_cast<unsigned>(u);
        xch[4 * part + 1] = static_cast<unsigned>(u >> 32);
        xch[4 * part + 2] = static_cast<unsigned>(bk);
    }
    __syncthreads();
    double a = INFINITY;
    int ak = 0x7fffffff;
#pragma unroll
    for (int p = 0; p < kParts; ++p) {
        const double d = __longlong_as_double(static_cast<long long>(
            static_cast<unsigned long long>(xch[4 * p]) | (static_cast<unsigned long long>(xch[4 * p + 1]) << 32)));
        const int k = static_cast<int>(xch[4 * p + 2]);
        if (d < a || (d == a && k < ak)) {
            a = d;
            ak = k;
        }
    }
    bd = a;
    bk = ak;
}

// A third candidate inside one or more key sets of frame f (lanes f, f+32):
// the wavefront takes every codeword of each overflowed set (bit 2h+s of
// `mask`) and the listed candidates of the other sets (l0 / l1 / cnt0 /
// ncand as held by lane f); float32 distances first, and the float64 direct
// form for every entry within 2^-16 of the smallest when the two smallest
// are that close (ties go to the lowest index). Returns the winner on every
// lane. Every lane must call it; `row` is a 64-float LDS row of this
// wavefront. With kParts > 1, kParts wavefronts holding the same frames
// share the work (this one is `part`; see exchange_f32).
template <int kParts>
__device__ int resolve_sets(const float (&n)[32], float *row, const float *book, int n_codes, int f, int lane,
                            unsigned mask, const int (&l0)[4], const int (&l1)[4], int cnt0, int ncand,
                            int part, unsigned *xch)
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
    // frame f's listed candidates, on every lane
    const int c0 = __builtin_amdgcn_readlane(cnt0, f);
    const int nc = __builtin_amdgcn_readlane(ncand, f);
    const int a0 = __builtin_amdgcn_readlane(l0[0], f), a1 = __builtin_amdgcn_readlane(l0[1], f);
    const int a2 = __builtin_amdgcn_readlane(l0[2], f), a3 = __builtin_amdgcn_readlane(l0[3], f);
    const int b0 = __builtin_amdgcn_readlane(l1[0], f), b1 = __builtin_amdgcn_readlane(l1[1], f);
    const int b2 = __builtin_amdgcn_readlane(l1[2], f), b3 = __builtin_amdgcn_readlane(l1[3], f);
    const int span = (n_codes + 127) / 128 * 32;   // index range of one set
    auto in_mask = [&](int k) { return ((mask >> (2 * ((k >> 2) & 1) + ((k >> 6) & 1))) & 1u) != 0; };
    // lane e < ncand takes listed candidate e (half 0's list, then half 1's)
    // unless its set is swept anyway
    int extra = -1;
    if (lane < nc) {
        const bool first = lane < c0;
        const int j = first ? lane : lane - c0;
        const int q0 = first ? a0 : b0, q1 = first ? a1 : b1, q2 = first ? a2 : b2, q3 = first ? a3 : b3;
        const int k = j == 0 ? q0 : j == 1 ? q1 : j == 2 ? q2 : q3;
        if (!in_mask(k)) extra = k;
    }
    // float32 pass
    float f1 = INFINITY, f2 = INFINITY;
    int k1 = 0x7fffffff;
    auto take = [&](int k) {
        const float d = row_distance_f32(row, book, k);
        f2 = d < f1 ? f1 : fminf(f2, d);
        k1 = d < f1 ? k : k1;
        f1 = fminf(f1, d);
    };
    for (int b = 0; b < 4; ++b) {
        if (!((mask >> b) & 1u)) continue;
        for (int i = lane + 64 * part; i < span; i += 64 * kParts) {
            const int k = subset_code(i, b >> 1, b & 1);
            if (k < n_codes) take(k);
        }
    }
    if (extra >= 0 && part == 0) take(extra);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float of1 = __shfl_xor(f1, off), of2 = __shfl_xor(f2, off);
        const int ok1 = __shfl_xor(k1, off);
        const float lo = fminf(f1, of1), hi = fmaxf(f1, of1);
        k1 = f1 < of1 ? k1 : (of1 < f1 ? ok1 : min(k1, ok1));
        f2 = fminf(fminf(f2, of2), hi);
        f1 = lo;
    }
    if (kParts > 1) exchange_f32<kParts>(f1, f2, k1, xch, part, lane);
    const float thr = f1 * (1.0f + 1.52587890625e-05f) + 1e-30f;
    int win = k1;
    if (f2 <= thr) {   // wave-uniform: float64 for every entry within thr of the smallest
        double bd = INFINITY;
        int bk = 0x7fffffff;
        auto exact = [&](int k) {
            if (row_distance_f32(row, book, k) <= thr) {
                const double d = row_distance_f64(row, book, k);
                if (d < bd || (d == bd && k < bk)) {
                    bd = d;
                    bk = k;
                }
            }
        };
        for (int b = 0; b < 4; ++b) {
            if (!((mask >> b) & 1u)) continue;
            for (int i = lane + 64 * part; i < span; i += 64 * kParts) {
                const int k = subset_code(i, b >> 1, b & 1);
                if (k < n_codes) exact(k);
            }
        }
        if (extra >= 0 && part == 0) exact(extra);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double od = __shfl_xor(bd, off);
            const int ok = __shfl_xor(bk, off);
            if (od < bd || (od == bd && ok < bk)) {
                bd = od;
                bk = ok;
            }
        }
        if (kParts > 1) exchange_f64<kParts>(bd, bk, xch, part, lane);
        win = bk;
    }
    // all reads of `row` are done before a later call overwrites it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    return win;
}

// The decision for one stage from this lane's two key sets (codeword slots
// of one half of a frame; lanes l and l^32 hold the two halves): every
// codeword within 2E (1) of the frame's smallest key is a candidate; two to
// eight candidates are re-ranked (float32, float64 for near ties); a third
// candidate inside a set (or ambiguous bookkeeping) sends the frame to the
// sweep of its overflowed sets, fp16 out of range to the full float64
// rescan. Then the pick is stored (code_out, when not null) and subtracted
// from the negated residual n (and added to acc for kRecon). Every lane
// must call it. With kParts > 1 the kParts wavefronts of the workgroup
// decide the same frames from the same key sets and share each sweep
// (wavefront `part`, LDS `xch`); they must all call it.
template <bool kRecon, int kParts = 1>
__device__ __forceinline__ void decide_stage(float (&n)[32], float (&acc)[32], const KeySet (&ks)[2],
                                             const float *book, int n_codes, float m16, int e, bool valid,
                                             int half, int col, int lane, float *frame_row, int32_t *code_out,
                                             int part = 0, unsigned *xch = nullptr)
{
    float r4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 32; ++j) r4[j & 3] = __builtin_fmaf(n[j], n[j], r4[j & 3]);
    float rn = (r4[0] + r4[1]) + (r4[2] + r4[3]);
    rn = rn + other_half(rn, half);
    // |n_j| < 2^15 keeps every fp16(n_j) finite; a stage out of the fp16
    // range has an infinite maximum
    const bool bad = !(rn < 1073741824.0f) || !(m16 <= FLT_MAX);

    const float r_up = sqrt_up(rn * (1.0f + 1.52587890625e-05f));
    const float m_up = m16 * (1.0f + 1.52587890625e-05f);
    const float c_up = sqrt_up(2.0f * m_up);
    const float t_up = ldexpf(m_up, -e);
    const float bound = (kRel * (t_up + r_up * c_up) + kAbsN * r_up + kAbsC * c_up + ldexpf(kAbsNorm, -e) +
                         kAbsConst) * (1.0f + 2.44140625e-04f);
    // Keys decode to real codewords whenever the frame's scores are finite;
    // a non-finite frame (decided by the rescan, its code then unspecified)
    // can decode padding slots past n_codes, so every index is clamped here,
    // before any row load of the re-rank, the sweep or the update.
    int kk[4] = {ks[0].best_k, ks[0].second_k, ks[1].best_k, ks[1].second_k};
#pragma unroll
    for (int i = 0; i < 4; ++i) kk[i] = min(max(kk[i], 0), n_codes - 1);
    const float lane_min = fminf(ks[0].best, ks[1].best);
    const int lane_k = ks[0].best <= ks[1].best ? kk[0] : kk[2];
    const float other_min = other_half(lane_min, half);
    const int other_k = other_half(lane_k, half);
    const float frame_min = fminf(lane_min, other_min);
    const float lim = frame_min + 2.0f * bound + fabsf(frame_min) * 2.4e-7f;
    // The smallest key's codeword (half 0's on equal keys) is the pick of
    // every frame with one candidate, and one candidate of every other frame:
    // its row is fetched now, for the re-rank and the update, so that the
    // decision waits for at most one more round of row loads.
    // half 0's codeword unless half 1's key is smaller: the same choice on
    // both lanes of the frame, also for non-finite keys
    const int pred = (half ? lane_min < other_min : other_min < lane_min) ? (half ? lane_k : other_k)
                                                                           : (half ? other_k : lane_k);
    f32x4 prow[8];
    load_row(prow, book, pred, half);
    int have = pred;   // the codeword whose row prow holds

    // key sets holding a third candidate (or ambiguous bookkeeping): bit s
    // for this lane, bit 2h+s for the frame
    unsigned ovs = 0u;
#pragma unroll
    for (int s = 0; s < 2; ++s)
        if (ks[s].third <= lim || (ks[s].second <= lim && kk[2 * s + 1] == kk[2 * s])) ovs |= 1u << s;
    // the shuffle must run on every lane: under a divergent mask the partner
    // lane could be inactive and the two halves of a frame could disagree
    const unsigned ovs_o = other_half(ovs, half);
    const unsigned ovmask = half ? (ovs_o | (ovs << 2)) : (ovs | (ovs_o << 2));
    const bool overflow = bad || ovmask != 0u;

    // this lane's candidates, compacted: set 0 best, second, set 1 best, second
    const float sv[4] = {ks[0].best, ks[0].second, ks[1].best, ks[1].second};
    const int sk[4] = {kk[0], kk[1], kk[2], kk[3]};
    int list[4] = {0, 0, 0, 0};
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool c = sv[i] <= lim;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (c && cnt == j) list[j] = sk[i];
        cnt += c;
    }
    int list_o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) list_o[j] = other_half(list[j], half);
    const int cnt_o = other_half(cnt, half);
    const int ncand = cnt + cnt_o;
    // frame candidate j: half 0's list, then half 1's
    const int cnt0 = half ? cnt_o : cnt;
    int l0[4], l1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        l0[j] = half ? list_o[j] : list[j];
        l1[j] = half ? list[j] : list_o[j];
    }
    int pick = pred;   // the one candidate when ncand == 1

    // Two to eight candidates. A float32 pass first: the direct form
    // sum_j fl(n_j + c_j)^2 with fused multiply-adds is within
    // (2u + u^2 + gamma_64) d < 4e-6 d of the exact distance d (u = 2^-24,
    // all terms >= 0) and the oracle's float64 sum within 1e-14 d of it, so a
    // candidate whose float32 distance exceeds the smallest one's by more than
    // 2^-16 of it cannot be the oracle's pick. Only frames whose two smallest
    // float32 distances are that close take the float64 re-rank of all their
    // candidates (equal distances included, so ties still go to the lowest
    // index). pred's row is already here; the loop loads the others, the
    // list without pred (which appears in it once).
    const bool rerank = valid && !overflow && ncand >= 2;
    if (__any(rerank)) {
        auto entry = [&](int e) { return e < cnt0 ? pick4(l0, e) : pick4(l1, e - cnt0); };
        int pos = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < ncand && entry(e & 7) == pred) pos = e;
        // the first other candidate's row is requested before pred's
        // distance waits for pred's row
        int k = rerank ? entry(pos == 0 ? 1 : 0) : pred;
        f32x4 cur[8];
        load_row(cur, book, k, half);
        float f1 = pair_distance_f32_row(n, prow, half), f2 = INFINITY;
        int k1 = pred;
        for (int j = 0; __any(rerank && j < ncand - 1); ++j) {
            const bool use = rerank && j < ncand - 1;
            if (j > 0) {
                k = use ? entry(j + (j >= pos)) : pred;
                load_row(cur, book, k, half);
            }
            const float f = pair_distance_f32_row(n, cur, half);
            if (use) {
                f2 = f < f1 ? f1 : fminf(f2, f);
                if (f < f1) {
                    k1 = k;
#pragma unroll
                    for (int t = 0; t < 8; ++t) prow[t] = cur[t];
                }
                f1 = fminf(f1, f);
            }
        }
        if (rerank) {
            pick = k1;
            have = k1;
        }
        const bool exact = rerank && f2 <= f1 * (1.0f + 1.52587890625e-05f) + 1e-30f;
        if (__any(exact)) {
            double bd = INFINITY;
            int bk = 0x7fffffff;
            for (int j = 0; __any(exact && j < ncand); ++j) {
                const bool use = exact && j < ncand;
                const int k = use ? entry(j) : pick;
                const double dist = pair_distance(n, book, k, half);
                if (use && (dist < bd || (dist == bd && k < bk))) {
                    bd = dist;
                    bk = k;
                }
            }
            if (exact) pick = bk;
        }
    }

    // A third candidate inside a key set: those sets swept, the other
    // candidates added. A frame or stage out of fp16's range: full rescan.
    uint64_t pending = __ballot(valid && overflow && half == 0);
    while (pending) {
        const int f = __ffsll(static_cast<unsigned long long>(pending)) - 1;
        pending &= pending - 1;
        const int w = __builtin_amdgcn_readlane(static_cast<int>(bad), f)
                          ? rescan_frame(n, frame_row, book, n_codes, f, lane)
                          : resolve_sets<kParts>(n, frame_row, book, n_codes, f, lane,
                                                 static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(ovmask), f)),
                                                 l0, l1, cnt0, ncand, part, xch);
        if (col == f) pick = w;
    }

    pick = min(max(pick, 0), n_codes - 1);
    if (code_out) *code_out = pick;
    if (__any(pick != have)) {   // an exact re-rank, sweep or rescan moved the pick
        if (pick != have) load_row(prow, book, pick, half);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            n[4 * t + i] = n[4 * t + i] + prow[t][i];   // = -(r - c), exactly
            if (kRecon) acc[4 * t + i] = acc[4 * t + i] + prow[t][i];
        }
    }
}

template <bool kRecon, bool kResidual>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void encode_f16_kernel(const float *__restrict__ x, int64_t n_frames,
                       const float *__restrict__ books, const uint8_t *__restrict__ prepared,
                       int n_stages, int n_codes,
                       int32_t *__restrict__ codes, int codes_ld,
                       float *__restrict__ residual, float *__restrict__ recon)
{
    __shared__ __align__(16) _Float16 s_rows[2][kChunk * kRowHalfs];
    __shared__ __align__(16) float s_frame[kWaves][kDim];   // rescan: one frame's residual

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kBlockFrames + wave * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    // the key mask in a vector register, so that each key is one
    // v_and_or_b32 whose index bits come from a scalar register
    unsigned kmask;
    asm volatile("v_mov_b32 %0, %1" : "=v"(kmask) : "i"(kKeyMask8));
    float n[32];     // negated residual, dims 32*half .. 32*half+31
    float acc[32];   // reconstruction (kRecon)
    if (valid) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(x + frame * kDim + 32 * half);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 v = src[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) n[4 * t + i] = -v[i];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) n[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.0f;

    const int64_t kp = prep::padded_codes(n_codes);
    const int64_t sbytes = prep::stage_bytes(n_codes);
    const int n_chunks = static_cast<int>(kp / kChunk);
    const int n_groups = (n_codes + 63) / 64;   // groups past it hold only padding rows and are not scanned
    const int total = n_stages * n_chunks;

    // wavefront w copies rows kWaveRows*w .. +kWaveRows-1 of chunk g (144
    // bytes each, contiguous in the prepared block and in LDS) into buffer
    // g % 2
    auto dma_chunk = [&](int g) {
        const int q = g / n_chunks;
        const int c = g - q * n_chunks;
        const uint8_t *blk = prepared + q * sbytes;
        const int k0 = c * kChunk + kWaveRows * wave;
        const uint8_t *src = blk + static_cast<int64_t>(k0) * prep::kF16Row + 16 * lane;
        _Float16 *dst = s_rows[g & 1] + kWaveRows * wave * kRowHalfs;
#pragma unroll
        for (int i = 0; i < kWaveLoads; ++i) dma16(src + 1024 * i, dst + i * 512);
    };

    dma_chunk(0);
    wait_all();
    __syncthreads();

    for (int q = 0; q < n_stages; ++q) {
        const uint8_t *blk = prepared + q * sbytes;
        const unsigned cmax = stage_max_part(blk, kp, lane);   // used at the decision
        const int e = *reinterpret_cast<const int *>(blk + prep::f16_exp(kp));
        f16x8 nb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) nb[s] = to_f16x8(&n[8 * s]);
        // half-norm step: this frame's operand is (2^-e, 2^-e, 0, ...) on half 0, zero on half 1
        const f16x2 sc = {static_cast<_Float16>(ldexpf(1.0f, -e)), static_cast<_Float16>(ldexpf(1.0f, -e))};
        const f16x8 nnorm = __builtin_bit_cast(f16x8, u32x4{half ? 0u : __builtin_bit_cast(unsigned, sc), 0u, 0u, 0u});

        KeySet ks[2];
        reset(ks[0]);
        reset(ks[1]);
        // best / second bits of each set at the start of its current span
        unsigned snap_b[2] = {__float_as_uint(kNoScore), __float_as_uint(kNoScore)};
        unsigned snap_s[2] = {__float_as_uint(kNoScore), __float_as_uint(kNoScore)};
        auto fold_set = [&](int set, int span) {
            fold(ks[set], snap_b[set], snap_s[set], span, set, half);
            snap_b[set] = __float_as_uint(ks[set].best);
            snap_s[set] = __float_as_uint(ks[set].second);
        };
        f32x16 da[2], db[2];
        int prev_base = 0;   // first codeword of the group held in db

        for (int c = 0; c < n_chunks; ++c) {
            const int g = q * n_chunks + c;
            if (c > 0) {
                wait_all();        // this wavefront's copies into chunk g's buffer have landed
                __syncthreads();   // everyone's have; chunk g-1's buffer is no longer read
            }
            if (g + 1 < total) dma_chunk(g + 1);
            const _Float16 *sb = s_rows[g & 1];
#pragma unroll 1
            for (int p = 0; p < kGroups / 2; ++p) {
                const int ka = 2 * p, kb = 2 * p + 1;
                // step A scores group 4c+ka and scans the odd group before it (set 1);
                // step B scores group 4c+kb and scans group 4c+ka (set 0)
                const bool scan_a = !(c == 0 && p == 0) && (prev_base >> 6) < n_groups;
                if (scan_a) {
                    if (prev_base + 64 > n_codes) mask_tail(db, prev_base, half, n_codes);
                    step_group<true>(da, db, ka, sb, col, half, nb, nnorm, group_bits(prev_base), kmask, ks[1]);
                    // the last odd group of a span: set 1's keys of that span are complete
                    if (((prev_base + 64) & (kSpan - 1)) == 0) fold_set(1, prev_base & ~(kSpan - 1));
                } else {
                    step_group<false>(da, db, ka, sb, col, half, nb, nnorm, 0, kmask, ks[1]);
                }
                const int base_a = c * kChunk + 64 * ka;
                if ((base_a >> 6) < n_groups) {
                    if (base_a + 64 > n_codes) mask_tail(da, base_a, half, n_codes);
                    step_group<true>(db, da, kb, sb, col, half, nb, nnorm, group_bits(base_a), kmask, ks[0]);
                    // the last even group of a span
                    if (((base_a + 128) & (kSpan - 1)) == 0) fold_set(0, base_a & ~(kSpan - 1));
                } else {
                    step_group<false>(db, da, kb, sb, col, half, nb, nnorm, 0, kmask, ks[0]);
                }
                prev_base = c * kChunk + 64 * kb;
            }
        }
        if ((prev_base >> 6) < n_groups) {
            if (prev_base + 64 > n_codes) mask_tail(db, prev_base, half, n_codes);
            scan_last(db, group_bits(prev_base), kmask, ks[1]);
        }
        // keys of the last span (partial, or not yet folded) of both sets
        const int last_span = ((n_groups - 1) * 64) & ~(kSpan - 1);
        fold_set(0, last_span);
        fold_set(1, last_span);

        // ---- stage q is scored for this wavefront's 32 frames: decide ----
        const float *book = books + static_cast<int64_t>(q) * n_codes * kDim;
        const float m16 = wave_max_bits(cmax);
        decide_stage<kRecon>(n, acc, ks, book, n_codes, m16, e, valid, half, col, lane, s_frame[wave],
                             (valid && half == 0) ? codes + frame * codes_ld + q : nullptr);
        if (q + 1 < n_stages) {
            wait_all();
            __syncthreads();   // the next stage's first chunk is in LDS; the last one's buffer is free
        }
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

// ---- small batches: the codebook split over a workgroup's wavefronts -------
//
// A workgroup of four wavefronts holds one 32-frame tile (every wavefront
// the same frames, in the same lanes); wavefront w scores the 256-codeword
// chunks w, w + 4, ... of every stage out of its own LDS buffer (copied
// straight from the prepared block, the next chunk as soon as the current
// one is scored, so the next stage's first chunk loads during the
// decision). Within a 1024-codeword span each wavefront holds one chunk,
// so its keys are folded into indices after every chunk. The wavefronts'
// key sets are then merged through LDS in wavefront order -- the smallest
// key and its codeword, the second smallest of the two sets' four keys,
// and a lower bound of the third -- and every wavefront takes the same
// decision from the same merged sets (the decision only reads the
// codebook), so each keeps the residual without a broadcast; a set sweep
// is shared among the four (each takes every fourth codeword, the partial
// results are combined through LDS). Wavefront 0 stores codes, residual
// and reconstruction. The keys, bound and decision are the wide kernel's,
// so the codes are too.
constexpr int kKsWaves = 4;
constexpr int kKsThreads = 64 * kKsWaves;
constexpr int kKsChunkLoads = kChunk * kRowSlots / 64;   // wavefront-wide 16-byte copies per chunk
constexpr int kKsKeyWords = 10;                          // per lane: 2 sets x (best, second, third, best_k, second_k)

// The two smallest keys of the union of sets a and b (with their codewords;
// equal keys: the lower codeword first) and a lower bound of the third
// smallest: the third order statistic of two sorted lists is
// min(a3, b3, max(a1, b2), max(a2, b1)), and a.third, b.third are at most a3, b3.
__device__ __forceinline__ KeySet merge_sets(const KeySet &a, const KeySet &b)
{
    const bool a_first = a.best < b.best || (a.best == b.best && a.best_k <= b.best_k);
    const float wb = a_first ? a.best : b.best, ws = a_first ? a.second : b.second;
    const int wbk = a_first ? a.best_k : b.best_k, wsk = a_first ? a.second_k : b.second_k;
    const float lb = a_first ? b.best : a.best;
    const int lbk = a_first ? b.best_k : a.best_k;
    const bool loser_second = lb < ws || (lb == ws && lbk <= wsk);
    KeySet m;
    m.best = wb;
    m.best_k = wbk;
    m.second = loser_second ? lb : ws;
    m.second_k = loser_second ? lbk : wsk;
    m.third = fminf(fminf(a.third, b.third), fminf(fmaxf(a.best, b.second), fmaxf(a.second, b.best)));
    return m;
}

template <bool kRecon, bool kResidual>
__global__ __attribute__((amdgpu_flat_work_group_size(kKsThreads, kKsThreads), amdgpu_waves_per_eu(1)))   // one workgroup per CU (LDS)
void encode_f16_ksplit_kernel(const float *__restrict__ x, int64_t n_frames,
                              const float *__restrict__ books, const uint8_t *__restrict__ prepared,
                              int n_stages, int n_codes,
                              int32_t *__restrict__ codes, int codes_ld,
                              float *__restrict__ residual, float *__restrict__ recon)
{
    __shared__ __align__(16) _Float16 s_rows[kKsWaves][kChunk * kRowHalfs];   // one chunk per wavefront
    __shared__ __align__(16) float s_frame[kKsWaves][kDim];                    // rescan: one frame's residual
    __shared__ unsigned s_keys[kKsWaves][kKsKeyWords][64];
    __shared__ unsigned s_xch[kKsWaves * 4];   // the shared sweeps' partial results

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    unsigned kmask;
    asm volatile("v_mov_b32 %0, %1" : "=v"(kmask) : "i"(kKeyMask8));
    float n[32];     // negated residual, dims 32*half .. 32*half+31
    float acc[32];   // reconstruction (kRecon)
    if (valid) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(x + frame * kDim + 32 * half);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 v = src[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) n[4 * t + i] = -v[i];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) n[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.0f;

    const int64_t kp = prep::padded_codes(n_codes);
    const int64_t sbytes = prep::stage_bytes(n_codes);
    const int n_chunks = static_cast<int>(kp / kChunk);
    const int n_groups = (n_codes + 63) / 64;
    _Float16 *sb = s_rows[wave];
    // chunk c of stage q into this wavefront's buffer (after its earlier
    // reads of the buffer have completed)
    auto dma_chunk = [&](int q, int c) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint8_t *src = prepared + q * sbytes + static_cast<int64_t>(c) * kChunk * prep::kF16Row + 16 * lane;
#pragma unroll 4
        for (int i = 0; i < kKsChunkLoads; ++i) dma16(src + 1024 * i, sb + i * 512);
    };
    if (wave < n_chunks) dma_chunk(0, wave);

    for (int q = 0; q < n_stages; ++q) {
        const uint8_t *blk = prepared + q * sbytes;
        const unsigned cmax = stage_max_part(blk, kp, lane);
        const int e = *reinterpret_cast<const int *>(blk + prep::f16_exp(kp));
        f16x8 nb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) nb[s] = to_f16x8(&n[8 * s]);
        const f16x2 sc = {static_cast<_Float16>(ldexpf(1.0f, -e)), static_cast<_Float16>(ldexpf(1.0f, -e))};
        const f16x8 nnorm = __builtin_bit_cast(f16x8, u32x4{half ? 0u : __builtin_bit_cast(unsigned, sc), 0u, 0u, 0u});

        KeySet ks[2];
        reset(ks[0]);
        reset(ks[1]);
        for (int c = wave; c < n_chunks; c += kKsWaves) {
            wait_all();   // this chunk has landed in the buffer
            const unsigned bb0[2] = {__float_as_uint(ks[0].best), __float_as_uint(ks[1].best)};
            const unsigned sb0[2] = {__float_as_uint(ks[0].second), __float_as_uint(ks[1].second)};
            f32x16 da[2], db[2];
            // groups 4c + 0..3: each step scores one group and scans the one before
            // (even groups into set 0, odd into set 1), the last one alone
#pragma unroll
            for (int kg = 0; kg < kGroups; ++kg) {
                f32x16 (&dn)[2] = (kg & 1) ? db : da;
                f32x16 (&dp)[2] = (kg & 1) ? da : db;
                const int pbase = c * kChunk + 64 * (kg - 1);   // the group scanned in this step
                if (kg > 0 && (pbase >> 6) < n_groups) {
                    if (pbase + 64 > n_codes) mask_tail(dp, pbase, half, n_codes);
                    step_group<true>(dn, dp, kg, sb, col, half, nb, nnorm, group_bits(pbase), kmask, ks[(kg - 1) & 1]);
                } else {
                    step_group<false>(dn, dp, kg, sb, col, half, nb, nnorm, 0, kmask, ks[0]);
                }
            }
            const int lbase = c * kChunk + 64 * (kGroups - 1);
            if ((lbase >> 6) < n_groups) {
                if (lbase + 64 > n_codes) mask_tail(db, lbase, half, n_codes);
                scan_last(db, group_bits(lbase), kmask, ks[1]);
            }
            // this wavefront holds no other chunk of the span: fold both sets
            const int span = (c * kChunk) & ~(kSpan - 1);
            fold(ks[0], bb0[0], sb0[0], span, 0, half);
            fold(ks[1], bb0[1], sb0[1], span, 1, half);
            // the buffer is free: the next chunk of this stage, or the next stage's first
            if (c + kKsWaves < n_chunks)
                dma_chunk(q, c + kKsWaves);
            else if (q + 1 < n_stages)
                dma_chunk(q + 1, wave);
        }

        // ---- merge the wavefronts' key sets (the same result on every wavefront) ----
        __syncthreads();   // the previous stage's merge has read s_keys
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s_keys[wave][5 * s + 0][lane] = __float_as_uint(ks[s].best);
            s_keys[wave][5 * s + 1][lane] = __float_as_uint(ks[s].second);
            s_keys[wave][5 * s + 2][lane] = __float_as_uint(ks[s].third);
            s_keys[wave][5 * s + 3][lane] = static_cast<unsigned>(ks[s].best_k);
            s_keys[wave][5 * s + 4][lane] = static_cast<unsigned>(ks[s].second_k);
        }
        __syncthreads();
        KeySet mk[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            for (int w = 0; w < kKsWaves; ++w) {
                KeySet o;
                o.best = __uint_as_float(s_keys[w][5 * s + 0][lane]);
                o.second = __uint_as_float(s_keys[w][5 * s + 1][lane]);
                o.third = __uint_as_float(s_keys[w][5 * s + 2][lane]);
                o.best_k = static_cast<int>(s_keys[w][5 * s + 3][lane]);
                o.second_k = static_cast<int>(s_keys[w][5 * s + 4][lane]);
                mk[s] = w == 0 ? o : merge_sets(mk[s], o);
            }
        }

        const float *book = books + static_cast<int64_t>(q) * n_codes * kDim;
        const float m16 = wave_max_bits(cmax);
        decide_stage<kRecon, kKsWaves>(n, acc, mk, book, n_codes, m16, e, valid, half, col, lane, s_frame[wave],
                                       (wave == 0 && valid && half == 0) ? codes + frame * codes_ld + q : nullptr,
                                       wave, s_xch);
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

// Up to this many frames the split-codebook kernel runs: at 32 frames per
// workgroup, one workgroup per CU, the batch still fits one round on 256 CUs
// (measured, 8 stages of 1024: 8,192 frames 72 us against 97 us for the
// wide kernel's 256-frame tiles).
constexpr int64_t kSplitMaxFrames = 8192;

hipError_t launch_ksplit(const float *x, int64_t n_frames, const float *books, const void *prepared,
                         int n_stages, int n_codes, int32_t *codes, int codes_ld, float *residual,
                         float *recon, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kFramesPerWave - 1) / kFramesPerWave;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kKsThreads);
    const uint8_t *p = static_cast<const uint8_t *>(prepared);
    if (recon && residual)
        hipLaunchKernelGGL((encode_f16_ksplit_kernel<true, true>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (recon)
        hipLaunchKernelGGL((encode_f16_ksplit_kernel<true, false>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (residual)
        hipLaunchKernelGGL((encode_f16_ksplit_kernel<false, true>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    else
        hipLaunchKernelGGL((encode_f16_ksplit_kernel<false, false>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    return hipGetLastError();
}

hipError_t launch_wide(const float *x, int64_t n_frames, const float *books, const void *prepared,
                       int n_stages, int n_codes, int32_t *codes, int codes_ld, float *residual,
                       float *recon, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kBlockFrames - 1) / kBlockFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    const uint8_t *p = static_cast<const uint8_t *>(prepared);
    if (recon && residual)
        hipLaunchKernelGGL((encode_f16_kernel<true, true>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (recon)
        hipLaunchKernelGGL((encode_f16_kernel<true, false>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    else if (residual)
        hipLaunchKernelGGL((encode_f16_kernel<false, true>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    else
        hipLaunchKernelGGL((encode_f16_kernel<false, false>), grid, block, 0, stream,
                           x, n_frames, books, p, n_stages, n_codes, codes, codes_ld, residual, recon);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_prepared(const float *x, int64_t n_frames, const float *books, const void *prepared,
                                  int n_stages, int n_codes, int32_t *codes, int codes_ld,
                                  float *residual, float *recon, hipStream_t stream)
{
    if (n_frames <= kSplitMaxFrames)
        return launch_ksplit(x, n_frames, books, prepared, n_stages, n_codes, codes, codes_ld, residual, recon,
                             stream);
    return launch_wide(x, n_frames, books, prepared, n_stages, n_codes, codes, codes_ld, residual, recon, stream);
}

}  // namespace rvq
