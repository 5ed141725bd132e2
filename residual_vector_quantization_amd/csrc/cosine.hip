// Normalized (cosine) per-stage projected residual vector quantization for
// gfx950 (CDNA4): the quantizer of the "Maintainer's guide -- moss-tts.cpp"
// page (gotchas, item 9). Each stage projects the hidden-width residual into
// an 8-dim codebook space (project_in, with bias), scales the projection and
// every codeword to unit L2 norm (dividing by max(norm, 1e-12)), picks the
// nearest unit codeword, and subtracts the projected-back stored codeword
// (project_out, with bias) from the residual -- the loop of the "RVQ codec"
// section of the "Architecture" page. The residual update and the decode
// use the table of projected codewords of projected.hip.
//
// Exactness. The oracle decides each pick in float64: u = e / max(|e|,
// 1e-12), v_k = c_k / max(|c_k|, 1e-12), d_k = sum_j (u_j - v_kj)^2 (j
// ascending), lowest k on ties. Here the unit codewords v_k are prepared
// once in exactly that float64 arithmetic (double sqrt and division are
// correctly rounded on gfx950). Scores are fp32:
//     s_k = 0.5 |v32_k|^2 - u32 . v32_k,   d_k = |u|^2 + 2 s_k (exact reals),
// with u32 normalized in fp32 and v32 = fp32(v_k). Every |u| and |v_k| is at
// most 1, so the normalization (<= 8u per element), the rounding of v, the
// 8-term dot product and the half-norm keep each s_k within kScoreError of
// its exact value (24u is the worst case; 96u is used). When the two lowest
// fp32 scores are more than 2 kScoreError + 1e-13 apart the fp32 winner is
// the float64 winner (float64 distances are within 1e-14 of exact);
// otherwise the frame is rescanned over all codewords in float64 by its
// whole wavefront with the oracle's formula.
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rvq_internal.h"

namespace rvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCosDim = 8;
constexpr float kUnit = 5.9604644775390625e-08f;       // 2^-24
constexpr float kScoreError = 96.0f * kUnit;
constexpr float kAmbiguous = 2.0f * kScoreError + 1e-13f;
// all-stage kernel: scores (from the matrix cores, within 42u of exact)
// travel as keys with their 4 low mantissa bits replaced by the codeword's
// slot, at most 16 ulp (< 32u, as |s| < 2) from the score: 42u + 32u in the
// worst case, 128u is used
constexpr float kKeyScoreError = 128.0f * kUnit;
constexpr float kKeyAmbiguous = 2.0f * kKeyScoreError + 1e-13f;
constexpr int kArgChunk = 256;                          // unit codewords per LDS chunk
constexpr int kProjWaves = 4;

// v = c / max(|c|, 1e-12) in float64 for every codeword of every stage.
__global__ __launch_bounds__(256)
void units_kernel(const float *__restrict__ books, int64_t rows, double *__restrict__ units)
{
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (r >= rows) return;
    const float *c = books + r * kCosDim;
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kCosDim; ++j)
        ss = __dadd_rn(ss, __dmul_rn(static_cast<double>(c[j]), static_cast<double>(c[j])));
    double norm = __builtin_sqrt(ss);
    if (norm < 1e-12) norm = 1e-12;
#pragma unroll
    for (int j = 0; j < kCosDim; ++j) units[r * kCosDim + j] = static_cast<double>(c[j]) / norm;
}

struct Update8 {
    const int32_t *codes;   // previous stage's column; row n at codes[n * ld]
    int ld;
    const float *table;     // previous stage's [n_codes, hidden] projected codewords
    int n_codes;
    float *dst;             // [N, hidden] updated residual
};

// y[n, 0..7] = W r_n + bias, W [8, hidden]; one wavefront per frame with
// lanes over float4 columns of the row (fully coalesced 1 KiB loads). W is
// staged once per workgroup in LDS (32 KiB at hidden 1024) and read per
// frame as contiguous 1 KiB rows (conflict-free), which keeps the kernel at
// about 50 VGPRs so that many wavefronts hide the memory latency of the
// residual rows. Partial sums are reduced by a butterfly that halves the
// number of outputs each lane carries. With kUpdate the previous stage's
// residual update is applied first: r = fl32(src - table[code]) is stored
// to up.dst (which may be src) and projected. Waves stride over the frames.
constexpr int kProjMaxHidden = 1024;

template <int kT, bool kBias, bool kUpdate>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kProjWaves, 64 * kProjWaves),
                          amdgpu_waves_per_eu(5)))   // 5 workgroups of 32 KiB LDS per CU
void proj8_kernel(const float *src, int64_t n_frames, int hidden, const float *__restrict__ w,
                  const float *__restrict__ bias, float *__restrict__ y, Update8 up)
{
    // W rows at a fixed stride, zero past `hidden`, so a lane's 8 reads per
    // column block differ only by immediate offsets and need no guard
    __shared__ __align__(16) float s_w[kCosDim * kProjMaxHidden];
    {
        const int c4s = hidden >> 2;
        for (int i = threadIdx.x; i < kCosDim * 64 * kT; i += 64 * kProjWaves) {
            const int o = i / (64 * kT), c4 = i - o * (64 * kT);
            *reinterpret_cast<f32x4 *>(&s_w[o * kProjMaxHidden + 4 * c4]) =
                c4 < c4s ? reinterpret_cast<const f32x4 *>(w)[o * c4s + c4] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int cols = hidden >> 2;   // float4 columns per row
    const int out_id = 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
    const float b_out = kBias ? bias[out_id] : 0.0f;
    const float nan = __builtin_nanf("");
    // column of block t: lane + 64 t; past the row it reads the last column
    // (always in bounds) and contributes 0
    int ccol[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) ccol[t] = min(lane + 64 * t, cols - 1);

    const int64_t stride = static_cast<int64_t>(gridDim.x) * kProjWaves;
    for (int64_t n = static_cast<int64_t>(blockIdx.x) * kProjWaves + (threadIdx.x >> 6); n < n_frames; n += stride) {
        // keeps the W reads inside the loop: hoisted, they would pin 32 kT VGPRs
        asm volatile("" ::: "memory");
        const float *row = src + n * hidden;
        f32x4 r[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) r[t] = *reinterpret_cast<const f32x4 *>(row + 4 * ccol[t]);
        if (kUpdate) {
            int k = up.codes[n * up.ld];
            const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(up.n_codes);
            k = ok ? k : 0;
            const float *prow = up.table + static_cast<int64_t>(k) * hidden;
            float *drow = up.dst + n * hidden;
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                const f32x4 p = *reinterpret_cast<const f32x4 *>(prow + 4 * ccol[t]);
#pragma unroll
                for (int e = 0; e < 4; ++e) r[t][e] = ok ? r[t][e] - p[e] : nan;
                if (lane + 64 * t < cols) *reinterpret_cast<f32x4 *>(drow + 4 * ccol[t]) = r[t];
            }
        }
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const bool in_row = lane + 64 * t < cols;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[t][e] = in_row ? r[t][e] : 0.0f;
        }
        float a[kCosDim];
#pragma unroll
        for (int o = 0; o < kCosDim; ++o) a[o] = 0.0f;
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            // one float4 column block at a time: 8 weight float4s live, not 8 kT
            f32x4 wv[kCosDim];
#pragma unroll
            for (int o = 0; o < kCosDim; ++o)
                wv[o] = *reinterpret_cast<const f32x4 *>(&s_w[o * kProjMaxHidden + 4 * (lane + 64 * t)]);
#pragma unroll
            for (int o = 0; o < kCosDim; ++o)
#pragma unroll
                for (int e = 0; e < 4; ++e) a[o] = __builtin_fmaf(wv[o][e], r[t][e], a[o]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // butterfly: after the xor-32, -16 and -8 steps lane l carries output out_id(l) only
        float b[4], c[2];
        const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float give = hi32 ? a[i] : a[i + 4];
            const float got = __shfl_xor(give, 32);
            b[i] = (hi32 ? a[i + 4] : a[i]) + got;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float give = hi16 ? b[i] : b[i + 2];
            const float got = __shfl_xor(give, 16);
            c[i] = (hi16 ? b[i + 2] : b[i]) + got;
        }
        float d;
        {
            const float give = hi8 ? c[0] : c[1];
            const float got = __shfl_xor(give, 8);
            d = (hi8 ? c[1] : c[0]) + got;
        }
        d += __shfl_xor(d, 4);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 1);
        if ((lane & 7) == 0) y[n * kCosDim + out_id] = kBias ? d + b_out : d;
    }
}

// Float64 distance of the unit encoding u to unit codeword k, the oracle's form.
__device__ inline double unit_distance(const double (&u)[kCosDim], const double *units, int k)
{
    const double *v = units + static_cast<int64_t>(k) * kCosDim;
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kCosDim; ++j) {
        const double t = __dadd_rn(u[j], -v[j]);
        acc = __dadd_rn(acc, __dmul_rn(t, t));
    }
    return acc;
}

// One frame per thread: fp32 scores against the stage's unit codewords
// (staged through LDS), then a float64 rescan by the whole wavefront for
// every frame whose two lowest scores are too close to call.
__global__ __launch_bounds__(256)
void cosine_argmin_kernel(const float *__restrict__ lat, int64_t n_frames, const double *__restrict__ units,
                          int n_codes, int32_t *__restrict__ codes, int codes_ld)
{
    __shared__ __align__(16) float s_v[kArgChunk * kCosDim];
    __shared__ float s_hn[kArgChunk];
    const int lane = threadIdx.x & 63;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const bool valid = frame < n_frames;
    float e[kCosDim];
    {
        const float *p = lat + (valid ? frame : 0) * kCosDim;
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            e[j] = lo[j];
            e[j + 4] = hi[j];
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kCosDim; ++j) ss = __builtin_fmaf(e[j], e[j], ss);
    // outside this range the fp32 norm may under- or overflow: decide in float64
    const bool norm_ok = ss >= 1e-30f && ss <= 1e30f;
    const float inv = 1.0f / fmaxf(__builtin_sqrtf(ss), 1e-12f);
    float nu[kCosDim];   // -u32
#pragma unroll
    for (int j = 0; j < kCosDim; ++j) nu[j] = -(e[j] * inv);

    float best = INFINITY, second = INFINITY;
    int bk = 0;
    for (int k0 = 0; k0 < n_codes; k0 += kArgChunk) {
        const int kn = min(kArgChunk, n_codes - k0);
        __syncthreads();   // the previous chunk is no longer read
        if (threadIdx.x < kn) {
            const double *v = units + static_cast<int64_t>(k0 + threadIdx.x) * kCosDim;
            float hn = 0.0f;
#pragma unroll
            for (int j = 0; j < kCosDim; ++j) {
                const float vj = static_cast<float>(v[j]);
                s_v[threadIdx.x * kCosDim + j] = vj;
                hn = __builtin_fmaf(vj, vj, hn);
            }
            s_hn[threadIdx.x] = 0.5f * hn;
        }
        __syncthreads();
        for (int kk = 0; kk < kn; ++kk) {
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(&s_v[kk * kCosDim]);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(&s_v[kk * kCosDim + 4]);
            float s = s_hn[kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) s = __builtin_fmaf(nu[j], v0[j], s);
#pragma unroll
            for (int j = 0; j < 4; ++j) s = __builtin_fmaf(nu[j + 4], v1[j], s);
            if (s < best) {
                second = best;
                best = s;
                bk = k0 + kk;
            } else if (s < second) {
                second = s;
            }
        }
    }
    bool ambiguous = valid && (!norm_ok || !(second - best > kAmbiguous));

    // float64 rescan, one ambiguous frame at a time, by the whole wavefront
    uint64_t mask = __ballot(ambiguous);
    while (mask) {
        const int srcl = __builtin_ctzll(mask);
        mask &= mask - 1;
        double u[kCosDim];
        double uss = 0.0;
#pragma unroll
        for (int j = 0; j < kCosDim; ++j) {
            const double ej = static_cast<double>(__shfl(e[j], srcl));
            u[j] = ej;
            uss = __dadd_rn(uss, __dmul_rn(ej, ej));
        }
        double norm = __builtin_sqrt(uss);
        if (norm < 1e-12) norm = 1e-12;
#pragma unroll
        for (int j = 0; j < kCosDim; ++j) u[j] = u[j] / norm;
        double bd = INFINITY;
        int bi = 0x7fffffff;
        for (int k = lane; k < n_codes; k += 64) {   // k ascends per lane: strict "<" keeps the lowest
            const double d = unit_distance(u, units, k);
            if (d < bd) {
                bd = d;
                bi = k;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double od = __shfl_xor(bd, off);
            const int oi = __shfl_xor(bi, off);
            if (od < bd || (od == bd && oi < bi)) {
                bd = od;
                bi = oi;
            }
        }
        if (lane == srcl) bk = bi;
    }
    // a non-finite projection finds no smaller distance and keeps the
    // sentinel: its (unspecified) code is clamped so that the next stage's
    // update reads a real table row
    if (valid) codes[frame * codes_ld] = min(max(bk, 0), n_codes - 1);
}

// ---- all stages in one kernel --------------------------------------------
//
// For codebooks of at most 1024 entries and hidden <= 1024 the whole loop
// runs in one kernel: a workgroup of 8 wavefronts owns 32 frames, each
// wavefront 4 of them with their hidden-width residual rows in VGPRs for all
// stages, so the residual crosses HBM once in and once out instead of twice
// per stage. Per stage the workgroup stages W_in[q] (padded row stride, zero
// past `hidden`) and the stage's unit codewords in fp32 with their half
// norms in LDS; every LDS value is then used for the 4 frames of a
// wavefront. The in-projection and the scores run on the fp32 matrix cores
// (v_mfma_f32_4x4x1f32, layout below); each lane keeps best / second keys
// of its frame for each of its 4 codeword rows, merged over the frame's 16
// lanes. The exactness rule and the float64 rescan are those of
// cosine_argmin_kernel: a matrix-core step may round its product and its
// sum separately (the 9-term sums measured within 3.4u of exact on 4 M
// random operands), at most 2u per step more than the fused chain's 24u
// worst case, so a score stays within 42u of its exact value. The
// residual update gathers the table row of the pick (r <- fl32(r - P[q, k]));
// the next stage's LDS contents are staged while the picks are decided and
// those rows are in flight, and at most 128 registers keep four wavefronts
// per SIMD, so other wavefronts' products hide the gathers' latency.
// The float held by lane `src` (a constant) on every lane; the readlane
// builtin moves 32-bit integers, so the value travels as its bit pattern.
__device__ __forceinline__ float lane_value(float v, int src)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

constexpr int kFusedWaves = 8;
constexpr int kFusedFrames = 4;           // frames per wavefront
constexpr int kFusedMaxCodes = 1024;
constexpr int kWRow = kProjMaxHidden + 16;   // LDS row stride of W_in: conflict-free operand reads

// Lane l = 4 b + j of a wavefront (block b = 0..15, j = 0..3) works on frame
// j of the wavefront's 4. It holds that frame's residual columns
// 64 t + 4 b .. 64 t + 4 b + 3 (t < hidden / 64), which are the columns block
// b of a v_mfma_f32_4x4x1f32 takes: that instruction multiplies, in each of
// its 16 blocks of 4 lanes, a 4-vector held one entry per lane (A: lane
// 4 b + i holds row i) by another (B: lane 4 b + j holds column j) and adds
// the outer product to a 4x4 accumulator of which lane 4 b + j holds column j
// (register i = row i).
//   in-projection: rows = outputs (0..3, then 4..7), columns = frames, one
//     hidden column per block and instruction; the 16 blocks' partial sums
//     are then added over the wavefront;
//   scores: rows = codewords 64 s + 4 b + i, columns = frames, one codebook
//     dimension per instruction, the accumulator starting at the half norms.
template <int kT4, bool kBias>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kFusedWaves, 64 * kFusedWaves),
                          amdgpu_waves_per_eu(4)))   // <= 128 registers: two workgroups per CU
void cosine_fused_kernel(const float *__restrict__ h, int64_t n_frames, int hidden,
                         const float *__restrict__ w_in, const float *__restrict__ b_in,
                         const double *__restrict__ units, const float *__restrict__ table,
                         int n_stages, int n_codes, int32_t *__restrict__ codes, int codes_ld,
                         float *__restrict__ latent, float *__restrict__ residual)
{
    constexpr int kT = 4 * kT4;   // column groups of 64 (past hidden: zero rows of W, zero residual)
    __shared__ __align__(16) float s_w[kCosDim * kWRow];
    __shared__ __align__(16) float s_vlo[kFusedMaxCodes * 4];   // unit codewords, dims 0..3
    __shared__ __align__(16) float s_vhi[kFusedMaxCodes * 4];   // dims 4..7
    __shared__ __align__(16) float s_hn[kFusedMaxCodes];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 3;    // frame of this lane; also row i of the A operand
    const int b = lane >> 2;   // block
    const int64_t frame0 = (static_cast<int64_t>(blockIdx.x) * kFusedWaves + wave) * kFusedFrames;
    const int64_t fr = frame0 + j;
    const bool valid = fr < n_frames;
    const int n_col = hidden >> 6;   // column groups in the rows (wave-uniform)

    // residual columns 64 t + 4 b .. +3 of frame j (read and written once,
    // non-temporally: the cache is left to the table rows gathered every stage)
    f32x4 r[kT];
    {
        const float *row = h + (valid ? fr : 0) * hidden + 4 * b;
#pragma unroll
        for (int t = 0; t < kT; ++t)
            r[t] = (valid && t < n_col) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 64 * t))
                                        : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // after the block reduction lane l holds output o(l) = 4 l5 + 2 l4 + l3 of frame l & 3
    const int out_id = 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
    const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8;
    const int n_slots = (n_codes + 63) / 64;   // codeword 64 s + 4 b + i, s < n_slots

    // stage q's W_in rows and unit codewords into LDS
    auto stage_lds = [&](int q) {
        {
            const float *wq = w_in + static_cast<int64_t>(q) * kCosDim * hidden;
            const int c4s = hidden >> 2;
            for (int i = threadIdx.x; i < kCosDim * 16 * kT; i += 64 * kFusedWaves) {
                const int o = i / (16 * kT), c4 = i - o * (16 * kT);
                *reinterpret_cast<f32x4 *>(&s_w[o * kWRow + 4 * c4]) =
                    c4 < c4s ? reinterpret_cast<const f32x4 *>(wq)[o * c4s + c4] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            const double *uq = units + static_cast<int64_t>(q) * n_codes * kCosDim;
            for (int k = threadIdx.x; k < 64 * n_slots; k += 64 * kFusedWaves) {
                float v[kCosDim];
                float hn = FLT_MAX;   // slots past n_codes never win
#pragma unroll
                for (int d = 0; d < kCosDim; ++d) v[d] = 0.0f;
                if (k < n_codes) {
                    hn = 0.0f;
#pragma unroll
                    for (int d = 0; d < kCosDim; ++d) {
                        v[d] = static_cast<float>(uq[static_cast<int64_t>(k) * kCosDim + d]);
                        hn = __builtin_fmaf(v[d], v[d], hn);
                    }
                    hn = 0.5f * hn;
                }
                *reinterpret_cast<f32x4 *>(&s_vlo[4 * k]) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(&s_vhi[4 * k]) = f32x4{v[4], v[5], v[6], v[7]};
                s_hn[k] = hn;
            }
        }
    };
    stage_lds(0);
    __syncthreads();

    for (int q = 0; q < n_stages; ++q) {
        // ---- in-projection on the matrix cores ----
        f32x4 p_lo = {0.0f, 0.0f, 0.0f, 0.0f}, p_hi = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const f32x4 wl = *reinterpret_cast<const f32x4 *>(&s_w[j * kWRow + 64 * t + 4 * b]);
            const f32x4 wh = *reinterpret_cast<const f32x4 *>(&s_w[(j + 4) * kWRow + 64 * t + 4 * b]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p_lo = __builtin_amdgcn_mfma_f32_4x4x1f32(wl[e], r[t][e], p_lo, 0, 0, 0);
                p_hi = __builtin_amdgcn_mfma_f32_4x4x1f32(wh[e], r[t][e], p_hi, 0, 0, 0);
            }
            // one column group's weights live at a time
            __builtin_amdgcn_sched_barrier(0);
        }
        // sum over the 16 blocks: a butterfly that halves the outputs each lane carries
        float ev;
        {
            float c[4], d2[2];
            const float a[8] = {p_lo[0], p_lo[1], p_lo[2], p_lo[3], p_hi[0], p_hi[1], p_hi[2], p_hi[3]};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float give = hi32 ? a[m] : a[m + 4];
                c[m] = (hi32 ? a[m + 4] : a[m]) + __shfl_xor(give, 32);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float give = hi16 ? c[m] : c[m + 2];
                d2[m] = (hi16 ? c[m + 2] : c[m]) + __shfl_xor(give, 16);
            }
            const float give = hi8 ? d2[0] : d2[1];
            ev = (hi8 ? d2[1] : d2[0]) + __shfl_xor(give, 8);
            ev += __shfl_xor(ev, 4);
            if (kBias) ev += b_in[q * kCosDim + out_id];
        }
        // this lane's frame's 8 projections: output o of frame j sits in lane
        // 32 o2 + 16 o1 + 8 o0 + j
        float e8[kCosDim];
#pragma unroll
        for (int o = 0; o < kCosDim; ++o) e8[o] = __shfl(ev, 32 * ((o >> 2) & 1) + 16 * ((o >> 1) & 1) + 8 * (o & 1) + j);
        if (valid && (lane & 4) == 0)
            latent[(static_cast<int64_t>(q) * n_frames + fr) * kCosDim + out_id] = ev;
        float ss = 0.0f;
#pragma unroll
        for (int o = 0; o < kCosDim; ++o) ss = __builtin_fmaf(e8[o], e8[o], ss);
        // outside [1e-30, 1e30] the float64 rescan decides; inside, 1/sqrt
        // within 1 ulp keeps every element of u within 8u
        const bool norm_ok = ss >= 1e-30f && ss <= 1e30f;
        const float inv = __builtin_amdgcn_rsqf(norm_ok ? ss : 1.0f);
        float nu[kCosDim];   // -u32 of frame j
#pragma unroll
        for (int o = 0; o < kCosDim; ++o) nu[o] = -(e8[o] * inv);

        // ---- scores on the matrix cores: per lane, codewords 64 s + 4 b + i of frame j ----
        // keys: the score with its 4 low mantissa bits replaced by s, kept per i
        float best[4], second[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            best[i] = INFINITY;
            second[i] = INFINITY;
        }
        for (int sl = 0; sl < n_slots; ++sl) {
            const int k = 64 * sl + 4 * b + j;   // this lane's A row: codeword 64 s + 4 b + (lane & 3)
            const f32x4 vl = *reinterpret_cast<const f32x4 *>(&s_vlo[4 * k]);
            const f32x4 vh = *reinterpret_cast<const f32x4 *>(&s_vhi[4 * k]);
            f32x4 sc = *reinterpret_cast<const f32x4 *>(&s_hn[64 * sl + 4 * b]);
#pragma unroll
            for (int d = 0; d < 4; ++d) sc = __builtin_amdgcn_mfma_f32_4x4x1f32(vl[d], nu[d], sc, 0, 0, 0);
#pragma unroll
            for (int d = 0; d < 4; ++d) sc = __builtin_amdgcn_mfma_f32_4x4x1f32(vh[d], nu[4 + d], sc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float key = __uint_as_float((__float_as_uint(sc[i]) & ~15u) | static_cast<unsigned>(sl));
                second[i] = __builtin_amdgcn_fmed3f(key, best[i], second[i]);
                best[i] = __builtin_amdgcn_fmed3f(key, best[i], -FLT_MAX);   // min (keys are finite)
            }
        }

        // the next stage's LDS contents are staged while this stage's picks are
        // decided and their table rows fetched
        __syncthreads();   // every wavefront has read this stage's LDS contents
        if (q + 1 < n_stages) stage_lds(q + 1);

        // ---- per frame: argmin over the wavefront's 16 lanes of the frame ----
        float bv = fminf(fminf(best[0], best[1]), fminf(best[2], best[3]));
        float sv;
        {
            // second smallest of the 8 (best, second) keys of this lane
            const float m01 = fmaxf(best[0], best[1]), m23 = fmaxf(best[2], best[3]);
            const float lo01 = fminf(best[0], best[1]), lo23 = fminf(best[2], best[3]);
            sv = fminf(fminf(fminf(second[0], second[1]), fminf(second[2], second[3])),
                       fminf(fminf(m01, m23), fmaxf(lo01, lo23)));
        }
        const float own = bv;
#pragma unroll
        for (int off = 4; off < 64; off <<= 1) {
            const float ob = __shfl_xor(bv, off);
            const float os = __shfl_xor(sv, off);
            sv = fminf(fminf(sv, os), fmaxf(bv, ob));
            bv = fminf(bv, ob);
        }
        // the codeword of the smallest key: the lowest block, then the lowest i,
        // holding it (equal keys share the slot bits, so that is the lowest codeword)
        int li = 4;
#pragma unroll
        for (int i = 3; i >= 0; --i) li = best[i] == bv ? i : li;
        const bool ambiguous = valid && (!norm_ok || !(sv - bv > kKeyAmbiguous));
        const uint64_t amb = __ballot(ambiguous);
        const uint64_t has = __ballot(own == bv);
        int pick_of[kFusedFrames];
#pragma unroll
        for (int f = 0; f < kFusedFrames; ++f) {
            const uint64_t m = has & (0x1111111111111111ull << f);
            const int wl = m ? __ffsll(static_cast<unsigned long long>(m)) - 1 : f;
            const int slot = static_cast<int>(__float_as_uint(lane_value(bv, f)) & 15u);
            pick_of[f] = 64 * slot + 4 * (wl >> 2) + __builtin_amdgcn_readlane(li, wl);
            if ((amb >> f) & 1ull) {   // wave-uniform: the float64 rescan of the oracle's formula
                double u[kCosDim];
                double uss = 0.0;
#pragma unroll
                for (int o = 0; o < kCosDim; ++o) {
                    // output o of frame f, where the block sum left it
                    const double eo = static_cast<double>(
                        lane_value(ev, 32 * ((o >> 2) & 1) + 16 * ((o >> 1) & 1) + 8 * (o & 1) + f));
                    u[o] = eo;
                    uss = __dadd_rn(uss, __dmul_rn(eo, eo));
                }
                double norm = __builtin_sqrt(uss);
                if (norm < 1e-12) norm = 1e-12;
#pragma unroll
                for (int o = 0; o < kCosDim; ++o) u[o] = u[o] / norm;
                const double *uq = units + static_cast<int64_t>(q) * n_codes * kCosDim;
                double bd = INFINITY;
                int bkk = 0x7fffffff;
                for (int k = lane; k < n_codes; k += 64) {   // k ascends per lane: strict "<" keeps the lowest
                    const double dd = unit_distance(u, uq, k);
                    if (dd < bd) {
                        bd = dd;
                        bkk = k;
                    }
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const double od = __shfl_xor(bd, off);
                    const int oi = __shfl_xor(bkk, off);
                    if (od < bd || (od == bd && oi < bkk)) {
                        bd = od;
                        bkk = oi;
                    }
                }
                pick_of[f] = bkk;
            }
            // a non-finite frame's pick is unspecified; clamped, so that the
            // table row read below exists
            pick_of[f] = __builtin_amdgcn_readfirstlane(min(max(pick_of[f], 0), n_codes - 1));
        }
        const int pick = j == 0 ? pick_of[0] : j == 1 ? pick_of[1] : j == 2 ? pick_of[2] : pick_of[3];
        if (valid && b == 0) codes[fr * codes_ld + q] = pick;
        // r <- fl32(r - P[q, pick]) over this lane's columns
        const float *prow = table + (static_cast<int64_t>(q) * n_codes + pick) * hidden + 4 * b;
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            if (t < n_col) {
                const f32x4 pv = *reinterpret_cast<const f32x4 *>(prow + 64 * t);
#pragma unroll
                for (int e = 0; e < 4; ++e) r[t][e] = r[t][e] - pv[e];
            }
        }
        __syncthreads();   // the next stage's LDS contents are in place
    }

    if (valid) {
        float *row = residual + fr * hidden + 4 * b;
#pragma unroll
        for (int t = 0; t < kT; ++t)
            if (t < n_col) __builtin_nontemporal_store(r[t], reinterpret_cast<f32x4 *>(row + 64 * t));
    }
}

template <int kT4>
hipError_t launch_fused_t(const float *h, int64_t n_frames, int hidden, const float *w_in, const float *b_in,
                          const double *units, const float *table, int n_stages, int n_codes, int32_t *codes,
                          int codes_ld, float *latent, float *residual, hipStream_t stream)
{
    const int64_t per_block = static_cast<int64_t>(kFusedWaves) * kFusedFrames;
    const int64_t blocks = (n_frames + per_block - 1) / per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kFusedWaves);
    if (b_in)
        hipLaunchKernelGGL((cosine_fused_kernel<kT4, true>), grid, block, 0, stream, h, n_frames, hidden, w_in, b_in,
                           units, table, n_stages, n_codes, codes, codes_ld, latent, residual);
    else
        hipLaunchKernelGGL((cosine_fused_kernel<kT4, false>), grid, block, 0, stream, h, n_frames, hidden, w_in,
                           b_in, units, table, n_stages, n_codes, codes, codes_ld, latent, residual);
    return hipGetLastError();
}

template <int kT>
hipError_t launch_proj8_t(const float *src, int64_t n_frames, int hidden, const float *w, const float *bias,
                          float *y, const Update8 &up, bool update, hipStream_t stream)
{
    const int64_t waves = (n_frames + 7) / 8;   // about 8 frames per wavefront, capped below
    int64_t blocks = (waves + kProjWaves - 1) / kProjWaves;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kProjWaves);
    if (update) {
        if (bias)
            hipLaunchKernelGGL((proj8_kernel<kT, true, true>), grid, block, 0, stream, src, n_frames, hidden, w, bias, y, up);
        else
            hipLaunchKernelGGL((proj8_kernel<kT, false, true>), grid, block, 0, stream, src, n_frames, hidden, w, bias, y, up);
    } else {
        if (bias)
            hipLaunchKernelGGL((proj8_kernel<kT, true, false>), grid, block, 0, stream, src, n_frames, hidden, w, bias, y, up);
        else
            hipLaunchKernelGGL((proj8_kernel<kT, false, false>), grid, block, 0, stream, src, n_frames, hidden, w, bias, y, up);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cosine_units(const float *books, int n_stages, int n_codes, double *units, hipStream_t stream)
{
    const int64_t rows = static_cast<int64_t>(n_stages) * n_codes;
    const int64_t blocks = (rows + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(units_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, books, rows, units);
    return hipGetLastError();
}

hipError_t launch_proj8(const float *src, const int32_t *prev_codes, int codes_ld, const float *prev_table,
                        int n_codes, float *dst, int64_t n_frames, int hidden, const float *w, const float *bias,
                        float *y, hipStream_t stream)
{
    const Update8 up = {prev_codes, codes_ld, prev_table, n_codes, dst};
    const bool update = prev_codes != nullptr;
    const int t = (hidden + 255) / 256;
    switch (t) {
    case 1: return launch_proj8_t<1>(src, n_frames, hidden, w, bias, y, up, update, stream);
    case 2: return launch_proj8_t<2>(src, n_frames, hidden, w, bias, y, up, update, stream);
    case 3: return launch_proj8_t<3>(src, n_frames, hidden, w, bias, y, up, update, stream);
    case 4: return launch_proj8_t<4>(src, n_frames, hidden, w, bias, y, up, update, stream);
    default: return hipErrorInvalidValue;
    }
}

bool cosine_fused_supported(int n_codes, int hidden) { return n_codes <= kFusedMaxCodes && hidden <= kProjMaxHidden; }

hipError_t launch_cosine_fused(const float *h, int64_t n_frames, int hidden, const float *w_in, const float *b_in,
                               const double *units, const float *table, int n_stages, int n_codes, int32_t *codes,
                               int codes_ld, float *latent, float *residual, hipStream_t stream)
{
    if (!cosine_fused_supported(n_codes, hidden)) return hipErrorInvalidValue;
    switch ((hidden + 255) / 256) {
    case 1: return launch_fused_t<1>(h, n_frames, hidden, w_in, b_in, units, table, n_stages, n_codes, codes, codes_ld, latent, residual, stream);
    case 2: return launch_fused_t<2>(h, n_frames, hidden, w_in, b_in, units, table, n_stages, n_codes, codes, codes_ld, latent, residual, stream);
    case 3: return launch_fused_t<3>(h, n_frames, hidden, w_in, b_in, units, table, n_stages, n_codes, codes, codes_ld, latent, residual, stream);
    case 4: return launch_fused_t<4>(h, n_frames, hidden, w_in, b_in, units, table, n_stages, n_codes, codes, codes_ld, latent, residual, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cosine_argmin(const float *lat, int64_t n_frames, const double *units, int n_codes,
                                int32_t *codes, int codes_ld, hipStream_t stream)
{
    const int64_t blocks = (n_frames + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cosine_argmin_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, lat,
                       n_frames, units, n_codes, codes, codes_ld);
    return hipGetLastError();
}

}  // namespace rvq
