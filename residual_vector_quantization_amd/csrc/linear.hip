// Linear layers around the quantizer on the matrix cores, gfx950 (CDNA4).
//
// The "Audio tokenizer pipeline" section of the "Architecture" page
// (omnivoice.cpp) puts a linear layer before the RVQ encode (fc) and one
// after the decode (fc2). The projected workload uses fc: hidden -> 64 and
// fc2: 64 -> hidden, weights in PyTorch (out, in) order:
//
//   linear_in : y[n, i]  = sum_k h[n, k] * W_in[i, k]  + b_in[i]   (i < 64)
//   linear_out: o[n, i]  = sum_k x[n, k] * W_out[i, k] + b_out[i]  (k < 64)
//
// linear_in runs on the bf16 matrix cores with fp32 accuracy: every fp32
// operand v is split into three bf16 parts, v = v_h + v_m + v_l exactly
// (v_h = bf16(v), v_m = bf16(v - v_h), v_l = bf16(v - v_h - v_m), each
// difference exact; for normal values v_l holds the last bits), and a
// product v w is summed as v_h w_l + v_l w_h + v_m w_m + v_h w_m + v_m w_h
// + v_h w_h (bf16 x bf16 products are exact in fp32). The dropped
// v_m w_l + v_l w_m + v_l w_l are at most 2^-23 |v w|, the size of one fp32
// rounding, so the result is as accurate as an fp32 contraction; six
// v_mfma_f32_32x32x16_bf16 do the work of eight fp32 32x32x2 steps. fc2,
// whose frame operand and weight tiles are small enough to scale by a
// power of two before splitting, takes a two-part fp16 split instead
// (three v_mfma_f32_32x32x16_f16 per step, each product within
// 3.01 * 2^-22 of exact; bound below) and makes its stores line-wide
// through LDS: linear_out_res_kernel (weights resident in registers) for
// hidden a multiple of 512, linear_out_split_kernel for other multiples of
// 32; linear_out_kernel, on v_mfma_f32_32x32x2_f32, remains for hidden
// sizes that are not a multiple of 32.
//
// linear_in and the fp32 linear_out_kernel put weight rows on the M side and
// 32 frames per wavefront on the N side, stream the weights through LDS
// (padded rows, double buffered, shared by the wavefronts of a workgroup;
// split into 8-column groups of 8 high, 8 middle and 8 low parts for
// linear_in) and keep the frame operand in VGPRs; linear_out_split_kernel
// (below) has every wavefront load and split its own weight tiles and
// carries two 32-frame groups. Lanes 0-31 supply one 32-wide half of each
// 64-wide chunk of the contraction, lanes 32-63 the other (one 8-wide half
// of each 16-wide step in the split fc2). Results are fp32 sums in the
// matrix core's order, the bias added last (in fc2 with the scale undone in
// the same rounding).
#include <stdint.h>

#include <algorithm>

#include <hip/hip_runtime.h>

#include "rvq_internal.h"

namespace rvq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFramesPerWave = 32;
constexpr int kInWaves = 8;                          // linear_in: 256 frames per workgroup
constexpr int kInFrames = kInWaves * kFramesPerWave;
constexpr int kOutWaves = 4;                         // linear_out: 128 frames per workgroup
constexpr int kOutFrames = kOutWaves * kFramesPerWave;
constexpr int kRow = 64 + 4;        // padded fp32 LDS row: 8 lanes of a b128 read hit 32 banks
constexpr int kSRow = 3 * 64 + 8;   // bf16 per split weight row: 8 groups of (8 h, 8 m, 8 l) + 16 B pad

// The three bf16 parts of 8 consecutive fp32 values.
struct Split3 {
    bf16x8 h, m, l;
};

// v = h + m + l exactly: each part is the round-to-nearest bf16 of what the
// previous ones leave, and each difference is exact in fp32. Converted two
// values at a time; a part is widened back by placing its 16 bits at the
// top of a word.
__device__ __forceinline__ Split3 split3(const float *v)
{
    u32x4 hp, mp, lp;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{v[2 * p], v[2 * p + 1]}, bf16x2));
        const float r0 = v[2 * p] - __uint_as_float(h << 16);
        const float r1 = v[2 * p + 1] - __uint_as_float(h & 0xFFFF0000u);
        const unsigned m = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
        const float s0 = r0 - __uint_as_float(m << 16);
        const float s1 = r1 - __uint_as_float(m & 0xFFFF0000u);
        hp[p] = h;
        mp[p] = m;
        lp[p] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{s0, s1}, bf16x2));
    }
    return {__builtin_bit_cast(bf16x8, hp), __builtin_bit_cast(bf16x8, mp), __builtin_bit_cast(bf16x8, lp)};
}

// acc += a . b over one 16-wide step of the contraction, in six products.
__device__ __forceinline__ void mfma6(f32x16 &acc, const Split3 &a, const Split3 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.h, b.l, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.l, b.h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.m, b.m, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.h, b.m, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.m, b.h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.h, b.h, acc, 0, 0, 0);
}

// Split weight row r of an LDS chunk: group g (columns 8g .. 8g+7) at
// row * kSRow + 24 g as (h, m, l).
__device__ __forceinline__ Split3 lds_split(const __bf16 *chunk, int row, int g)
{
    const __bf16 *p = chunk + row * kSRow + 24 * g;
    return {*reinterpret_cast<const bf16x8 *>(p), *reinterpret_cast<const bf16x8 *>(p + 8),
            *reinterpret_cast<const bf16x8 *>(p + 16)};
}

__device__ __forceinline__ void lds_store_split(__bf16 *chunk, int row, int g, const Split3 &s)
{
    __bf16 *p = chunk + row * kSRow + 24 * g;
    *reinterpret_cast<bf16x8 *>(p) = s.h;
    *reinterpret_cast<bf16x8 *>(p + 8) = s.m;
    *reinterpret_cast<bf16x8 *>(p + 16) = s.l;
}

// ---- linear_in: [N, hidden] x [64, hidden]^T -> [N, 64] -------------------

// Each wavefront loads its 32 frames chunk by chunk (64 columns) with
// coalesced 1 KiB row loads into a padded LDS tile, and reads the tile back
// in the matrix-core operand layout (lane (col, half): frame col, columns
// 32 half .. 32 half + 31 of the chunk). The residual update of the
// previous stage of a per-stage projected quantizer can ride along
// (kUpdate): the table row of each frame's previous code is subtracted
// from the loaded chunk, r <- fl32(r - P[code]), and the result is stored
// to `dst` (which may be `h` itself: every element is loaded, then stored,
// by the same lane) and used as the operand. A code outside [0, n_codes)
// makes the row NaN.
struct Update {
    const int32_t *codes;   // previous stage's column; row n at codes[n * ld]
    int ld;
    const float *table;     // previous stage's [n_codes, hidden] projected codewords
    int n_codes;
    float *dst;             // [N, hidden] updated residual
};

template <bool kBias, bool kUpdate>
__global__ __launch_bounds__(64 * kInWaves)
void linear_in_kernel(const float *h, int64_t n_frames, int hidden,
                      const float *__restrict__ w, const float *__restrict__ bias,
                      float *__restrict__ y, Update up)
{
    // one chunk = 64 weight rows (all outputs) x 64 columns of the hidden dim, split
    __shared__ __align__(16) __bf16 s_w[2][kDim * kSRow];
    // per wavefront: its 32 frames x 64 columns of the current chunk
    __shared__ __align__(16) float s_h[kInWaves][kFramesPerWave * kRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame0 = static_cast<int64_t>(blockIdx.x) * kInFrames + wave * kFramesPerWave;
    const int64_t frame = frame0 + col;
    const bool valid = frame < n_frames;

    // Tile loads are coalesced: load i covers frames 4i .. 4i+3 of the
    // wavefront, 16 lanes per frame, one float4 each (a 256 B row chunk).
    const int trow = lane >> 4;
    const int tc4 = lane & 15;
    int64_t roff[8];     // element offset of this lane's row in h / dst
    bool rvalid[8];
    const float *prow[8];   // kUpdate: table row of the frame's previous code
    unsigned bad = 0u;      // kUpdate: bit i: frame 4i + trow has a code outside [0, n_codes)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t fr = frame0 + 4 * i + trow;
        rvalid[i] = fr < n_frames;
        roff[i] = (rvalid[i] ? fr : 0) * static_cast<int64_t>(hidden) + 4 * tc4;
        if (kUpdate) {
            int k = up.codes[(rvalid[i] ? fr : 0) * up.ld];
            const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(up.n_codes);
            bad |= ok ? 0u : (1u << i);
            prow[i] = up.table + static_cast<int64_t>(ok ? k : 0) * hidden + 4 * tc4;
        }
    }

    // staging: wavefront w stages weight rows 8w..8w+7; lane -> (row, 8-column group)
    const int srow = wave * 8 + (lane & 7);
    const int sgrp = lane >> 3;
    const int n_chunks = hidden / 64;

    f32x4 ws[2];
    f32x4 hv[8], pv[8];
    auto fetch_w = [&](int c) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(w + static_cast<int64_t>(srow) * hidden + 64 * c + 8 * sgrp);
        ws[0] = p[0];
        ws[1] = p[1];
    };
    auto commit_w = [&](int buf) {
        const float v[8] = {ws[0][0], ws[0][1], ws[0][2], ws[0][3], ws[1][0], ws[1][1], ws[1][2], ws[1][3]};
        lds_store_split(s_w[buf], srow, sgrp, split3(v));
    };
    auto fetch_h = [&](int c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // read once: non-temporal, so that the rows do not displace cached
            // data (the per-stage quantizer's residual rows are read again by
            // its update and are left to the cache)
            const f32x4 *src = reinterpret_cast<const f32x4 *>(h + roff[i] + 64 * c);
            hv[i] = kUpdate ? *src : __builtin_nontemporal_load(src);
            if (kUpdate) pv[i] = *reinterpret_cast<const f32x4 *>(prow[i] + 64 * c);
        }
    };

    f32x16 acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.0f;

    fetch_w(0);
    commit_w(0);
    fetch_h(0);
    __syncthreads();

    float *tile = s_h[wave];
    const float nan = __builtin_nanf("");
    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        // this chunk's rows (updated: r - P[code], stored back) into the wavefront's tile
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f32x4 r = hv[i];
            if (kUpdate) {
                const bool ok = !((bad >> i) & 1u);
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = ok ? r[e] - pv[i][e] : nan;
                if (rvalid[i]) *reinterpret_cast<f32x4 *>(up.dst + roff[i] + 64 * c) = r;
            }
            *reinterpret_cast<f32x4 *>(&tile[(4 * i + trow) * kRow + 4 * tc4]) = r;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // this lane's operand: frame col, columns 32 half + 8 s .. + 7 in step s
        Split3 fs[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const f32x4 u = *reinterpret_cast<const f32x4 *>(&tile[col * kRow + 32 * half + 8 * st]);
            const f32x4 v = *reinterpret_cast<const f32x4 *>(&tile[col * kRow + 32 * half + 8 * st + 4]);
            const float e[8] = {u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
            fs[st] = split3(e);
        }
        if (c + 1 < n_chunks) {
            fetch_w(c + 1);
            fetch_h(c + 1);
        }
        const __bf16 *sb = s_w[buf];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const Split3 a0 = lds_split(sb, col, 4 * half + st);
            const Split3 a1 = lds_split(sb, 32 + col, 4 * half + st);
            mfma6(acc[0], a0, fs[st]);
            mfma6(acc[1], a1, fs[st]);
        }
        if (c + 1 < n_chunks) commit_w(buf ^ 1);
        // every lane has read the tile (and the weight buffer) before they are overwritten
        __syncthreads();
    }

    if (valid) {
        // accumulator v of block b in this lane is output 32b + 8*(v/4) + 4*half + v%4
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i0 = 32 * b + 8 * m + 4 * half;
                f32x4 o = {acc[b][4 * m], acc[b][4 * m + 1], acc[b][4 * m + 2], acc[b][4 * m + 3]};
                if (kBias) {
                    const f32x4 bb = *reinterpret_cast<const f32x4 *>(bias + i0);
                    o = o + bb;
                }
                *reinterpret_cast<f32x4 *>(y + frame * kDim + i0) = o;
            }
        }
    }
}

// ---- linear_out: [N, 64] x [hidden, 64]^T -> [N, hidden] ------------------

constexpr int kOutChunk = 128;   // weight rows (outputs) per LDS chunk

template <bool kBias>
__global__ __launch_bounds__(64 * kOutWaves)
void linear_out_kernel(const float *__restrict__ x, int64_t n_frames, int hidden,
                       const float *__restrict__ w, const float *__restrict__ bias,
                       float *__restrict__ out)
{
    __shared__ __align__(16) float s_w[2][kOutChunk * kRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame = static_cast<int64_t>(blockIdx.x) * kOutFrames +
                          wave * kFramesPerWave + col;
    const bool valid = frame < n_frames;

    float xv[32];
    if (valid) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(x + frame * kDim + 32 * half);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 v = src[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[4 * t + e] = v[e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) xv[j] = 0.0f;
    }

    // staging: wavefront w stages rows 32w..32w+31 of the chunk, lane -> (row, half)
    const int srow = wave * 32 + col;
    const int scol = half * 32;
    const int n_chunks = (hidden + kOutChunk - 1) / kOutChunk;
    f32x4 ws[8];
    auto fetch_w = [&](int c) {
        const int row = min(c * kOutChunk + srow, hidden - 1);
        const f32x4 *p = reinterpret_cast<const f32x4 *>(w + static_cast<int64_t>(row) * kDim + scol);
#pragma unroll
        for (int i = 0; i < 8; ++i) ws[i] = p[i];
    };
    auto commit_w = [&](int buf) {
        float *dst = &s_w[buf][srow * kRow + scol];
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4 *>(dst + 4 * i) = ws[i];
    };

    fetch_w(0);
    commit_w(0);
    __syncthreads();

    float *orow = out + (valid ? frame : 0) * static_cast<int64_t>(hidden);
    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < n_chunks) fetch_w(c + 1);
        const float *sb = s_w[buf];
#pragma unroll
        for (int pb = 0; pb < kOutChunk / 64; ++pb) {
            const int row0 = c * kOutChunk + pb * 64;
            if (row0 >= hidden) break;   // uniform: hidden is a multiple of 64
            f32x16 acc[2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[b][v] = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x4 a[2];
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    a[b] = *reinterpret_cast<const f32x4 *>(sb + (pb * 64 + b * 32 + col) * kRow + 32 * half + 4 * t);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[b][e], xv[4 * t + e], acc[b], 0, 0, 0);
            }
            if (valid) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int i0 = row0 + 32 * b + 8 * m + 4 * half;
                        f32x4 o = {acc[b][4 * m], acc[b][4 * m + 1], acc[b][4 * m + 2], acc[b][4 * m + 3]};
                        if (kBias) {
                            const f32x4 bb = *reinterpret_cast<const f32x4 *>(bias + i0);
                            o = o + bb;
                        }
                        *reinterpret_cast<f32x4 *>(orow + i0) = o;
                    }
                }
            }
        }
        if (c + 1 < n_chunks) commit_w(buf ^ 1);
        __syncthreads();
    }
}

// ---- linear_out on fp16 matrix cores in a scaled two-part split -----------
//
// The same contraction as linear_out_kernel. Every operand value is scaled
// by a power of two and split into two fp16 parts: with v' = 2^e v (exact),
// v_h = fp16(v') and v_l = fp16(v' - v_h) (the difference is exact in fp32),
// v' = v_h + v_l + d with |d| <= 2^-22 |v'| + 2^-25. A product x' w' is
// summed as x_l w_h + x_h w_l + x_h w_h (fp16 x fp16 products are exact in
// fp32); what is dropped, x_l w_l and the d terms, is at most
// 3.01 * 2^-22 |x' w'| + 2^-25 (|x'| + |w'|). The exponents put the largest
// magnitude of each frame's 64 values, and of each tile's 32 x 64 weights,
// in [2^14, 2^15): no part overflows, and the 2^-25 terms stay below 2^-37
// of the largest product of the frame and tile. So each output carries at
// most 3.01 * 2^-22 of sum |x_k w_k| beyond the fp32 accumulation's own
// error (a fifth of the worst-case bound of a 64-term fp32 sum), with three
// v_mfma_f32_32x32x16_f16 per 16-wide step instead of eight fp32 32x32x2
// products. The scale 2^-(e_frame + e_tile) is undone in the bias step:
// one fused multiply-add by an exact power of two, so the result is the
// accumulated sum scaled back and the bias added with one rounding (two
// steps instead where that power of two is not a float).
//
// The four wavefronts of a workgroup share 64 frames (two groups of 32)
// and take every fourth tile of 32 outputs, so that together they write
// neighbouring 128 B pieces of the same rows; each is otherwise independent
// (no barrier): it holds the split operand of both groups in VGPRs, and for
// each of its tiles loads the 32 weight rows' fp32 values of its lanes
// (128 B per lane, from L2) and splits them once for both groups, whose
// product chains are interleaved. Each 32x32 result goes through a
// wavefront-private LDS tile so that each store instruction writes 8 frames
// x 128 contiguous bytes (whole cache lines) instead of 32 frames x 32
// bytes.
//
// Loads and stores share one in-order completion counter, so a wait for a
// load issued after a store also waits for the store. The next tile's bias
// and weights are therefore requested before the current tile's products
// and stores, all rows of the transposed tile are read from LDS before any
// of them is stored, tiles go in pairs with the weight registers
// alternating, and the prefetches are unconditional (past the last tile
// they reload it): a wait for a tile's weights then leaves the stores
// issued after them in flight.
constexpr int kOutSplitWaves = 4;
constexpr int kOutGroups = 2;                              // groups of 32 frames per wavefront
constexpr int kOutWaveFrames = kOutGroups * kFramesPerWave;
constexpr int kTileRow = 36;   // floats per LDS tile row (32 outputs + pad)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct Split2 {
    f16x8 h, l;
};

template <bool kValue>
struct Flag {
    static constexpr bool value = kValue;
};

// 2^e v of 8 values in two fp16 parts (v_h + v_l).
__device__ __forceinline__ Split2 split2(const float *v, int e)
{
    f16x8 hp, lp;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float s = __builtin_amdgcn_ldexpf(v[t], e);
        const _Float16 h = static_cast<_Float16>(s);
        hp[t] = h;
        lp[t] = static_cast<_Float16>(s - static_cast<float>(h));
    }
    return {hp, lp};
}

// The exponent e that puts m (>= 0) in [2^14, 2^15) as 2^e m; 15 for m = 0
// or a non-finite m (whose values stay non-finite).
__device__ __forceinline__ int scale_exponent(float m) { return 15 - __builtin_amdgcn_frexp_expf(m); }

__device__ __forceinline__ float wave_max(float m)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    return m;
}
__device__ __forceinline__ int wave_min_int(int m)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = min(m, __shfl_xor(m, off));
    return m;
}
__device__ __forceinline__ int wave_max_int(int m)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = max(m, __shfl_xor(m, off));
    return m;
}

template <bool kBias>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kOutSplitWaves, 64 * kOutSplitWaves),
                          amdgpu_waves_per_eu(2)))   // at most 256 registers: no spills
void linear_out_split_kernel(const float *__restrict__ x, int64_t n_frames, int hidden,
                             const float *__restrict__ w, const float *__restrict__ bias,
                             float *__restrict__ out)
{
    __shared__ __align__(16) float s_tile[kOutSplitWaves][kOutWaveFrames * kTileRow];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t frame0 = static_cast<int64_t>(blockIdx.x) * kOutWaveFrames;   // shared by the workgroup
    float *tile = s_tile[wave];

    // B operand of group g: frame 32 g + col, dims 16 s + 8 half .. +7 of step s,
    // scaled by the frame's 2^ef[g] and split once
    Split2 xb[kOutGroups][4];
    int ef[kOutGroups];
#pragma unroll
    for (int g = 0; g < kOutGroups; ++g) {
        const int64_t frame = frame0 + 32 * g + col;
        const bool valid = frame < n_frames;
        const float *src = x + (valid ? frame : 0) * kDim + 8 * half;
        float v[4][8];
        float m = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(src + 16 * s);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(src + 16 * s + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[s][e] = valid ? a[e] : 0.0f;
                v[s][4 + e] = valid ? b[e] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[s][e]));
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        ef[g] = scale_exponent(m);
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[g][s] = split2(v[s], ef[g]);
    }
    // store j of a tile: frame 8 j + lane / 8 (group j / 4), outputs 4 (lane % 8) .. +3
    const int sf = lane >> 3, sseg = lane & 7;
    int efs[4 * kOutGroups];   // exponent of the frame of store j
#pragma unroll
    for (int j = 0; j < 4 * kOutGroups; ++j) efs[j] = __shfl(ef[j >> 2], 8 * (j & 3) + sf);
    // (read from the first lane: known to the compiler to be the same on every lane)
    const int ef_lo = __builtin_amdgcn_readfirstlane(wave_min_int(min(ef[0], ef[1])));
    const int ef_hi = __builtin_amdgcn_readfirstlane(wave_max_int(max(ef[0], ef[1])));

    // A operand of tile t: weight row 32 t + col, dims 16 s + 8 half .. +7
    auto load_tile = [&](int t, f32x4 (&wv)[8]) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(w + static_cast<int64_t>(32 * t + col) * kDim + 8 * half);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            wv[2 * s] = p[4 * s];
            wv[2 * s + 1] = p[4 * s + 1];
        }
    };
    const int n_tiles = hidden / 32;
    // products and stores of tile t from its weights wv and bias bv; kAll: all
    // 64 frames exist, so that every path stores the same number of times
    auto tile_out = [&](auto all_tag, int t, const f32x4 (&wv)[8], const f32x4 &bv) {
        constexpr bool kAll = decltype(all_tag)::value;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(wv[i][e]));
        const int et = __builtin_amdgcn_readfirstlane(scale_exponent(wave_max(m)));
        f32x16 acc[kOutGroups] = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float v[8] = {wv[2 * s][0], wv[2 * s][1], wv[2 * s][2], wv[2 * s][3],
                                wv[2 * s + 1][0], wv[2 * s + 1][1], wv[2 * s + 1][2], wv[2 * s + 1][3]};
            const Split2 a = split2(v, et);
            // small products first, the two groups' chains interleaved
#pragma unroll
            for (int g = 0; g < kOutGroups; ++g) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.l, xb[g][s].h, acc[g], 0, 0, 0);
#pragma unroll
            for (int g = 0; g < kOutGroups; ++g) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, xb[g][s].l, acc[g], 0, 0, 0);
#pragma unroll
            for (int g = 0; g < kOutGroups; ++g) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, xb[g][s].h, acc[g], 0, 0, 0);
        }
        // lane (col, half) holds outputs 8 m + 4 half .. +3 (m < 4) of frame 32 g + col
#pragma unroll
        for (int g = 0; g < kOutGroups; ++g)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<f32x4 *>(&tile[(32 * g + col) * kTileRow + 8 * m + 4 * half]) =
                    f32x4{acc[g][4 * m], acc[g][4 * m + 1], acc[g][4 * m + 2], acc[g][4 * m + 3]};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // every row of the tile is read (into its own registers) before any is
        // stored; scaled back by 2^-(ef + et) with the bias added: one fused
        // multiply-add by an exact power of two while every such factor is a
        // float (2^-149 .. 2^127), else the scaling and the bias apart
        f32x4 o[4 * kOutGroups];
#pragma unroll
        for (int j = 0; j < 4 * kOutGroups; ++j)
            o[j] = *reinterpret_cast<const f32x4 *>(&tile[(8 * j + sf) * kTileRow + 4 * sseg]);
        if (et + ef_hi <= 149 && et + ef_lo >= -127) {   // scalar: the same on every lane
#pragma unroll
            for (int j = 0; j < 4 * kOutGroups; ++j) {
                const float f = __builtin_amdgcn_ldexpf(1.0f, -(efs[j] + et));
#pragma unroll
                for (int e = 0; e < 4; ++e) o[j][e] = kBias ? __builtin_fmaf(o[j][e], f, bv[e]) : o[j][e] * f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4 * kOutGroups; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[j][e] = __builtin_amdgcn_ldexpf(o[j][e], -(efs[j] + et));
                    if (kBias) o[j][e] += bv[e];
                }
        }
        float *dst = out + (frame0 + sf) * static_cast<int64_t>(hidden) + 32 * t + 4 * sseg;
        const int64_t jstride = 8 * static_cast<int64_t>(hidden);
        if constexpr (kAll) {
#pragma unroll
            for (int j = 0; j < 4 * kOutGroups; ++j) *reinterpret_cast<f32x4 *>(dst + j * jstride) = o[j];
        } else {
#pragma unroll
            for (int j = 0; j < 4 * kOutGroups; ++j)
                if (frame0 + 8 * j + sf < n_frames) *reinterpret_cast<f32x4 *>(dst + j * jstride) = o[j];
        }
        // every lane has read the tile before the next tile overwrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
    };
    auto load_bias = [&](int t, f32x4 &bv) {
        if (kBias) bv = *reinterpret_cast<const f32x4 *>(bias + 32 * t + 4 * sseg);
    };
    // Wavefront w takes tiles w, w + 4, ... (the four write neighbouring 128 B
    // of the same rows), in pairs, the weight and bias registers alternating
    // (no copies). The loop has no path around either tile of a pair (an odd
    // last tile follows it), and the workgroup with frames past n_frames runs
    // its own copy of the loop, so that the compiler's count of the memory
    // operations issued after a tile's loads is exact.
    if (wave >= n_tiles) return;   // no tile for this wavefront (no barrier follows)
    const int n_w = (n_tiles - 1 - wave) / kOutSplitWaves + 1;   // tiles of this wavefront
    auto tile_of = [&](int i) { return wave + kOutSplitWaves * min(i, n_w - 1); };
    auto run = [&](auto all_tag) {
        f32x4 wa[8], wb[8];
        f32x4 ba = {0.0f, 0.0f, 0.0f, 0.0f}, bb = {0.0f, 0.0f, 0.0f, 0.0f};
        load_bias(tile_of(0), ba);
        load_tile(tile_of(0), wa);
        int i = 0;
        // (scheduling barriers keep each request where it is written: ahead of
        // the stores that precede its tile)
        for (; i + 1 < n_w; i += 2) {
            load_bias(tile_of(i + 1), bb);
            load_tile(tile_of(i + 1), wb);
            __builtin_amdgcn_sched_barrier(0);
            tile_out(all_tag, tile_of(i), wa, ba);
            __builtin_amdgcn_sched_barrier(0);
            load_bias(tile_of(i + 2), ba);
            load_tile(tile_of(i + 2), wa);
            __builtin_amdgcn_sched_barrier(0);
            tile_out(all_tag, tile_of(i + 1), wb, bb);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (i < n_w) tile_out(all_tag, tile_of(i), wa, ba);
    };
    if (frame0 + kOutWaveFrames <= n_frames)
        run(Flag<true>{});
    else
        run(Flag<false>{});
}

// ---- fc2 with the weight split resident in registers ------------------------
//
// For hidden a multiple of 512: a workgroup of 16 wavefronts owns 512
// outputs (wavefront w: tile 16 blockIdx.y + w of 32 outputs), scales and
// splits its weights once into registers, and then runs through groups of
// 32 frames (blockIdx.x, + gridDim.x, ...). The whole workgroup stages each
// group's frame operand: thread i loads two values of frame i / 32, the
// frame's 32 threads agree on its exponent, and the scaled fp16 parts go
// to LDS in the matrix-core operand layout (double buffered, one barrier
// per group). Each wavefront then runs its tile's twelve products, passes
// the result through its LDS tile and stores 8 frames x 128 B per store
// instruction; together the 16 write 2 KB of each frame's row. Same
// arithmetic, bound and rounding as linear_out_split_kernel.
//
// The outputs (4 KiB per frame at hidden 1024) are written with
// non-temporal stores, and the inputs (256 B per frame) are read once by
// touch_kernel just before, in chunks of at most 2^20 frames (256 MiB, the
// size of the memory-side cache): the
// kernel's input reads then come from the memory-side cache instead of
// reaching DRAM between the output writes, where they cost about a quarter
// of the kernel's time.
__global__ __launch_bounds__(256) void touch_kernel(const f32x4 *p, int64_t n4)
{
    f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<int64_t>(gridDim.x) * 256)
        a += p[i];
    asm volatile("" ::"v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));   // the loads stay
}

constexpr int kResWaves = 16;
constexpr int kResFrames = 32;

template <bool kBias>
__global__ __launch_bounds__(64 * kResWaves)
void linear_out_res_kernel(const float *__restrict__ x, int64_t n_frames, int hidden,
                           const float *__restrict__ w, const float *__restrict__ bias,
                           float *__restrict__ out)
{
    // frame operand of a group: [step][part][lane], part 0 = v_h, 1 = v_l
    __shared__ __align__(16) f16x8 s_b[2][4 * 2 * 64];
    __shared__ int s_ef[2][kResFrames];   // the frames' exponents
    __shared__ __align__(16) float s_tile[kResWaves][kResFrames * kTileRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int t = blockIdx.y * kResWaves + wave;   // this wavefront's tile (hidden % 512 == 0: all exist)
    const int64_t n_groups = (n_frames + kResFrames - 1) / kResFrames;
    const int64_t n_full = n_frames / kResFrames;
    const int64_t g0 = blockIdx.x, gs = gridDim.x;
    if (g0 >= n_groups) return;   // whole workgroup, before any barrier

    // A operand: weight row 32 t + col, dims 16 s + 8 half .. +7, scaled by 2^et and split
    Split2 wa[4];
    int et;
    {
        float v[4][8];
        float m = 0.0f;
        const float *src = w + static_cast<int64_t>(32 * t + col) * kDim + 8 * half;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(src + 16 * s);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(src + 16 * s + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[s][e] = a[e];
                v[s][4 + e] = b[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[s][e]));
        }
        et = __builtin_amdgcn_readfirstlane(scale_exponent(wave_max(m)));
#pragma unroll
        for (int s = 0; s < 4; ++s) wa[s] = split2(v[s], et);
    }
    // store j of a group: frame 8 j + lane / 8, outputs 32 t + 4 (lane % 8) .. +3
    const int sf = lane >> 3, sseg = lane & 7;
    f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
    if (kBias) bv = *reinterpret_cast<const f32x4 *>(bias + 32 * t + 4 * sseg);

    // staging: thread tid takes dims pd, pd + 1 of frame pf (step ps, half ph, entry pe)
    const int pf = tid >> 5, pd = 2 * (tid & 31);
    const int pidx = ((pd >> 4) * 2) * 64 + ((pd >> 3) & 1) * 32 + pf, pe = pd & 7;
    // (a frame past n_frames loads the last frame's values, and stages zeros)
    auto load_x = [&](int64_t g) {
        const int64_t fr = g * kResFrames + pf;
        return *reinterpret_cast<const f32x2 *>(x + (fr < n_frames ? fr : n_frames - 1) * kDim + pd);
    };
    auto stage = [&](f32x2 v, int64_t g, int buf) {
        if (g * kResFrames + pf >= n_frames) v = f32x2{0.0f, 0.0f};
        float m = fmaxf(fabsf(v[0]), fabsf(v[1]));
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));   // the frame's 32 threads
        const int e = scale_exponent(m);
        const float s0 = __builtin_amdgcn_ldexpf(v[0], e), s1 = __builtin_amdgcn_ldexpf(v[1], e);
        const _Float16 h0 = static_cast<_Float16>(s0), h1 = static_cast<_Float16>(s1);
        const _Float16 l0 = static_cast<_Float16>(s0 - static_cast<float>(h0));
        const _Float16 l1 = static_cast<_Float16>(s1 - static_cast<float>(h1));
        _Float16 *ph = reinterpret_cast<_Float16 *>(&s_b[buf][pidx]) + pe;
        _Float16 *pl = reinterpret_cast<_Float16 *>(&s_b[buf][pidx + 64]) + pe;
        *reinterpret_cast<f16x2 *>(ph) = f16x2{h0, h1};
        *reinterpret_cast<f16x2 *>(pl) = f16x2{l0, l1};
        if ((tid & 31) == 0) s_ef[buf][pf] = e;
    };

    float *tile = s_tile[wave];
    // products, transpose and stores of group g (operands in buffer buf)
    auto group_out = [&](auto all_tag, int64_t g, int buf) {
        constexpr bool kAll = decltype(all_tag)::value;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f16x8 bh = s_b[buf][(2 * s) * 64 + lane];
            const f16x8 bl = s_b[buf][(2 * s + 1) * 64 + lane];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa[s].l, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa[s].h, bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa[s].h, bh, acc, 0, 0, 0);
        }
        // lane (col, half) holds outputs 8 m + 4 half .. +3 (m < 4) of frame col
#pragma unroll
        for (int m = 0; m < 4; ++m)
            *reinterpret_cast<f32x4 *>(&tile[col * kTileRow + 8 * m + 4 * half]) =
                f32x4{acc[4 * m], acc[4 * m + 1], acc[4 * m + 2], acc[4 * m + 3]};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        f32x4 o[4];
        int k[4];
        bool inside = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[j] = *reinterpret_cast<const f32x4 *>(&tile[(8 * j + sf) * kTileRow + 4 * sseg]);
            k[j] = -(s_ef[buf][8 * j + sf] + et);
            inside = inside && k[j] >= -149 && k[j] <= 127;
        }
        // scaled back by 2^k with the bias added: one fused multiply-add by an
        // exact power of two when every factor of the wavefront is a float
        if (__builtin_amdgcn_ballot_w64(!inside) == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = __builtin_amdgcn_ldexpf(1.0f, k[j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[j][e] = kBias ? __builtin_fmaf(o[j][e], f, bv[e]) : o[j][e] * f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[j][e] = __builtin_amdgcn_ldexpf(o[j][e], k[j]);
                    if (kBias) o[j][e] += bv[e];
                }
        }
        const int64_t f0 = g * kResFrames;
        float *dst = out + (f0 + sf) * static_cast<int64_t>(hidden) + 32 * t + 4 * sseg;
        const int64_t jstride = 8 * static_cast<int64_t>(hidden);
        if constexpr (kAll) {
#pragma unroll
            for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(o[j], reinterpret_cast<f32x4 *>(dst + j * jstride));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (f0 + 8 * j + sf < n_frames) *reinterpret_cast<f32x4 *>(dst + j * jstride) = o[j];
        }
        // every lane has read the tile before the next group overwrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
    };

    // The loop holds no conditional memory operation (requests are clamped to
    // the last group), so that the compiler's count of what was issued after
    // a request is exact; the partial last group follows it. The values of
    // the next kAhead groups are requested ahead, each after the stores of
    // its iteration, so that the wait for a group's values covers only
    // stores issued kAhead iterations earlier; slot j of xs is loaded and
    // consumed in the j-th iteration of each unrolled block, so no register
    // copy waits for a load early.
    constexpr int kAhead = 4;
    const int64_t last = n_groups - 1;
    const f32x2 x0 = load_x(g0);
    __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0): weights, bias and the first values
    stage(x0, g0, 0);
    f32x2 xs[kAhead];   // xs[j]: the group of the iteration's successor, j iterations on
#pragma unroll
    for (int j = 0; j < kAhead; ++j) xs[j] = load_x(min(g0 + (j + 1) * gs, last));
    __syncthreads();
    int buf = 0;
    int64_t g = g0;
    auto full_group = [&](int j) {
        group_out(Flag<true>{}, g, buf);
        __builtin_amdgcn_sched_barrier(0);
        stage(xs[j], min(g + gs, last), buf ^ 1);
        xs[j] = load_x(min(g + (kAhead + 1) * gs, last));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        buf ^= 1;
        g += gs;
    };
    // whole blocks of kAhead full groups (no path leaves a block early), then the rest
    const int64_t n_it = n_full > g0 ? (n_full - g0 + gs - 1) / gs : 0;
    for (int64_t b = 0; b < n_it / kAhead; ++b) {
#pragma unroll
        for (int j = 0; j < kAhead; ++j) full_group(j);
    }
    const int rest = static_cast<int>(n_it % kAhead);
#pragma unroll
    for (int j = 0; j < kAhead - 1; ++j)
        if (j < rest) full_group(j);
    if (g < n_groups) group_out(Flag<false>{}, g, buf);
}

}  // namespace

hipError_t launch_linear_in(const float *h, int64_t n_frames, int hidden, const float *w,
                            const float *bias, float *y, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kInFrames - 1) / kInFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kInWaves);
    const Update none = {nullptr, 0, nullptr, 0, nullptr};
    if (bias)
        hipLaunchKernelGGL((linear_in_kernel<true, false>), grid, block, 0, stream, h, n_frames, hidden, w, bias,
                           y, none);
    else
        hipLaunchKernelGGL((linear_in_kernel<false, false>), grid, block, 0, stream, h, n_frames, hidden, w, bias,
                           y, none);
    return hipGetLastError();
}

hipError_t launch_linear_in_update(const float *src, const int32_t *codes, int codes_ld, const float *table,
                                   int n_codes, float *dst, int64_t n_frames, int hidden, const float *w,
                                   const float *bias, float *y, hipStream_t stream)
{
    const int64_t blocks = (n_frames + kInFrames - 1) / kInFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kInWaves);
    const Update up = {codes, codes_ld, table, n_codes, dst};
    if (bias)
        hipLaunchKernelGGL((linear_in_kernel<true, true>), grid, block, 0, stream, src, n_frames, hidden, w, bias,
                           y, up);
    else
        hipLaunchKernelGGL((linear_in_kernel<false, true>), grid, block, 0, stream, src, n_frames, hidden, w, bias,
                           y, up);
    return hipGetLastError();
}

hipError_t launch_linear_out(const float *x, int64_t n_frames, int hidden, const float *w,
                             const float *bias, float *out, hipStream_t stream)
{
    if (hidden % (32 * kResWaves) == 0) {
        const int halves = hidden / (32 * kResWaves);
        constexpr int64_t kChunk = int64_t(1) << 20;   // frames per touch + product pair
        for (int64_t f = 0; f < n_frames; f += kChunk) {
            const int64_t n = std::min(kChunk, n_frames - f);
            hipLaunchKernelGGL(touch_kernel, dim3(1024), dim3(256), 0, stream,
                               reinterpret_cast<const f32x4 *>(x + f * kDim), n * kDim / 4);
            // one workgroup of 16 wavefronts per CU, 256 CUs
            const int64_t n_groups = (n + kResFrames - 1) / kResFrames;
            const int64_t slices = std::max<int64_t>(1, std::min<int64_t>(n_groups, 256 / std::min(halves, 256)));
            const dim3 grid(static_cast<unsigned>(slices), static_cast<unsigned>(halves)), block(64 * kResWaves);
            if (bias)
                hipLaunchKernelGGL((linear_out_res_kernel<true>), grid, block, 0, stream, x + f * kDim, n, hidden, w,
                                   bias, out + f * hidden);
            else
                hipLaunchKernelGGL((linear_out_res_kernel<false>), grid, block, 0, stream, x + f * kDim, n, hidden, w,
                                   bias, out + f * hidden);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (hidden % 32 == 0) {
        const int64_t per_block = kOutWaveFrames;
        const int64_t blocks = (n_frames + per_block - 1) / per_block;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kOutSplitWaves);
        if (bias)
            hipLaunchKernelGGL((linear_out_split_kernel<true>), grid, block, 0, stream, x, n_frames, hidden, w, bias,
                               out);
        else
            hipLaunchKernelGGL((linear_out_split_kernel<false>), grid, block, 0, stream, x, n_frames, hidden, w, bias,
                               out);
        return hipGetLastError();
    }
    const int64_t blocks = (n_frames + kOutFrames - 1) / kOutFrames;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kOutWaves);
    if (bias)
        hipLaunchKernelGGL((linear_out_kernel<true>), grid, block, 0, stream, x, n_frames, hidden, w, bias, out);
    else
        hipLaunchKernelGGL((linear_out_kernel<false>), grid, block, 0, stream, x, n_frames, hidden, w, bias, out);
    return hipGetLastError();
}

}  // namespace rvq
