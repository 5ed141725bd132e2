// Ceiling probes for gfx950, measurement tooling beside the library (built
// into its own librvq_probe.so, not part of the quantizer):
//   - row gathers: the rate at which the CU array gathers random 256-byte
//     rows (16 lanes x 16 bytes, the access pattern of the decode) out of a
//     table that lives in L2 / MALL, with no load that the row address
//     depends on and no store per row. The decode's row gathers are bound by
//     this rate rather than by HBM, so it is the ceiling the decode is
//     compared with;
//   - matrix cores: back-to-back independent v_mfma_f32_32x32x16_f16 or
//     v_mfma_f32_32x32x2_f32 chains on register operands with full-mantissa
//     values, the measured peaks beside the published ones;
//   - HBM reads: a grid-stride sum of 16-byte loads over a buffer much larger
//     than the caches, one store per thread, the read-only rate the
//     in-projection (which reads 4 KiB and writes 256 B per frame) is
//     compared with.
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kRowFloats = 64;

// A row index from a counter: two rounds of multiply / xor-shift, uniform
// enough over power-of-two tables for a cache-rate probe.
__device__ __forceinline__ uint32_t row_of(uint32_t i, uint32_t mask)
{
    i ^= i >> 16;
    i *= 0x7feb352du;
    i ^= i >> 15;
    i *= 0x846ca68bu;
    i ^= i >> 16;
    return i & mask;
}

// Each group of 16 lanes gathers `per_group` rows (row r of the group's
// sequence: row_of(group * per_group + r), or with `permute` the odd
// multiple (group * per_group + r) * 0x9E3779B1 mod the table size, which
// visits every row once when the groups gather table-size rows in all),
// 8 at a time so that 8 row loads are in flight per lane, and sums them;
// one float4 per lane is stored at the end so that the loads are not
// removed.
__global__ __launch_bounds__(kThreads)
void gather_probe_kernel(const float *__restrict__ table, uint32_t row_mask, int per_group, int permute,
                         float *__restrict__ sink)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const uint32_t group = static_cast<uint32_t>(gid / kLanesPerRow);
    const int part = static_cast<int>(gid % kLanesPerRow);
    const float *base = table + 4 * part;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t first = group * static_cast<uint32_t>(per_group);
    for (int r = 0; r < per_group; r += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = first + r + j;
            const uint32_t row = permute ? (i * 0x9E3779B1u) & row_mask : row_of(i, row_mask);
            v[j] = *reinterpret_cast<const f32x4 *>(base + static_cast<int64_t>(row) * kRowFloats);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j];
    }
    reinterpret_cast<f32x4 *>(sink)[gid] = acc;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Operand values with full mantissas, different per lane and element.
__device__ __forceinline__ float operand(uint32_t lane, uint32_t j)
{
    return 0.5f + static_cast<float>(row_of(lane * 64u + j, 0xFFFFFFu)) * 5.9604645e-08f;
}

// Four independent chains of `iters` fp16 32x32x16 products per wavefront.
__global__ __launch_bounds__(kThreads)
void mfma_f16_probe_kernel(int iters, float *__restrict__ sink)
{
    const uint32_t lane = threadIdx.x + blockIdx.x * kThreads;
    f16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = static_cast<_Float16>(operand(lane, j));
        b[j] = static_cast<_Float16>(operand(lane, j + 8));
    }
    f32x16 c[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += c[k][j];
    sink[lane] = s;
}

// Four independent chains of `iters` fp32 32x32x2 products per wavefront.
__global__ __launch_bounds__(kThreads)
void mfma_f32_probe_kernel(int iters, float *__restrict__ sink)
{
    const uint32_t lane = threadIdx.x + blockIdx.x * kThreads;
    const float a = operand(lane, 0), b = operand(lane, 1);
    f32x16 c[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c[k], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += c[k][j];
    sink[lane] = s;
}

// Grid-stride sum of n4 float4 (one 16-byte load per lane per step), one
// float per thread to sink.
__global__ __launch_bounds__(kThreads)
void read_probe_kernel(const f32x4 *__restrict__ src, int64_t n4, float *__restrict__ sink)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += stride) acc += src[i];
    sink[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

}  // namespace

extern "C" {

// Reads n_floats floats of `src` (device memory, 16-byte aligned, n_floats a
// multiple of 4) with `blocks` workgroups of 256 threads; `sink` receives
// blocks * 256 floats (device memory). Returns 0, -1 for invalid arguments,
// -3 if the launch failed.
__attribute__((visibility("default"))) int rvqprobe_read(const float *src, int64_t n_floats, int32_t blocks,
                                                          float *sink, void *stream)
{
    if (!src || !sink || n_floats <= 0 || n_floats % 4 != 0 || blocks <= 0) return -1;
    hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const f32x4 *>(src), n_floats / 4, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Runs `blocks` workgroups of 256 threads, each wavefront 4 chains of
// `iters` matrix-core products: fp16 32x32x16 (32768 flop each) when
// `fp16` is nonzero, else fp32 32x32x2 (4096 flop each). `sink` receives
// blocks * 256 floats (device memory). Returns 0, -1 for invalid
// arguments, -3 if the launch failed.
__attribute__((visibility("default"))) int rvqprobe_mfma(int32_t fp16, int32_t blocks, int32_t iters, float *sink,
                                                          void *stream)
{
    if (!sink || blocks <= 0 || iters <= 0) return -1;
    if (fp16)
        hipLaunchKernelGGL(mfma_f16_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), iters, sink);
    else
        hipLaunchKernelGGL(mfma_f32_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Gathers n_groups * per_group rows of 64 floats from `table` (table_rows
// rows, a power of two; device memory, 16-byte aligned) on `stream`, at
// random (permute 0) or as a permutation of the rows (permute 1: each row
// once when n_groups * per_group == table_rows); `sink` receives
// n_groups * 16 float4 (device memory). per_group must be a positive
// multiple of 8 and n_groups * 16 a multiple of 256. Returns 0, or -1 for
// invalid arguments, -3 if the launch failed.
__attribute__((visibility("default"))) int rvqprobe_gather_rows(const float *table, int64_t table_rows,
                                                                 int64_t n_groups, int32_t per_group,
                                                                 int32_t permute, float *sink, void *stream)
{
    if (!table || !sink || table_rows <= 0 || (table_rows & (table_rows - 1)) != 0 || table_rows > (int64_t(1) << 31))
        return -1;
    if (per_group <= 0 || per_group % 8 != 0 || n_groups <= 0 || (n_groups * kLanesPerRow) % kThreads != 0)
        return -1;
    if (n_groups * per_group > (int64_t(1) << 32)) return -1;
    const int64_t blocks = n_groups * kLanesPerRow / kThreads;
    if (blocks > 0x7fffffff) return -1;
    hipLaunchKernelGGL(gather_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), table, static_cast<uint32_t>(table_rows - 1), per_group,
                       permute ? 1 : 0, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
