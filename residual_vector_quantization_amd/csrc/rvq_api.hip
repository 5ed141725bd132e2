// C ABI of librvq: argument validation, then one kernel launch on the
// caller's stream. Declarations, layouts and the numerical contract are in
// include/rvq.h. No allocation, no global state.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rvq.h"
#include "rvq_internal.h"

namespace {

constexpr int32_t kMaxStages = 65536;
constexpr int32_t kCosineDim = 8;          // codebook dim of the normalized quantizer
constexpr int32_t kCosineMaxHidden = 1024;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by every entry point; pointers are checked by callers.
rvq_status check_shape(int64_t n_frames, int32_t dim, int32_t n_stages, int32_t n_codes)
{
    if (n_frames < 0 || dim <= 0 || n_stages <= 0 || n_codes <= 0) return RVQ_ERR_INVALID_ARG;
    if (dim != rvq::kDim || n_stages > kMaxStages) return RVQ_ERR_UNSUPPORTED;
    return RVQ_OK;
}

rvq_status from_hip(hipError_t e) { return e == hipSuccess ? RVQ_OK : RVQ_ERR_DEVICE; }

hipError_t launch_scored(rvq_scoring scoring, const float *x, int64_t n_frames, const float *books,
                         int n_stages, int n_codes, int32_t *codes, int codes_ld, float *residual,
                         float *recon, hipStream_t stream)
{
    if (scoring == RVQ_SCORING_FP32)
        return rvq::launch_encode(x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon, stream);
    return rvq::launch_encode_bf16(x, n_frames, books, n_stages, n_codes, codes, codes_ld, residual, recon,
                                   stream);
}

rvq_status encode_common(const float *x, int64_t n_frames, int32_t dim, const float *books,
                         int32_t n_stages, int32_t n_codes, int32_t *codes, int32_t codes_ld,
                         float *recon, bool want_recon, float *residual, rvq_scoring scoring, void *stream)
{
    if (scoring != RVQ_SCORING_DEFAULT && scoring != RVQ_SCORING_BF16X3 && scoring != RVQ_SCORING_FP32)
        return RVQ_ERR_INVALID_ARG;
    rvq_status st = check_shape(n_frames, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (n_frames == 0) return RVQ_OK;
    if (!x || !books || !codes || (want_recon && !recon)) return RVQ_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(books, 16) || !aligned(codes, 4) ||
        (recon && !aligned(recon, 16)) || (residual && !aligned(residual, 16)))
        return RVQ_ERR_INVALID_ARG;
    return from_hip(launch_scored(scoring, x, n_frames, books, n_stages, n_codes, codes, codes_ld,
                                  residual, recon, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

RVQ_API const char *rvq_version(void)
{
    return "0.1.0 (gfx950)";
}

RVQ_API const char *rvq_status_string(rvq_status status)
{
    switch (status) {
    case RVQ_OK: return "ok";
    case RVQ_ERR_INVALID_ARG: return "invalid argument";
    case RVQ_ERR_UNSUPPORTED: return "unsupported shape";
    case RVQ_ERR_DEVICE: return "device error";
    case RVQ_ERR_OOM: return "out of memory";
    }
    return "unknown status";
}

RVQ_API rvq_status rvq_encode(const float *x, int64_t n_frames, int32_t dim,
                              const float *codebooks, int32_t n_stages, int32_t n_codes,
                              int32_t *codes, int32_t codes_ld, float *residual, void *stream)
{
    return encode_common(x, n_frames, dim, codebooks, n_stages, n_codes, codes, codes_ld,
                         nullptr, false, residual, RVQ_SCORING_DEFAULT, stream);
}

RVQ_API rvq_status rvq_roundtrip(const float *x, int64_t n_frames, int32_t dim,
                                 const float *codebooks, int32_t n_stages, int32_t n_codes,
                                 int32_t *codes, int32_t codes_ld, float *recon,
                                 float *residual, void *stream)
{
    return encode_common(x, n_frames, dim, codebooks, n_stages, n_codes, codes, codes_ld,
                         recon, true, residual, RVQ_SCORING_DEFAULT, stream);
}

RVQ_API rvq_status rvq_encode_scored(const float *x, int64_t n_frames, int32_t dim,
                                     const float *codebooks, int32_t n_stages, int32_t n_codes,
                                     int32_t *codes, int32_t codes_ld, float *recon, float *residual,
                                     rvq_scoring scoring, void *stream)
{
    return encode_common(x, n_frames, dim, codebooks, n_stages, n_codes, codes, codes_ld,
                         recon, false, residual, scoring, stream);
}

RVQ_API rvq_status rvq_decode(const int32_t *codes, int32_t codes_ld, int64_t n_frames,
                              const float *codebooks, int32_t n_stages, int32_t n_codes,
                              int32_t dim, float *out, void *stream)
{
    rvq_status st = check_shape(n_frames, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (n_frames == 0) return RVQ_OK;
    if (!codes || !codebooks || !out) return RVQ_ERR_INVALID_ARG;
    if (!aligned(codes, 4) || !aligned(codebooks, 16) || !aligned(out, 16)) return RVQ_ERR_INVALID_ARG;
    return from_hip(rvq::launch_decode(codes, codes_ld, n_frames, codebooks, n_stages, n_codes, out,
                                       static_cast<hipStream_t>(stream)));
}

RVQ_API int64_t rvq_prepared_bytes(int32_t n_stages, int32_t n_codes, int32_t dim)
{
    const rvq_status st = check_shape(0, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    return rvq::prepared_bytes(n_stages, n_codes);
}

RVQ_API rvq_status rvq_prepare_codebooks(const float *codebooks, int32_t n_stages, int32_t n_codes,
                                         int32_t dim, void *prepared, int64_t prepared_bytes, void *stream)
{
    const rvq_status st = check_shape(0, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (!codebooks || !prepared || !aligned(codebooks, 16) || !aligned(prepared, 16)) return RVQ_ERR_INVALID_ARG;
    if (prepared_bytes < rvq::prepared_bytes(n_stages, n_codes)) return RVQ_ERR_INVALID_ARG;
    return from_hip(rvq::launch_prepare(codebooks, n_stages, n_codes, prepared, static_cast<hipStream_t>(stream)));
}

RVQ_API rvq_status rvq_encode_prepared(const float *x, int64_t n_frames, int32_t dim, const float *codebooks,
                                       const void *prepared, int32_t n_stages, int32_t n_codes,
                                       int32_t *codes, int32_t codes_ld, float *recon, float *residual,
                                       void *stream)
{
    rvq_status st = check_shape(n_frames, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (n_frames == 0) return RVQ_OK;
    if (!x || !codebooks || !prepared || !codes) return RVQ_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(codebooks, 16) || !aligned(prepared, 16) || !aligned(codes, 4) ||
        (recon && !aligned(recon, 16)) || (residual && !aligned(residual, 16)))
        return RVQ_ERR_INVALID_ARG;
    return from_hip(rvq::launch_encode_prepared(x, n_frames, codebooks, prepared, n_stages, n_codes, codes,
                                                codes_ld, residual, recon, static_cast<hipStream_t>(stream)));
}

RVQ_API rvq_status rvq_project_roundtrip(const float *h, int64_t n_frames, int32_t hidden,
                                         const float *w_in, const float *b_in,
                                         const float *codebooks, const void *prepared,
                                         int32_t n_stages, int32_t n_codes,
                                         int32_t dim, const float *w_out, const float *b_out,
                                         int32_t *codes, int32_t codes_ld, float *latent,
                                         float *latent_recon, float *h_recon, void *stream)
{
    rvq_status st = check_shape(n_frames, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (hidden <= 0 || codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (hidden % 64 != 0) return RVQ_ERR_UNSUPPORTED;
    if (n_frames == 0) return RVQ_OK;
    if (!h || !w_in || !codebooks || !w_out || !codes || !latent || !latent_recon || !h_recon)
        return RVQ_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(w_in, 16) || !aligned(codebooks, 16) || !aligned(w_out, 16) ||
        !aligned(codes, 4) || !aligned(latent, 16) || !aligned(latent_recon, 16) || !aligned(h_recon, 16) ||
        (b_in && !aligned(b_in, 16)) || (b_out && !aligned(b_out, 16)) || (prepared && !aligned(prepared, 16)))
        return RVQ_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = rvq::launch_linear_in(h, n_frames, hidden, w_in, b_in, latent, s);
    if (e == hipSuccess)
        e = prepared ? rvq::launch_encode_prepared(latent, n_frames, codebooks, prepared, n_stages, n_codes, codes,
                                                   codes_ld, nullptr, latent_recon, s)
                     : launch_scored(RVQ_SCORING_DEFAULT, latent, n_frames, codebooks, n_stages, n_codes, codes,
                                     codes_ld, nullptr, latent_recon, s);
    if (e == hipSuccess)
        e = rvq::launch_linear_out(latent_recon, n_frames, hidden, w_out, b_out, h_recon, s);
    return from_hip(e);
}

RVQ_API rvq_status rvq_projected_prepare(const float *codebooks, int32_t n_stages, int32_t n_codes,
                                         int32_t dim, const float *w_out, const float *b_out,
                                         int32_t hidden, float *table, void *stream)
{
    // codeword dim 64 (per-stage projected RVQ) or 8 (normalized quantizer)
    const rvq_status st = check_shape(0, dim == kCosineDim ? rvq::kDim : dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (hidden <= 0) return RVQ_ERR_INVALID_ARG;
    if (hidden % 64 != 0) return RVQ_ERR_UNSUPPORTED;
    if (!codebooks || !w_out || !table) return RVQ_ERR_INVALID_ARG;
    if (!aligned(codebooks, 16) || !aligned(w_out, 16) || !aligned(table, 16) || (b_out && !aligned(b_out, 16)))
        return RVQ_ERR_INVALID_ARG;
    return from_hip(rvq::launch_projected_table(codebooks, n_stages, n_codes, dim, w_out, b_out, hidden, table,
                                                static_cast<hipStream_t>(stream)));
}

RVQ_API rvq_status rvq_projected_encode(const float *h, int64_t n_frames, int32_t hidden,
                                        const float *w_in, const float *b_in,
                                        const float *codebooks, const void *prepared, const float *table,
                                        int32_t n_stages, int32_t n_codes, int32_t dim,
                                        int32_t *codes, int32_t codes_ld,
                                        float *latent, float *residual, void *stream)
{
    const rvq_status st = check_shape(n_frames, dim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (hidden <= 0 || codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (hidden % 64 != 0) return RVQ_ERR_UNSUPPORTED;
    if (n_frames == 0) return RVQ_OK;
    if (!h || !w_in || !codebooks || !table || !codes || !latent || !residual) return RVQ_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(w_in, 16) || !aligned(codebooks, 16) || !aligned(table, 16) ||
        !aligned(codes, 4) || !aligned(latent, 16) || !aligned(residual, 16) || (b_in && !aligned(b_in, 16)) ||
        (prepared && !aligned(prepared, 16)))
        return RVQ_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const int64_t table_stage = static_cast<int64_t>(n_codes) * hidden;
    const int64_t prepared_stage = rvq::prepared_bytes(1, n_codes);   // stage blocks are consecutive
    for (int32_t q = 0; q < n_stages && e == hipSuccess; ++q) {
        float *lat = latent + static_cast<int64_t>(q) * n_frames * rvq::kDim;
        const float *book = codebooks + static_cast<int64_t>(q) * n_codes * rvq::kDim;
        const float *wq = w_in + static_cast<int64_t>(q) * rvq::kDim * hidden;
        const float *bq = b_in ? b_in + static_cast<int64_t>(q) * rvq::kDim : nullptr;
        if (q == 0) {
            e = rvq::launch_linear_in(h, n_frames, hidden, wq, bq, lat, s);
        } else {
            // stage q - 1's residual update rides along with stage q's in-projection:
            // it reads h at q = 1 and the residual buffer afterwards
            e = rvq::launch_linear_in_update(q == 1 ? h : residual, codes + (q - 1), codes_ld,
                                             table + (q - 1) * table_stage, n_codes, residual, n_frames,
                                             hidden, wq, bq, lat, s);
        }
        if (e == hipSuccess)
            e = prepared ? rvq::launch_encode_prepared(lat, n_frames, book,
                                                       static_cast<const uint8_t *>(prepared) + q * prepared_stage,
                                                       1, n_codes, codes + q, codes_ld, nullptr, nullptr, s)
                         : launch_scored(RVQ_SCORING_DEFAULT, lat, n_frames, book, 1, n_codes, codes + q, codes_ld,
                                         nullptr, nullptr, s);
    }
    if (e == hipSuccess)
        e = rvq::launch_projected_update(n_stages == 1 ? h : residual, codes + (n_stages - 1), codes_ld, n_frames,
                                         table + (n_stages - 1) * table_stage, n_codes, hidden, residual, s);
    return from_hip(e);
}

RVQ_API rvq_status rvq_projected_decode(const int32_t *codes, int32_t codes_ld, int64_t n_frames,
                                        const float *table, int32_t n_stages, int32_t n_codes,
                                        int32_t hidden, float *out, void *stream)
{
    const rvq_status st = check_shape(n_frames, rvq::kDim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (hidden <= 0 || codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (hidden % 64 != 0) return RVQ_ERR_UNSUPPORTED;
    if (n_frames == 0) return RVQ_OK;
    if (!codes || !table || !out) return RVQ_ERR_INVALID_ARG;
    if (!aligned(codes, 4) || !aligned(table, 16) || !aligned(out, 16)) return RVQ_ERR_INVALID_ARG;
    return from_hip(rvq::launch_projected_decode(codes, codes_ld, n_frames, table, n_stages, n_codes, hidden,
                                                 out, static_cast<hipStream_t>(stream)));
}

RVQ_API rvq_status rvq_cosine_prepare(const float *codebooks, int32_t n_stages, int32_t n_codes, int32_t dim,
                                      double *units, void *stream)
{
    const rvq_status st = check_shape(0, rvq::kDim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (dim <= 0) return RVQ_ERR_INVALID_ARG;
    if (dim != kCosineDim) return RVQ_ERR_UNSUPPORTED;
    if (!codebooks || !units || !aligned(codebooks, 16) || !aligned(units, 16)) return RVQ_ERR_INVALID_ARG;
    return from_hip(rvq::launch_cosine_units(codebooks, n_stages, n_codes, units, static_cast<hipStream_t>(stream)));
}

RVQ_API rvq_status rvq_cosine_encode(const float *h, int64_t n_frames, int32_t hidden,
                                     const float *w_in, const float *b_in,
                                     const double *units, const float *table,
                                     int32_t n_stages, int32_t n_codes, int32_t dim,
                                     int32_t *codes, int32_t codes_ld,
                                     float *latent, float *residual, void *stream)
{
    const rvq_status st = check_shape(n_frames, rvq::kDim, n_stages, n_codes);
    if (st != RVQ_OK) return st;
    if (dim <= 0 || hidden <= 0 || codes_ld < n_stages) return RVQ_ERR_INVALID_ARG;
    if (dim != kCosineDim || hidden % 64 != 0 || hidden > kCosineMaxHidden) return RVQ_ERR_UNSUPPORTED;
    if (n_frames == 0) return RVQ_OK;
    if (!h || !w_in || !units || !table || !codes || !latent || !residual) return RVQ_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(w_in, 16) || !aligned(units, 16) || !aligned(table, 16) ||
        !aligned(codes, 4) || !aligned(latent, 16) || !aligned(residual, 16) || (b_in && !aligned(b_in, 16)))
        return RVQ_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rvq::cosine_fused_supported(n_codes, hidden))
        return from_hip(rvq::launch_cosine_fused(h, n_frames, hidden, w_in, b_in, units, table, n_stages, n_codes,
                                                 codes, codes_ld, latent, residual, s));
    // larger codebooks: one projection and one argmin launch per stage
    hipError_t e = hipSuccess;
    const int64_t table_stage = static_cast<int64_t>(n_codes) * hidden;
    for (int32_t q = 0; q < n_stages && e == hipSuccess; ++q) {
        float *lat = latent + static_cast<int64_t>(q) * n_frames * kCosineDim;
        const float *wq = w_in + static_cast<int64_t>(q) * kCosineDim * hidden;
        const float *bq = b_in ? b_in + static_cast<int64_t>(q) * kCosineDim : nullptr;
        if (q == 0)
            e = rvq::launch_proj8(h, nullptr, codes_ld, nullptr, n_codes, nullptr, n_frames, hidden, wq, bq, lat, s);
        else
            e = rvq::launch_proj8(q == 1 ? h : residual, codes + (q - 1), codes_ld, table + (q - 1) * table_stage,
                                  n_codes, residual, n_frames, hidden, wq, bq, lat, s);
        if (e == hipSuccess)
            e = rvq::launch_cosine_argmin(lat, n_frames, units + static_cast<int64_t>(q) * n_codes * kCosineDim,
                                          n_codes, codes + q, codes_ld, s);
    }
    if (e == hipSuccess)
        e = rvq::launch_projected_update(n_stages == 1 ? h : residual, codes + (n_stages - 1), codes_ld, n_frames,
                                         table + (n_stages - 1) * table_stage, n_codes, hidden, residual, s);
    return from_hip(e);
}

}  // extern "C"
