/*
 * rvq.h -- C ABI of the MI355X (gfx950) residual vector quantization library.
 *
 * Plain C99, extern "C", no HIP or torch types in any signature. Only the
 * rvq_* symbols below are exported from librvq.so; everything else is built
 * with hidden visibility.
 *
 * What the operations compute follows the "RVQ codec" section of the
 * "Architecture" page (omnivoice.cpp port of OmniVoice / Higgs-Audio-v2):
 *   - encode is the residual loop: for stage q = 0..Q-1, pick the codeword
 *     of codebook q nearest (squared L2) to the current residual, emit its
 *     index, subtract the codeword from the residual;
 *   - decode is the per-codebook gather and accumulate: gather row
 *     codes[n, q] of codebook q and add it to an accumulator, q ascending.
 * The codebooks act directly on the D-dim latent (identity per-stage
 * projections). The code layout is frame-major [N, Q], as in gotcha 8 of
 * the "Maintainer's guide -- moss-tts.cpp" page ("ne0 = NQ, ne1 = T").
 *
 * Numerical contract:
 *   - ties in distance go to the lowest codeword index;
 *   - the pick of every stage equals the argmin of the float64 direct-form
 *     distance sum_j (r_j - c_j)^2 (j ascending, one rounding per
 *     operation) over all K codewords. Scores are computed on the matrix
 *     cores (split-bf16 by default, or fp32, see rvq_encode_scored; fp16
 *     for rvq_encode_prepared); every codeword whose score
 *     lies within a proven error bound of the best is re-ranked with that
 *     float64 sum, so score rounding never decides a pick and all scorings
 *     give identical results;
 *   - residuals are float32, r <- fl32(r - c) per element;
 *   - decode (and the reconstruction of rvq_roundtrip) is a float32 sum
 *     that starts at +0 and adds stage 0 first.
 *
 * Memory, ownership, streams:
 *   - every array argument is DEVICE memory owned by the caller (for
 *     example a torch tensor's data pointer). The library never allocates,
 *     frees or keeps a caller buffer, and keeps no state between calls;
 *   - float arrays must be 16-byte aligned, int32 arrays 4-byte aligned;
 *   - all arrays are dense row-major:
 *       x, residual, recon, out   [n_frames, dim]          float32
 *       codebooks                 [n_stages, n_codes, dim] float32
 *       codes                     [n_frames, codes_ld]     int32, columns 0..n_stages-1 used
 *     Passing n_stages smaller than the codebook tensor's stage count uses
 *     its first n_stages codebooks (bitrate control: first k of Q stages);
 *   - `stream` is a hipStream_t cast to void* (NULL = the default stream).
 *     Calls enqueue work and return; results are ready once the stream has
 *     been synchronised. Calls on different streams may overlap safely as
 *     long as their output buffers do not alias;
 *   - argument errors are reported synchronously, before anything is
 *     enqueued. A failed kernel launch returns RVQ_ERR_DEVICE; faults inside
 *     a kernel surface at the caller's next synchronisation.
 *
 * Supported shapes: dim == 64; n_codes >= 1; 1 <= n_stages <= 65536;
 * n_frames >= 0 (0 is a no-op that returns RVQ_OK and touches nothing).
 * Inputs must be finite; non-finite values give unspecified codes, but no
 * out-of-bounds access.
 */
#ifndef RVQ_H
#define RVQ_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define RVQ_API __attribute__((visibility("default")))
#else
#define RVQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define RVQ_VERSION_MAJOR 0
#define RVQ_VERSION_MINOR 1
#define RVQ_VERSION_PATCH 0

/*
 * Status codes: 0 on success, negative on failure (no output written). The
 * convention -- 0 for success, small negative integers for each kind of
 * failure, a static string per code -- is that of the ov_status enum in the
 * "Public API" section of the "Architecture" page.
 */
typedef enum rvq_status {
    RVQ_OK = 0,
    RVQ_ERR_INVALID_ARG = -1,  /* null pointer, negative size, codes_ld < n_stages, misalignment */
    RVQ_ERR_UNSUPPORTED = -2,  /* valid but unsupported shape (dim != 64, n_stages > 65536) */
    RVQ_ERR_DEVICE = -3,       /* the HIP runtime refused the launch or has no device */
    RVQ_ERR_OOM = -4           /* out of memory; reserved: no call allocates device memory today */
} rvq_status;

/* How encode scores codewords before the exact float64 decision. */
typedef enum rvq_scoring {
    RVQ_SCORING_DEFAULT = 0,  /* the fastest available: RVQ_SCORING_BF16X3 */
    RVQ_SCORING_BF16X3 = 1,   /* split-bf16 (hi*hi + hi*lo + lo*hi) on bf16 matrix cores */
    RVQ_SCORING_FP32 = 2      /* fp32 matrix cores */
} rvq_scoring;

/*
 * Static string "MAJOR.MINOR.PATCH (gfx950)". Never NULL. The counterpart
 * of ov_version in the "Public API" section of the "Architecture" page.
 */
RVQ_API const char *rvq_version(void);

/*
 * Static, human-readable name of a status code ("unknown status" for any
 * other value). Never NULL. Like the status strings of the "Public API"
 * section of the "Architecture" page.
 */
RVQ_API const char *rvq_status_string(rvq_status status);

/*
 * rvq_encode -- greedy residual encode of n_frames latents.
 *
 *   x          [n_frames, dim] input latents (read only)
 *   codebooks  [n_stages, n_codes, dim] (read only)
 *   codes      [n_frames, codes_ld] output; column q receives stage q's pick
 *   residual   [n_frames, dim] output, the residual left after the last
 *              stage; NULL to skip it
 *
 * The "RVQ codec" section of the "Architecture" page: residual loop.
 */
RVQ_API rvq_status rvq_encode(const float *x, int64_t n_frames, int32_t dim,
                              const float *codebooks, int32_t n_stages, int32_t n_codes,
                              int32_t *codes, int32_t codes_ld,
                              float *residual, void *stream);

/*
 * rvq_decode -- gather-sum decode.
 *
 *   codes      [n_frames, codes_ld] input; columns 0..n_stages-1 are read
 *   codebooks  [n_stages, n_codes, dim] (read only)
 *   out        [n_frames, dim] output, out[n] = sum_q codebooks[q, codes[n, q]]
 *
 * A code outside [0, n_codes) is a caller error: that frame's output row is
 * all quiet NaN and nothing outside the codebooks is read.
 *
 * The "RVQ codec" section of the "Architecture" page: per-codebook
 * get_rows, accumulated codebook 0 first.
 */
RVQ_API rvq_status rvq_decode(const int32_t *codes, int32_t codes_ld, int64_t n_frames,
                              const float *codebooks, int32_t n_stages, int32_t n_codes,
                              int32_t dim, float *out, void *stream);

/*
 * rvq_roundtrip -- encode, and reconstruct in the same pass.
 *
 * Same arguments as rvq_encode plus
 *   recon      [n_frames, dim] output, equal bit for bit to what rvq_decode
 *              returns for the codes written by this call.
 * residual may be NULL. This is the encode-then-decode reconstruction that
 * the moss-tts.cpp codec API calls "reconstruct" ("Maintainer's guide --
 * moss-tts.cpp", layout section), done without a second pass over memory.
 */
RVQ_API rvq_status rvq_roundtrip(const float *x, int64_t n_frames, int32_t dim,
                                 const float *codebooks, int32_t n_stages, int32_t n_codes,
                                 int32_t *codes, int32_t codes_ld,
                                 float *recon, float *residual, void *stream);

/*
 * rvq_encode_scored -- rvq_encode / rvq_roundtrip with an explicit scoring.
 *
 * recon and residual are both optional (NULL skips them). Any valid
 * `scoring` returns the same codes, residual and recon bit for bit; only
 * the speed differs. An unknown scoring value is RVQ_ERR_INVALID_ARG.
 */
RVQ_API rvq_status rvq_encode_scored(const float *x, int64_t n_frames, int32_t dim,
                                     const float *codebooks, int32_t n_stages, int32_t n_codes,
                                     int32_t *codes, int32_t codes_ld,
                                     float *recon, float *residual, rvq_scoring scoring, void *stream);

/*
 * Prepared codebooks: the codebook tensor in the layout the fp16
 * matrix-core encodes read, computed once (codebooks are model constants)
 * so that each encode only copies rows.
 *
 * rvq_prepared_bytes returns the size of the buffer for the given shape
 * (a negative rvq_status for invalid or unsupported shapes).
 * rvq_prepare_codebooks writes it on `stream` into caller-allocated device
 * memory `prepared` (16-byte aligned, at least rvq_prepared_bytes bytes).
 * Per stage it holds one power of two 2^e that brings max |c| into
 * [1/2, 1), each codeword as fp16(2^e c), 0.5*||2^e c||^2 as two fp16
 * parts, and the largest of those per 256 codewords (about 144 bytes per
 * codeword). The buffer depends only on the codebook values.
 *
 * rvq_encode_prepared reads `prepared` (which must have been prepared from
 * the same `codebooks` with at least `n_stages` stages and the same n_codes
 * and dim; the library cannot check this) and scores with one fp16
 * product per dimension: up to 8192 frames split every stage's codebook
 * over the wavefronts of a workgroup, more tile the frames. Either way
 * every codeword within the scores' proven error of the best is re-ranked
 * in float64, so results are identical to rvq_encode. Codebook entries
 * beyond 2^20 or residual entries beyond 2^15 leave fp16's range; such
 * stages and frames are decided by the full float64 rescan (same results,
 * slower).
 */
RVQ_API int64_t rvq_prepared_bytes(int32_t n_stages, int32_t n_codes, int32_t dim);
RVQ_API rvq_status rvq_prepare_codebooks(const float *codebooks, int32_t n_stages, int32_t n_codes,
                                         int32_t dim, void *prepared, int64_t prepared_bytes, void *stream);
RVQ_API rvq_status rvq_encode_prepared(const float *x, int64_t n_frames, int32_t dim,
                                       const float *codebooks, const void *prepared,
                                       int32_t n_stages, int32_t n_codes,
                                       int32_t *codes, int32_t codes_ld,
                                       float *recon, float *residual, void *stream);

/*
 * rvq_encode_noalloc -- rvq_encode_prepared without a caller buffer, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, results and errors as rvq_encode_prepared (recon and residual
 * may be NULL), with no `prepared` argument: every call prepares the
 * codebooks on `stream` into a fixed array of RVQ_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on each GPU it runs on (from first use until
 * the process ends), then encodes from it. The call allocates and frees
 * nothing. Shapes whose prepared layout exceeds the array
 * (rvq_prepared_bytes(n_stages, n_codes, dim) > RVQ_NOALLOC_SCRATCH_BYTES,
 * e.g. 113 stages of 1024 codewords or 28 of 4096 fit, 29 of 4096 do not)
 * return RVQ_ERR_UNSUPPORTED before anything is enqueued. The array is
 * shared by all calls on one GPU and keeps the last call's contents: calls
 * that overlap on one GPU (other streams or threads) race and must be
 * serialised by the caller. The stream's device is the GPU used.
 */
#define RVQ_NOALLOC_SCRATCH_BYTES (16LL * 1024 * 1024)
RVQ_API rvq_status rvq_encode_noalloc(const float *x, int64_t n_frames, int32_t dim,
                                      const float *codebooks, int32_t n_stages, int32_t n_codes,
                                      int32_t *codes, int32_t codes_ld,
                                      float *recon, float *residual, void *stream);

/*
 * rvq_project_roundtrip -- linear in, encode, decode, linear out.
 *
 * The "Audio tokenizer pipeline" section of the "Architecture" page puts a
 * linear layer (fc) before the RVQ encode and one (fc2) after the decode.
 * This runs, on `stream`, in order:
 *   latent       = h W_in^T + b_in              [n_frames, dim]
 *   codes        = encode(latent)               [n_frames, codes_ld]
 *   latent_recon = decode(codes)                [n_frames, dim]
 *   h_recon      = latent_recon W_out^T + b_out [n_frames, hidden]
 *
 *   h            [n_frames, hidden] input (read only)
 *   w_in         [dim, hidden]  PyTorch (out, in) order; b_in [dim] or NULL
 *   codebooks    [n_stages, n_codes, dim]
 *   prepared     NULL, or rvq_prepare_codebooks' output for these codebooks
 *                (16-byte aligned, at least rvq_prepared_bytes(n_stages,
 *                n_codes, dim) bytes); the encode then reads it as
 *                rvq_encode_prepared does (same results, faster)
 *   w_out        [hidden, dim]  PyTorch (out, in) order; b_out [hidden] or NULL
 *   codes, latent, latent_recon, h_recon: caller-allocated outputs
 *
 * The linear layers are fp32 sums on the matrix cores (bias added last):
 * fc as accurate as an fp32 contraction, fc2 within 3.01 * 2^-22 of
 * sum_k |x_k w_k| per output beyond the fp32 accumulation's own error;
 * encode and decode keep the contract above, applied to `latent`.
 * hidden must be a positive multiple of 64 (RVQ_ERR_UNSUPPORTED otherwise).
 */
RVQ_API rvq_status rvq_project_roundtrip(const float *h, int64_t n_frames, int32_t hidden,
                                         const float *w_in, const float *b_in,
                                         const float *codebooks, const void *prepared,
                                         int32_t n_stages, int32_t n_codes,
                                         int32_t dim, const float *w_out, const float *b_out,
                                         int32_t *codes, int32_t codes_ld, float *latent,
                                         float *latent_recon, float *h_recon, void *stream);

/*
 * Per-stage projected RVQ -- the codec quantizer of the "RVQ codec" section
 * of the "Architecture" page, where codebook q has its own project_in
 * (hidden -> dim, with bias) and project_out (dim -> hidden, with bias) and
 * the residual has the hidden width:
 *
 *   r = h;  for q: e_q = W_in[q] r + b_in[q];
 *                  k_q = argmin_i ||e_q - C[q,i]||^2 (lowest i on ties);
 *                  r   = r - (W_out[q] C[q,k_q] + b_out[q])
 *   decode: out = sum_q (W_out[q] C[q,k_q] + b_out[q]), stage 0 first
 *
 * Weights are in PyTorch (out, in) order and stacked over the stages:
 *   w_in [n_stages, dim, hidden], b_in [n_stages, dim] or NULL,
 *   w_out [n_stages, hidden, dim], b_out [n_stages, hidden] or NULL.
 * dim must be 64 (8 for the table of the normalized quantizer below) and
 * hidden a positive multiple of 64 (RVQ_ERR_UNSUPPORTED otherwise). All
 * pointers are caller-owned device memory, 16-byte aligned (codes 4-byte);
 * calls enqueue on `stream` and return.
 *
 * rvq_projected_prepare writes the table of projected codewords
 *   table [n_stages, n_codes, hidden] float32,
 *   table[q,k,i] = float32(sum_j W_out[q,i,j] C[q,k,j] + b_out[q,i]),
 * each entry a float64 sum over j ascending with the bias added last,
 * rounded once. It depends only on the weights and codebooks.
 *
 * rvq_projected_encode runs the loop above on n_frames hidden vectors h
 * [n_frames, hidden], reading the out-projections from `table` (prepared
 * from the same codebooks and weights; the library cannot check this).
 * `prepared` is NULL or rvq_prepare_codebooks' output for `codebooks`
 * (at least rvq_prepared_bytes(n_stages, n_codes, dim) bytes): each
 * stage's argmin then reads its stage block (same results, faster).
 *   codes    [n_frames, codes_ld] output, column q = k_q
 *   latent   [n_stages, n_frames, dim] output, latent[q] = e_q, computed as
 *            fp32 sums on the matrix cores (bias added last); the argmin of
 *            stage q is exact for these values
 *   residual [n_frames, hidden] output, the residual after the last stage,
 *            each update r_i = float32(r_i - table[q,k_q,i]); it is also the
 *            working buffer between stages and may be h itself (h is then
 *            overwritten).
 * latent must not overlap h, residual or codes.
 *
 * rvq_projected_decode: out [n_frames, hidden] = sum_q table[q, codes[n,q]],
 * a float32 accumulator from +0, stage 0 first; a code outside
 * [0, n_codes) gives a NaN row.
 */
RVQ_API rvq_status rvq_projected_prepare(const float *codebooks, int32_t n_stages, int32_t n_codes,
                                         int32_t dim, const float *w_out, const float *b_out,
                                         int32_t hidden, float *table, void *stream);
RVQ_API rvq_status rvq_projected_encode(const float *h, int64_t n_frames, int32_t hidden,
                                        const float *w_in, const float *b_in,
                                        const float *codebooks, const void *prepared, const float *table,
                                        int32_t n_stages, int32_t n_codes, int32_t dim,
                                        int32_t *codes, int32_t codes_ld,
                                        float *latent, float *residual, void *stream);
RVQ_API rvq_status rvq_projected_decode(const int32_t *codes, int32_t codes_ld, int64_t n_frames,
                                        const float *table, int32_t n_stages, int32_t n_codes,
                                        int32_t hidden, float *out, void *stream);

/*
 * Normalized (cosine) per-stage projected RVQ -- the quantizer of the
 * "Maintainer's guide -- moss-tts.cpp" page (gotchas, item 9): the same
 * loop as rvq_projected_encode with an 8-dim codebook space, where the
 * argmin compares the projection and the codewords scaled to unit L2 norm:
 *
 *   u = e_q / max(|e_q|, 1e-12),  v_k = C[q,k] / max(|C[q,k]|, 1e-12),
 *   k_q = argmin_k sum_j (u_j - v_kj)^2   (lowest k on ties)
 *
 * decided exactly as in float64 (a frame the fp32 scores cannot separate
 * is rescanned in float64). The residual update and the decode use the
 * stored, unscaled codeword: table from rvq_projected_prepare with dim 8,
 * decode with rvq_projected_decode.
 *
 * rvq_cosine_prepare writes units [n_stages, n_codes, 8] float64 (16-byte
 * aligned, caller-owned), the unit codewords v computed in float64
 * (squares summed in order, sqrt, one division per element).
 *
 * rvq_cosine_encode: arguments as rvq_projected_encode, with `units` in
 * place of `codebooks` and `prepared`, dim == 8, hidden a multiple of 64
 * and at most 1024 (RVQ_ERR_UNSUPPORTED otherwise),
 * `units` from rvq_cosine_prepare and `table` from rvq_projected_prepare
 * (both from the same codebooks and weights), latent [n_stages, n_frames, 8]
 * the fp32 projections e_q (bias added last).
 */
RVQ_API rvq_status rvq_cosine_prepare(const float *codebooks, int32_t n_stages, int32_t n_codes, int32_t dim,
                                      double *units, void *stream);
RVQ_API rvq_status rvq_cosine_encode(const float *h, int64_t n_frames, int32_t hidden,
                                     const float *w_in, const float *b_in,
                                     const double *units, const float *table,
                                     int32_t n_stages, int32_t n_codes, int32_t dim,
                                     int32_t *codes, int32_t codes_ld,
                                     float *latent, float *residual, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RVQ_H */
