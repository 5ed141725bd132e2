/* Plain C99 consumer of include/rvq.h: compiled with -std=c99 -Wall -Werror
 * -pedantic by tests/test_abi.py, and run on the CPU. Every call below takes
 * an early-return path (argument checks or the n_frames == 0 no-op), so no
 * GPU is touched. */
#include <stdio.h>
#include <string.h>

#include "rvq.h"

static int expect(const char *what, rvq_status got, rvq_status want)
{
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d\n", what, (int)got, rvq_status_string(got), (int)want);
        return 1;
    }
    return 0;
}

int main(void)
{
    int bad = 0;
    float *fx = (float *)0x1000;  /* never dereferenced: each call fails validation first */
    int32_t *ic = (int32_t *)0x2000;
    if (strlen(rvq_version()) == 0) bad++;
    bad += expect("status string", strcmp(rvq_status_string(RVQ_ERR_DEVICE), "device error") == 0 ? RVQ_OK : RVQ_ERR_INVALID_ARG, RVQ_OK);
    bad += expect("encode null x", rvq_encode(NULL, 10, 64, fx, 8, 1024, ic, 8, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode n<0", rvq_encode(fx, -1, 64, fx, 8, 1024, ic, 8, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode dim 32", rvq_encode(fx, 10, 32, fx, 8, 1024, ic, 8, NULL, NULL), RVQ_ERR_UNSUPPORTED);
    bad += expect("encode q 0", rvq_encode(fx, 10, 64, fx, 0, 1024, ic, 8, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode k 0", rvq_encode(fx, 10, 64, fx, 8, 0, ic, 8, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode ld<q", rvq_encode(fx, 10, 64, fx, 8, 1024, ic, 7, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode misaligned", rvq_encode(fx + 1, 10, 64, fx, 8, 1024, ic, 8, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode too many stages", rvq_encode(fx, 10, 64, fx, 70000, 1024, ic, 70000, NULL, NULL), RVQ_ERR_UNSUPPORTED);
    bad += expect("encode empty", rvq_encode(NULL, 0, 64, NULL, 8, 1024, NULL, 8, NULL, NULL), RVQ_OK);
    bad += expect("roundtrip null recon", rvq_roundtrip(fx, 10, 64, fx, 8, 1024, ic, 8, NULL, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("roundtrip empty", rvq_roundtrip(NULL, 0, 64, NULL, 8, 1024, NULL, 8, NULL, NULL, NULL), RVQ_OK);
    bad += expect("decode null out", rvq_decode(ic, 8, 10, fx, 8, 1024, 64, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("decode dim 16", rvq_decode(ic, 8, 10, fx, 8, 1024, 16, fx, NULL), RVQ_ERR_UNSUPPORTED);
    bad += expect("decode ld<q", rvq_decode(ic, 4, 10, fx, 8, 1024, 64, fx, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("decode misaligned out", rvq_decode(ic, 8, 10, fx, 8, 1024, 64, fx + 2, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("decode empty", rvq_decode(NULL, 8, 0, NULL, 8, 1024, 64, NULL, NULL), RVQ_OK);
    bad += expect("project hidden 100", rvq_project_roundtrip(fx, 10, 100, fx, NULL, fx, NULL, 8, 1024, 64, fx, NULL,
                                                              ic, 8, fx, fx, fx, NULL), RVQ_ERR_UNSUPPORTED);
    bad += expect("project null h_recon", rvq_project_roundtrip(fx, 10, 1024, fx, NULL, fx, NULL, 8, 1024, 64, fx, NULL,
                                                                ic, 8, fx, fx, NULL, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("project misaligned bias", rvq_project_roundtrip(fx, 10, 1024, fx, fx + 1, fx, NULL, 8, 1024, 64, fx,
                                                                   NULL, ic, 8, fx, fx, fx, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("project misaligned prepared", rvq_project_roundtrip(fx, 10, 1024, fx, NULL, fx, (const char *)fx + 4,
                                                                       8, 1024, 64, fx, NULL, ic, 8, fx, fx, fx, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("project empty", rvq_project_roundtrip(NULL, 0, 1024, NULL, NULL, NULL, NULL, 8, 1024, 64, NULL, NULL,
                                                         NULL, 8, NULL, NULL, NULL, NULL), RVQ_OK);
    bad += expect("scored bad mode", rvq_encode_scored(fx, 10, 64, fx, 8, 1024, ic, 8, NULL, NULL, (rvq_scoring)7, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("scored empty", rvq_encode_scored(NULL, 0, 64, NULL, 8, 1024, NULL, 8, NULL, NULL, RVQ_SCORING_FP32, NULL),
                  RVQ_OK);
    bad += expect("prepared bytes dim", (rvq_status)rvq_prepared_bytes(8, 1024, 16), RVQ_ERR_UNSUPPORTED);
    if (rvq_prepared_bytes(8, 1024, 64) <= 0) bad++;
    bad += expect("prepare too small", rvq_prepare_codebooks(fx, 8, 1024, 64, fx, 16, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("prepare null", rvq_prepare_codebooks(NULL, 8, 1024, 64, fx, 1 << 30, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("encode prepared null", rvq_encode_prepared(fx, 10, 64, fx, NULL, 8, 1024, ic, 8, NULL, NULL, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("encode prepared empty", rvq_encode_prepared(NULL, 0, 64, NULL, NULL, 8, 1024, NULL, 8, NULL, NULL, NULL),
                  RVQ_OK);
    bad += expect("noalloc beyond its array", rvq_encode_noalloc(fx, 10, 64, fx, 64, 4096, ic, 64, NULL, NULL, NULL),
                  RVQ_ERR_UNSUPPORTED);
    bad += expect("noalloc null x", rvq_encode_noalloc(NULL, 10, 64, fx, 8, 1024, ic, 8, NULL, NULL, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("noalloc ld<q", rvq_encode_noalloc(fx, 10, 64, fx, 8, 1024, ic, 7, NULL, NULL, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("noalloc empty", rvq_encode_noalloc(NULL, 0, 64, NULL, 8, 1024, NULL, 8, NULL, NULL, NULL), RVQ_OK);
    bad += expect("projected prepare hidden 96", rvq_projected_prepare(fx, 8, 1024, 64, fx, NULL, 96, fx, NULL),
                  RVQ_ERR_UNSUPPORTED);
    bad += expect("projected prepare null table", rvq_projected_prepare(fx, 8, 1024, 64, fx, NULL, 1024, NULL, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("projected prepare misaligned bias", rvq_projected_prepare(fx, 8, 1024, 64, fx, fx + 1, 1024, fx, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("projected encode null latent", rvq_projected_encode(fx, 10, 1024, fx, NULL, fx, NULL, fx, 8, 1024, 64,
                                                                       ic, 8, NULL, fx, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("projected encode dim 32", rvq_projected_encode(fx, 10, 1024, fx, NULL, fx, NULL, fx, 8, 1024, 32,
                                                                  ic, 8, fx, fx, NULL), RVQ_ERR_UNSUPPORTED);
    bad += expect("projected encode ld<q", rvq_projected_encode(fx, 10, 1024, fx, NULL, fx, NULL, fx, 8, 1024, 64,
                                                                ic, 7, fx, fx, NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("projected encode misaligned prepared",
                  rvq_projected_encode(fx, 10, 1024, fx, NULL, fx, (const char *)fx + 8, fx, 8, 1024, 64, ic, 8, fx, fx,
                                       NULL), RVQ_ERR_INVALID_ARG);
    bad += expect("projected encode empty", rvq_projected_encode(NULL, 0, 1024, NULL, NULL, NULL, NULL, NULL, 8, 1024, 64,
                                                                 NULL, 8, NULL, NULL, NULL), RVQ_OK);
    bad += expect("projected decode null out", rvq_projected_decode(ic, 8, 10, fx, 8, 1024, 1024, NULL, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("projected decode hidden 0", rvq_projected_decode(ic, 8, 10, fx, 8, 1024, 0, fx, NULL),
                  RVQ_ERR_INVALID_ARG);
    bad += expect("projected decode empty", rvq_projected_decode(NULL, 8, 0, NULL, 8, 1024, 1024, NULL, NULL), RVQ_OK);
    {
        double *ud = (double *)0x3000;
        bad += expect("cosine prepare dim 64", rvq_cosine_prepare(fx, 32, 1024, 64, ud, NULL), RVQ_ERR_UNSUPPORTED);
        bad += expect("cosine prepare null", rvq_cosine_prepare(fx, 32, 1024, 8, NULL, NULL), RVQ_ERR_INVALID_ARG);
        bad += expect("cosine encode hidden 2048", rvq_cosine_encode(fx, 10, 2048, fx, NULL, ud, fx, 32, 1024, 8,
                                                                     ic, 32, fx, fx, NULL), RVQ_ERR_UNSUPPORTED);
        bad += expect("cosine encode dim 64", rvq_cosine_encode(fx, 10, 1024, fx, NULL, ud, fx, 32, 1024, 64,
                                                                ic, 32, fx, fx, NULL), RVQ_ERR_UNSUPPORTED);
        bad += expect("cosine encode null units", rvq_cosine_encode(fx, 10, 1024, fx, NULL, NULL, fx, 32, 1024, 8,
                                                                    ic, 32, fx, fx, NULL), RVQ_ERR_INVALID_ARG);
        bad += expect("cosine encode empty", rvq_cosine_encode(NULL, 0, 1024, NULL, NULL, NULL, NULL, 32, 1024, 8,
                                                               NULL, 32, NULL, NULL, NULL), RVQ_OK);
        bad += expect("projected prepare dim 8 hidden 96", rvq_projected_prepare(fx, 32, 1024, 8, fx, NULL, 96, fx, NULL),
                      RVQ_ERR_UNSUPPORTED);
        bad += expect("projected prepare dim 16", rvq_projected_prepare(fx, 32, 1024, 16, fx, NULL, 1024, fx, NULL),
                      RVQ_ERR_UNSUPPORTED);
    }
    printf("%s\n", bad ? "abi_c99: FAILED" : "abi_c99: ok");
    return bad ? 1 : 0;
}
