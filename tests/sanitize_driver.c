/* Host-side validation paths of every entry point of include/absa.h, for a
 * build of the host layer with AddressSanitizer and UndefinedBehaviorSanitizer.
 * No call here reaches the device: every one is rejected by argument checks,
 * so the driver runs without a GPU. Exit status 0 when every call returns the
 * expected status. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "absa.h"

static int failures = 0;

static void expect(const char* what, absa_status got, absa_status want) {
    if (got != want) {
        fprintf(stderr, "%s: got %s, want %s (%s)\n", what, absa_status_string(got),
                absa_status_string(want), absa_last_error());
        ++failures;
    } else if (want != ABSA_OK && absa_last_error()[0] == '\0') {
        fprintf(stderr, "%s: no detail message\n", what);
        ++failures;
    }
}

int main(void) {
    void* fake = (void*)0x1000;     /* never dereferenced */
    absa_plan plan = NULL;
    absa_plan_params p;
    expect("params init", absa_plan_params_init(&p), ABSA_OK);
    expect("params init NULL", absa_plan_params_init(NULL), ABSA_ERR_INVALID_ARG);
    p.budget_blocks = 10;

    /* plan_create: shapes and parameters */
    expect("create out NULL", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 64, &p, NULL, NULL),
           ABSA_ERR_INVALID_ARG);
    expect("create q NULL", absa_plan_create(NULL, fake, ABSA_BF16, 1, 1, 1024, 64, &p, NULL, &plan),
           ABSA_ERR_INVALID_ARG);
    expect("create d", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 96, &p, NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    expect("create N", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1026, 64, &p, NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    expect("create huge", absa_plan_create(fake, fake, ABSA_BF16, INT64_MAX / 2, 1 << 20, 1024, 64,
                                           &p, NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    expect("create dtype", absa_plan_create(fake, fake, (absa_dtype)9, 1, 1, 1024, 64, &p, NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    p.n_clusters = 17;
    expect("create clusters", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 64, &p, NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    p.n_clusters = 8;
    p.budget_blocks = 257;
    expect("create budget", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 64, &p, NULL, &plan),
           ABSA_ERR_INVALID_ARG);
    p.budget_blocks = 10;
    p.sampling = 7;
    expect("create sampling", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 64, &p, NULL, &plan),
           ABSA_ERR_INVALID_ARG);
    p.sampling = ABSA_SAMPLING_POISSON;
    p.fused = 1;
    p.n_clusters = 12;
    expect("create fused clusters", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 64, &p, NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    p.n_clusters = 8;
    expect("create fused long rows", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 4 * 20228, 64, &p,
                                                      NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    p.keep_intermediates = 1;
    expect("create fused intermediates", absa_plan_create(fake, fake, ABSA_BF16, 1, 1, 1024, 64, &p,
                                                          NULL, &plan),
           ABSA_ERR_UNSUPPORTED);
    p.keep_intermediates = 0;
    p.fused = 0;
    if (plan != NULL) { fprintf(stderr, "a rejected call returned a plan\n"); ++failures; }

    /* plan_from_scores */
    expect("scores NULL", absa_plan_from_scores(NULL, 1, 1, 1024, 64, 10, 0, 0, NULL, &plan),
           ABSA_ERR_INVALID_ARG);
    expect("scores budget", absa_plan_from_scores((const float*)fake, 1, 1, 1024, 64, 0, 0, 0, NULL, &plan),
           ABSA_ERR_INVALID_ARG);

    /* plan_import: host CSR checks (B=1, H=1, N=256: one row, M = 64) */
    {
        int64_t rowptr_bad0[3] = {1, 2, 2};
        int64_t rowptr[3] = {0, 3, 3};
        int32_t idx_desc[3] = {5, 4, 9};
        int32_t idx_range[3] = {1, 2, 64};
        int32_t idx_ok[3] = {1, 2, 63};
        float logw[3] = {0.0f, 0.5f, 1.0f};
        float logw_inf[3] = {0.0f, 1.0f / 0.0f, 1.0f};
        int64_t rowptr2[3] = {0, 65, 65};
        int32_t many[65];
        float lw65[65];
        for (int i = 0; i < 65; ++i) { many[i] = i; lw65[i] = 0.0f; }
        int64_t rp_one[2] = {0, 3};
        expect("import rowptr[0]", absa_plan_import(rowptr_bad0, idx_ok, logw, NULL, 1, 1, 256, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
        /* N = 256 has 2 rows of 128 queries */
        expect("import descending", absa_plan_import(rowptr, idx_desc, logw, NULL, 1, 1, 256, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
        expect("import range", absa_plan_import(rowptr, idx_range, logw, NULL, 1, 1, 256, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
        expect("import logw", absa_plan_import(rowptr, idx_ok, logw_inf, NULL, 1, 1, 256, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
        expect("import too many", absa_plan_import(rowptr2, many, lw65, NULL, 1, 1, 256, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
        expect("import NULL idx", absa_plan_import(rp_one, NULL, logw, NULL, 1, 1, 128, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
        expect("import NULL rowptr", absa_plan_import(NULL, idx_ok, logw, NULL, 1, 1, 128, 64, NULL, &plan),
               ABSA_ERR_INVALID_ARG);
    }

    /* calls on a plan, attention */
    expect("info NULL", absa_plan_info(NULL, NULL, NULL, NULL, NULL), ABSA_ERR_INVALID_ARG);
    expect("export NULL", absa_plan_export(NULL, NULL, NULL, NULL, NULL), ABSA_ERR_INVALID_ARG);
    expect("intermediate NULL", absa_plan_export_intermediate(NULL, ABSA_INTER_SCORES, 0, 0, NULL),
           ABSA_ERR_INVALID_ARG);
    {
        const float* sp = (const float*)fake;
        expect("scores accessor NULL", absa_plan_scores(NULL, &sp), ABSA_ERR_INVALID_ARG);
    }
    expect("sparse NULL plan", absa_sparse_attention(NULL, fake, fake, fake, fake, ABSA_BF16, 1, 1, 1024, 64, NULL),
           ABSA_ERR_INVALID_ARG);
    expect("noalloc NULL plan",
           absa_sparse_attention_noalloc(NULL, fake, fake, fake, fake, ABSA_BF16, 1, 1, 1024, 64, NULL),
           ABSA_ERR_INVALID_ARG);
    expect("dense v NULL", absa_dense_attention(fake, fake, NULL, fake, ABSA_BF16, 1, 1, 1024, 64, NULL),
           ABSA_ERR_INVALID_ARG);
    expect("dense d", absa_dense_attention(fake, fake, fake, fake, ABSA_BF16, 1, 1, 1024, 48, NULL),
           ABSA_ERR_UNSUPPORTED);
    absa_plan_destroy(NULL);
    if (strcmp(absa_status_string(ABSA_ERR_PLAN_MISMATCH), "ABSA_ERR_PLAN_MISMATCH") != 0) ++failures;
    if (strcmp(absa_status_string((absa_status)99), "ABSA_UNKNOWN_STATUS") != 0) ++failures;
    printf("sanitized host checks: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
