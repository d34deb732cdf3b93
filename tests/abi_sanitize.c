/* Drives every entry point of libaaren through its argument validation (test
 * program, CPU only): each call below is rejected before anything reaches
 * the HIP runtime, so it runs without a GPU. Built together with a copy of
 * the library whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py): an out-of-bounds
 * access, a signed overflow in the size arithmetic or a misaligned load in
 * any validation path ends the program with a report.
 *
 * Each case states the status it expects; the program prints the number of
 * cases and exits with status 1 on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "aaren.h"

static int cases, failures;

static void expect(int line, aaren_status got, aaren_status want)
{
    ++cases;
    if (got != want) {
        fprintf(stderr, "line %d: status %d, expected %d (%s)\n", line, (int)got, (int)want,
                aaren_last_error());
        ++failures;
    } else if (got != AAREN_OK && strlen(aaren_last_error()) == 0) {
        fprintf(stderr, "line %d: status %d without a description\n", line, (int)got);
        ++failures;
    }
}

#define EXPECT(call, want) expect(__LINE__, (call), (want))

int main(void)
{
    /* addresses that are never dereferenced: aligned and misaligned */
    char *const A = (char *)0x10000, *const M = (char *)0x10004;
    float *const FA = (float *)A;
    const int64_t BIG = INT64_MAX, NEG = -1;
    const size_t WS = (size_t)1 << 40;
    const aaren_dtype F = AAREN_F32, BF = AAREN_BF16, BAD = (aaren_dtype)9;
    const int64_t st3[3] = {64, 64, 64}, neg3[3] = {-64, 64, 64}, odd3[3] = {1, 64, 64};
    const int64_t huge3[3] = {INT64_MAX, 64, 64};
    const int64_t *offs = (const int64_t *)A;

    /* status strings and the version */
    for (int s = -3; s < 12; ++s)
        if (!aaren_status_string((aaren_status)s))
            ++failures;
    if (aaren_version() <= 0)
        ++failures;

    /* size queries: rejected shapes give 0, extreme ones never overflow */
    const int64_t dims[] = {NEG, 0, 1, 4096, (int64_t)1 << 31, (int64_t)1 << 62, BIG};
    const int64_t ds[] = {NEG, 0, 63, 64, 128, BIG};
    for (unsigned a = 0; a < sizeof dims / sizeof *dims; ++a)
        for (unsigned b = 0; b < sizeof dims / sizeof *dims; ++b)
            for (unsigned c = 0; c < sizeof ds / sizeof *ds; ++c) {
                const int64_t x = dims[a], y = dims[b], d = ds[c];
                (void)aaren_scan_workspace_size(x, y, x, d);
                (void)aaren_scan_workspace_size(1, x, y, d);
                (void)aaren_scan_segmented_workspace_size(x, y, 8, d);
                (void)aaren_scan_segmented_workspace_size(1, x, y, d);
                (void)aaren_scan_backward_workspace_size(x, 1, y, d);
                (void)aaren_scan_segmented_backward_workspace_size(x, y, 8, d);
                (void)aaren_reduce_workspace_size(x, 1, y, d);
                (void)aaren_reduce_workspace_size(1, x, y, d);
                (void)aaren_self_attention_workspace_size(x, 1, y, d);
                (void)aaren_mean_query_attention_workspace_size(x, 1, y, d);
                (void)aaren_layer_workspace_size(x, y, 64, 8, d);
                (void)aaren_layer_workspace_size(1, x, y, 8, d);
                ++cases;
            }

    /* dense scan and its lse form */
    EXPECT(aaren_scan(A, A, A, A, NEG, 1, 16, 64, .125f, F, F, A, WS, NULL), AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan(A, A, A, A, 1, 1, 16, 65, .125f, F, F, A, WS, NULL), AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan(A, A, A, A, 1, 1, 16, 64, .125f, BAD, F, A, WS, NULL), AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan(A, A, A, A, BIG, BIG, BIG, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan(A, A, A, A, 1 << 20, 1 << 20, 1 << 20, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan(NULL, A, A, A, 1, 1, 16, 64, .125f, F, F, A, WS, NULL), AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan(A, M, A, A, 1, 1, 16, 64, .125f, F, F, A, WS, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_scan(A, A, A, A, 1, 1, 16, 64, .125f, F, F, A, 100, NULL), AAREN_ERR_WORKSPACE);
    EXPECT(aaren_scan(A, A, A, A, 1, 1, 16, 64, .125f, F, F, M, WS, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_scan(NULL, NULL, NULL, NULL, 0, 1, 16, 64, .125f, F, F, NULL, 0, NULL), AAREN_OK);
    EXPECT(aaren_scan_lse(A, A, A, A, NULL, 1, 1, 16, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan_lse(A, A, A, A, (float *)(A + 2), 1, 1, 16, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_scan_strided(A, A, A, A, NULL, 1, 8, 100, 64, NULL, st3, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan_strided(A, A, A, A, NULL, 1, 8, 100, 64, neg3, st3, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan_strided(A, A, A, A, NULL, 1, 8, 100, 64, odd3, st3, .125f, F, F, A, WS, NULL),
           AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_scan_strided(A, A, A, A, NULL, 1, 8, 100, 64, huge3, st3, .125f, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);

    EXPECT(aaren_scan_noalloc(A, A, A, A, 1, 1, (int64_t)1 << 27, 64, .125f, F, F, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan_noalloc(A, A, A, A, BIG, BIG, BIG, 64, .125f, F, F, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan_noalloc(A, A, A, A, 1, 1, 16, 64, .125f, BAD, F, NULL), AAREN_ERR_UNSUPPORTED);

    /* packed scan */
    EXPECT(aaren_scan_segmented(A, A, A, A, NULL, 2, 10, 1, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan_segmented(A, A, A, A, (const int64_t *)M, 2, 10, 1, 64, .125f, F, F, A, WS,
                                NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_scan_segmented(A, A, A, A, offs, 0, 10, 1, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan_segmented(A, A, A, A, offs, 2, BIG, BIG, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan_segmented(A, A, A, A, offs, 2, 10, 1, 64, .125f, F, BF, A, 64, NULL),
           AAREN_ERR_WORKSPACE);
    EXPECT(aaren_scan_segmented(A, A, A, A, offs, 0, 0, 1, 64, .125f, F, F, NULL, 0, NULL), AAREN_OK);
    EXPECT(aaren_scan_segmented_lse(A, A, A, A, NULL, offs, 2, 10, 1, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);

    /* gradients */
    EXPECT(aaren_scan_backward(A, A, A, A, A, NULL, FA, FA, FA, 1, 1, 16, 64, .125f, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_scan_backward(A, A, A, A, A, FA, FA, FA, FA, 1, 1, 16, 64, .125f, F, A, 10, NULL),
           AAREN_ERR_WORKSPACE);
    EXPECT(aaren_scan_backward(A, A, A, A, A, FA, FA, FA, FA, BIG, 2, BIG, 64, .125f, F, A, WS,
                               NULL), AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_scan_segmented_backward(A, A, A, A, A, FA, (const int64_t *)M, FA, FA, FA, 3, 50, 2,
                                         64, .125f, F, A, WS, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_scan_segmented_backward(A, A, A, A, A, FA, offs, FA, FA, FA, 0, 50, 2, 64, .125f, F,
                                         A, WS, NULL), AAREN_ERR_INVALID_ARG);

    /* step, state, append */
    EXPECT(aaren_state_init(FA, FA, (float *)(A + 4), 4, 2, 64, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_state_init(FA, FA, FA, BIG, BIG, 64, NULL), AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_step(A, A, A, NULL, FA, FA, NULL, 4, 2, 64, .125f, F, F, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_step(A, A, A, FA, FA, FA, M, 4, 2, 64, .125f, F, F, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_step(A, A, A, FA, FA, FA, NULL, BIG, BIG, 64, .125f, F, F, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_append(A, A, A, FA, FA, FA, NULL, 4, NEG, 2, 64, .125f, F, F, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_append(A, A, A, FA, FA, FA, NULL, BIG, BIG, 2, 64, .125f, F, F, NULL),
           AAREN_ERR_UNSUPPORTED);

    /* reduce and mean query */
    EXPECT(aaren_reduce(A, A, A, A, NULL, NULL, 1, 2, 0, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_reduce(A, A, A, A, (float *)(A + 1), NULL, 1, 2, 10, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_reduce(A, A, A, A, NULL, NULL, BIG, BIG, 10, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_reduce(A, A, A, A, NULL, NULL, 1, 2, 10, 64, .125f, F, F, A, 8, NULL),
           AAREN_ERR_WORKSPACE);
    EXPECT(aaren_mean_query_attention(A, A, A, A, NULL, 1, 2, 0, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_mean_query_attention(A, A, A, A, FA, BIG, 2, BIG, 64, .125f, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);

    /* self-attention */
    EXPECT(aaren_self_attention(A, A, A, A, NULL, 1, 2, 100, 64, .125f, 1, F, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_self_attention(A, A, A, A, NULL, 1, 2, (int64_t)1 << 23, 64, .125f, 1, BF, F, A, WS,
                                NULL), AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_self_attention(A, A, A, A, NULL, 1 << 17, 1, 100, 64, .125f, 1, BF, F, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_self_attention(A, A, A, A, NULL, 1, 2, 100, 64, .125f, 1, BF, F, A, 16, NULL),
           AAREN_ERR_WORKSPACE);

    /* layer */
    EXPECT(aaren_layer_forward(A, A, FA, A, 1, 10, 0, 2, 64, .125f, BF, A, WS, NULL),
           AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_layer_forward(A, A, FA, A, 1, (int64_t)1 << 40, 64, 2, 64, .125f, BF, A, WS, NULL),
           AAREN_ERR_UNSUPPORTED);
    EXPECT(aaren_layer_forward(A, M, FA, A, 1, 10, 64, 2, 64, .125f, BF, A, WS, NULL),
           AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_layer_forward(A, A, FA, A, 1, 10, 64, 2, 64, .125f, BF, A, 64, NULL),
           AAREN_ERR_WORKSPACE);

    /* workspaces */
    EXPECT(aaren_workspace_clear(M, 4096, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_workspace_clear(NULL, 4096, NULL), AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_workspace_clear(NULL, 0, NULL), AAREN_OK);
    EXPECT(aaren_workspace_status(NULL, 4096, (uint32_t *)A, 0, NULL), AAREN_ERR_INVALID_ARG);
    EXPECT(aaren_workspace_status(A, 4096, (uint32_t *)(A + 2), 0, NULL), AAREN_ERR_ALIGNMENT);
    EXPECT(aaren_workspace_status(A, 100, (uint32_t *)A, 0, NULL), AAREN_ERR_WORKSPACE);

    printf("%d cases, %d failures\n", cases, failures);
    return failures ? 1 : 0;
}
