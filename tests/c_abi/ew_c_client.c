/*
 * ew_c_client.c -- a plain C11 client of the libew C ABI (include/ew.h):
 * no C++, no torch.  Test infrastructure: it allocates device memory with
 * the HIP runtime's C API, calls the library on a non-default stream, and
 * compares every element with the CPU oracle (liboracle.so).  Exit status 0
 * when every check passes.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include "ew.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's entry points (oracle/oracle.c). */
void oracle_add_f32(const float *a, const float *b, float *c, size_t n);
void oracle_relu_f32(const float *x, float *y, size_t n);
void oracle_gather_f32(const float *in, float *out, size_t n, size_t stride);
void oracle_copy2d_f32(const float *in, int64_t stride_r, int64_t stride_c, float *out,
                       size_t rows, size_t cols);
void oracle_sqrt_f32(const float *x, float *y, size_t n);
void oracle_scale_f32(float alpha, const float *x, float *y, size_t n);

static int failures = 0, checks = 0;

#define HIP_OK(call)                                                                 \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,          \
                    hipGetErrorString(e_));                                          \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

/* Finite test values in [-2, 2): a counter hashed to 24 random bits. */
static void fill(float *x, size_t n, uint32_t seed)
{
    for (size_t i = 0; i < n; ++i) {
        uint32_t h = (uint32_t)i * 2654435761u ^ seed;
        h ^= h >> 15;
        h *= 2246822519u;
        h ^= h >> 13;
        x[i] = (float)((int32_t)(h >> 8) - (1 << 23)) * (1.0f / (1 << 22));
    }
}

static void expect_equal(const char *what, const float *got, const float *ref, size_t n)
{
    ++checks;
    if (memcmp(got, ref, n * sizeof(float)) != 0) {
        size_t i = 0;
        while (i < n && memcmp(&got[i], &ref[i], sizeof(float)) == 0) ++i;
        fprintf(stderr, "FAIL %s: first difference at %zu (%a vs %a)\n", what, i,
                (double)got[i], (double)ref[i]);
        ++failures;
    }
}

static void expect_status(const char *what, ew_status_t got, ew_status_t want)
{
    ++checks;
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d (%s), expected %d\n", what, (int)got,
                ew_status_string(got), (int)want);
        ++failures;
    }
}

int main(void)
{
    const size_t n = 1000003;                   /* ragged, and coprime with 3 */
    const size_t rows = 300, cols = 517;        /* a transposed view of cols x rows */
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    float *ha = malloc((n + 1) * sizeof *ha), *hb = malloc(n * sizeof *hb);
    float *got = malloc(n * sizeof *got), *ref = malloc(n * sizeof *ref);
    if (!ha || !hb || !got || !ref) return 2;
    fill(ha, n + 1, 1u);
    fill(hb, n, 2u);

    float *da, *db, *dc;
    HIP_OK(hipMalloc((void **)&da, (n + 1) * sizeof *da));
    HIP_OK(hipMalloc((void **)&db, n * sizeof *db));
    HIP_OK(hipMalloc((void **)&dc, n * sizeof *dc));
    HIP_OK(hipMemcpy(da, ha, (n + 1) * sizeof *da, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(db, hb, n * sizeof *db, hipMemcpyHostToDevice));

    /* add with A one element past its allocation (misaligned body) */
    expect_status("ew_add_f32", ew_add_f32(da + 1, db, dc, n, s), EW_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dc, n * sizeof *got, hipMemcpyDeviceToHost));
    oracle_add_f32(ha + 1, hb, ref, n);
    expect_equal("ew_add_f32", got, ref, n);

    /* gather with stride 3 (three passes) */
    expect_status("ew_gather_f32", ew_gather_f32(db, dc, n, 3, s), EW_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dc, n * sizeof *got, hipMemcpyDeviceToHost));
    oracle_gather_f32(hb, ref, n, 3);
    expect_equal("ew_gather_f32 stride 3", got, ref, n);

    /* transposed view: out[r*cols + c] = b[r + c*rows] */
    expect_status("ew_copy2d_f32", ew_copy2d_f32(db, 1, (int64_t)rows, dc, rows, cols, s), EW_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dc, rows * cols * sizeof *got, hipMemcpyDeviceToHost));
    oracle_copy2d_f32(hb, 1, (int64_t)rows, ref, rows, cols);
    expect_equal("ew_copy2d_f32 transpose", got, ref, rows * cols);

    /* in-place ReLU on b */
    expect_status("ew_relu_inplace_f32", ew_relu_inplace_f32(db, n, s), EW_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, db, n * sizeof *got, hipMemcpyDeviceToHost));
    oracle_relu_f32(hb, ref, n);
    expect_equal("ew_relu_inplace_f32", got, ref, n);

    /* a unary map: sqrt of |a| (abs first, in place on c) */
    expect_status("ew_abs_f32", ew_abs_f32(da + 1, dc, n, s), EW_OK);
    expect_status("ew_sqrt_f32", ew_sqrt_f32(dc, dc, n, s), EW_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dc, n * sizeof *got, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < n; ++i) ref[i] = ha[i + 1] < 0 ? -ha[i + 1] : ha[i + 1];
    oracle_sqrt_f32(ref, ref, n);
    expect_equal("ew_abs_f32 + ew_sqrt_f32", got, ref, n);

    /* a batched call: 130 items (two launches) of a scale by 2.5, item k
     * covering k * 7 + 1 elements of a at offset k, written to c */
    {
        enum { ITEMS = 130 };
        ew_batch_item_t items[ITEMS];
        size_t at = 0;
        for (int k = 0; k < ITEMS; ++k) {
            const size_t m = (size_t)k * 7 + 1;
            items[k].out = dc + at;
            items[k].in0 = da + at + (size_t)(k % 4);
            items[k].in1 = NULL;
            items[k].n = m;
            at += m + 5;
        }
        HIP_OK(hipMemset(dc, 0, n * sizeof *dc));
        expect_status("ew_batch scale_f32", ew_batch("scale_f32", 2.5f, items, ITEMS, s), EW_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(got, dc, at * sizeof *got, hipMemcpyDeviceToHost));
        memset(ref, 0, at * sizeof *ref);
        at = 0;
        for (int k = 0; k < ITEMS; ++k) {
            const size_t m = (size_t)k * 7 + 1;
            oracle_scale_f32(2.5f, ha + at + (size_t)(k % 4), ref + at, m);
            at += m + 5;
        }
        expect_equal("ew_batch scale_f32", got, ref, at);
        items[1].out = dc;                         /* meets item 0's output */
        expect_status("ew_batch overlap", ew_batch("scale_f32", 2.5f, items, ITEMS, s),
                      EW_ERR_OVERLAP);
        expect_status("ew_batch op", ew_batch("gather_f32", 0.0f, items, ITEMS, s),
                      EW_ERR_INVALID_ARG);
    }

    /* the same batch through a device item table: one launch */
    {
        enum { ITEMS = 130 };
        ew_batch_item_t items[ITEMS];
        size_t at = 0;
        for (int k = 0; k < ITEMS; ++k) {
            const size_t m = (size_t)k * 7 + 1;
            items[k].out = dc + at;
            items[k].in0 = da + at + (size_t)(k % 4);
            items[k].in1 = NULL;
            items[k].n = m;
            at += m + 5;
        }
        ew_batch_plan_t plan;
        expect_status("ew_batch_build size", ew_batch_build("scale_f32", items, ITEMS, NULL, 0,
                                                            &plan), EW_OK);
        uint64_t *image = malloc(plan.bytes);
        void *table = NULL;
        if (!image) return 2;
        expect_status("ew_batch_build", ew_batch_build("scale_f32", items, ITEMS, image,
                                                       plan.bytes, &plan), EW_OK);
        HIP_OK(hipMalloc(&table, plan.bytes));
        HIP_OK(hipMemcpy(table, image, plan.bytes, hipMemcpyHostToDevice));
        HIP_OK(hipMemset(dc, 0, n * sizeof *dc));
        expect_status("ew_batch_run", ew_batch_run(&plan, 2.5f, table, s), EW_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(got, dc, at * sizeof *got, hipMemcpyDeviceToHost));
        memset(ref, 0, at * sizeof *ref);
        at = 0;
        for (int k = 0; k < ITEMS; ++k) {
            const size_t m = (size_t)k * 7 + 1;
            oracle_scale_f32(2.5f, ha + at + (size_t)(k % 4), ref + at, m);
            at += m + 5;
        }
        expect_equal("ew_batch_run scale_f32", got, ref, at);
        expect_status("ew_batch_run misaligned table",
                      ew_batch_run(&plan, 2.5f, (const char *)table + 4, s), EW_ERR_MISALIGNED);
        HIP_OK(hipFree(table));
        free(image);
    }

    /* the per-output index walk of the strided gather, stride 2 */
    expect_status("ew_gather_walk_f32", ew_gather_walk_f32(da, dc, n, 2, s), EW_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dc, n * sizeof *got, hipMemcpyDeviceToHost));
    oracle_gather_f32(ha, ref, n, 2);
    expect_equal("ew_gather_walk_f32 stride 2", got, ref, n);

    /* one launch configuration for every size: what get reports is what the
     * next call launches (block, unroll; grid = min(4 * CUs, tiles)) */
    {
        int dev = 0, cus = 0, block = 0, grid = 0, unroll = 0;
        HIP_OK(hipGetDevice(&dev));
        HIP_OK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
        expect_status("ew_set_launch_config", ew_set_launch_config("copy_f32", 256, 4, 2), EW_OK);
        expect_status("ew_get_launch_config",
                      ew_get_launch_config("copy_f32", n, &block, &grid, &unroll), EW_OK);
        const size_t tiles = (n / 4 + 511) / 512;
        const int want = (size_t)(4 * cus) < tiles ? 4 * cus : (int)tiles;
        checks++;
        if (block != 256 || unroll != 2 || grid != want) {
            printf("FAIL ew_get_launch_config: block %d grid %d unroll %d, expected 256 %d 2\n",
                   block, grid, unroll, want);
            failures++;
        }
        expect_status("ew_set_launch_config range", ew_set_launch_config("copy_f32", 96, 4, 2),
                      EW_ERR_INVALID_ARG);
        expect_status("ew_copy_f32", ew_copy_f32(db, dc, n, s), EW_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(got, dc, n * sizeof *got, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ref, db, n * sizeof *ref, hipMemcpyDeviceToHost));
        expect_equal("ew_copy_f32 under the set configuration", got, ref, n);
        ew_reset_launch_config();
    }

    /* errors are status codes, checked before any HIP call */
    expect_status("null pointer", ew_add_f32(NULL, db, dc, n, s), EW_ERR_INVALID_ARG);
    expect_status("misaligned", ew_add_f32((const float *)((const char *)da + 2), db, dc, n, s),
                  EW_ERR_MISALIGNED);
    expect_status("partial overlap", ew_add_f32(da, db, da + 1, n, s), EW_ERR_OVERLAP);
    expect_status("n == 0", ew_add_f32(NULL, NULL, NULL, 0, s), EW_OK);

    HIP_OK(hipFree(da));
    HIP_OK(hipFree(db));
    HIP_OK(hipFree(dc));
    HIP_OK(hipStreamDestroy(s));
    free(ha);
    free(hb);
    free(got);
    free(ref);
    printf("c-abi client (ABI %d): %d of %d checks passed\n", ew_abi_version(),
           checks - failures, checks);
    return failures ? 1 : 0;
}
