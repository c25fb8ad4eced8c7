/* Randomised calls of every host-side path of the C ABI -- argument
 * validation, the plans, batch table images, launch rows, launch-table
 * files and status strings -- with fabricated device addresses (the host
 * code only does arithmetic on them) and edge-case sizes, strides and
 * offsets.  tests/test_abi_fuzz_cpu.py builds this with AddressSanitizer
 * and UndefinedBehaviorSanitizer against a library whose host code is
 * instrumented the same way and runs it where no GPU is visible: every call
 * that passes validation then ends with EW_ERR_NO_DEVICE before any launch.
 *
 * Checked besides the sanitizers: every status is one the header defines,
 * every status string is non-null, a plan that is returned satisfies the
 * identities the header states (head + vectors * vec + tail == n, tiles,
 * grid), and a built table image holds its items in order with every tile's
 * item index in range.
 *
 * usage: ew_fuzz ITERATIONS SEED SCRATCH_FILE
 * exit: 0 = clean, 1 = a check failed, 77 = a GPU is visible (not run). */
#include "ew.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t g_state;

static uint64_t rnd(void)   /* splitmix64 */
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t below(uint64_t m) { return m ? rnd() % m : 0; }

static int g_failures;
static long g_status_count[7];   /* EW_OK .. EW_ERR_TOO_LARGE, by -status */

static void fail(const char *what, long long a, long long b)
{
    if (g_failures++ < 20) fprintf(stderr, "FAIL %s (%lld, %lld)\n", what, a, b);
}

static void status_ok(ew_status_t st, const char *what)
{
    if (st > 0 || st < EW_ERR_TOO_LARGE) fail(what, (long long)st, 0);
    else ++g_status_count[-(int)st];
    if (!ew_status_string(st)) fail("null status string", (long long)st, 0);
}

static size_t pick_n(void)
{
    static const size_t fixed[] = {0, 1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 64, 1023, 1024,
                                   (size_t)1 << 20, ((size_t)1 << 31) - 1, (size_t)1 << 31,
                                   (size_t)1 << 32, ((size_t)1 << 32) + 5, (size_t)1 << 62,
                                   SIZE_MAX, SIZE_MAX / 2, SIZE_MAX / 4 + 1, SIZE_MAX / 16};
    switch (below(4)) {
    case 0: return fixed[below(sizeof fixed / sizeof fixed[0])];
    case 1: return (size_t)below(5000);
    case 2: return (size_t)below((uint64_t)1 << 30);
    default: return (size_t)rnd();
    }
}

/* Fabricated device addresses: mostly near a few bases, at every small
 * offset, so that ranges meet, overlap and miss each other; sometimes null,
 * tiny, near the top of the address space or random. */
static uintptr_t pick_ptr(void)
{
    static const uintptr_t base[] = {(uintptr_t)1 << 40, ((uintptr_t)1 << 40) + 4096,
                                     ((uintptr_t)1 << 40) + ((uintptr_t)1 << 30),
                                     (uintptr_t)1 << 44};
    switch (below(10)) {
    case 0: return 0;
    case 1: return (uintptr_t)below(64);
    case 2: return UINTPTR_MAX - (uintptr_t)below(256);
    case 3: return (uintptr_t)rnd();
    default: return base[below(4)] + (uintptr_t)below(1 << 16) * (below(2) ? 2 : 4) +
                    (uintptr_t)below(3);
    }
}

static int64_t pick_stride(void)
{
    static const int64_t fixed[] = {0, 1, -1, 2, -2, 3, 7, 8, 9, 16, 1024, 16384, -16384,
                                    INT64_MAX, INT64_MIN, INT64_MIN + 1};
    if (below(3)) return fixed[below(sizeof fixed / sizeof fixed[0])];
    return (int64_t)rnd();
}

static const char *const kOps[] = {
    "add_f32", "add_f16", "add_bf16", "saxpy_f32", "relu_f32", "copy_f32", "gather_f32",
    "gather_walk_f32", "add_relu_f32", "saxpy_relu_f32", "bias_relu_f32", "saxpy_f16",
    "saxpy_bf16", "relu_f16", "relu_bf16", "copy2d_f32", "relu_inplace_f32", "scale_f32",
    "scale_f16", "scale_bf16", "add_scalar_f32", "add_scalar_f16", "add_scalar_bf16",
    "sqrt_f32", "sqrt_f16", "sqrt_bf16", "abs_f32", "abs_f16", "abs_bf16",
    "", "add", "ADD_F32", "add_f32 ", "gather_f64", NULL};

static const char *pick_op(void) { return kOps[below(sizeof kOps / sizeof kOps[0])]; }

typedef ew_status_t (*Bin16)(const uint16_t *, const uint16_t *, uint16_t *, size_t, hipStream_t);
typedef ew_status_t (*Un16)(const uint16_t *, uint16_t *, size_t, hipStream_t);
typedef ew_status_t (*Map16)(float, const uint16_t *, uint16_t *, size_t, hipStream_t);
typedef ew_status_t (*Un32)(const float *, float *, size_t, hipStream_t);
typedef ew_status_t (*Map32)(float, const float *, float *, size_t, hipStream_t);

static void stream_calls(void)
{
    const float *a = (const float *)pick_ptr(), *b = (const float *)pick_ptr();
    float *c = (float *)pick_ptr();
    const uint16_t *ha = (const uint16_t *)pick_ptr(), *hb = (const uint16_t *)pick_ptr();
    uint16_t *hc = (uint16_t *)pick_ptr();
    const size_t n = pick_n();
    const float alpha = (float)(int64_t)below(9) - 4.0f;
    static const Bin16 bin16[] = {ew_add_f16, ew_add_bf16};
    static const Un16 un16[] = {ew_relu_f16, ew_relu_bf16, ew_sqrt_f16, ew_sqrt_bf16,
                                ew_abs_f16, ew_abs_bf16};
    static const Map16 map16[] = {ew_saxpy_f16, ew_saxpy_bf16, ew_scale_f16, ew_scale_bf16,
                                  ew_add_scalar_f16, ew_add_scalar_bf16};
    static const Un32 un32[] = {ew_relu_f32, ew_copy_f32, ew_sqrt_f32, ew_abs_f32};
    static const Map32 map32[] = {ew_scale_f32, ew_add_scalar_f32};
    switch (below(10)) {
    case 0: status_ok(ew_add_f32(a, b, c, n, NULL), "add_f32"); break;
    case 1: status_ok(ew_add_relu_f32(a, b, c, n, NULL), "add_relu_f32"); break;
    case 2: status_ok(bin16[below(2)](ha, hb, hc, n, NULL), "add16"); break;
    case 3: status_ok(ew_saxpy_f32(alpha, a, c, n, NULL), "saxpy_f32"); break;
    case 4: status_ok(ew_saxpy_relu_f32(alpha, a, c, n, NULL), "saxpy_relu_f32"); break;
    case 5: status_ok(un16[below(6)](ha, hc, n, NULL), "unary16"); break;
    case 6: status_ok(map16[below(6)](alpha, ha, hc, n, NULL), "map16"); break;
    case 7: status_ok(un32[below(4)](a, c, n, NULL), "unary32"); break;
    case 8: status_ok(map32[below(2)](alpha, a, c, n, NULL), "map32"); break;
    default: status_ok(ew_relu_inplace_f32(c, n, NULL), "relu_inplace_f32"); break;
    }
}

static void strided_calls(void)
{
    const float *in = (const float *)pick_ptr();
    float *out = (float *)pick_ptr();
    switch (below(4)) {
    case 0: status_ok(ew_gather_f32(in, out, pick_n(), (size_t)pick_stride(), NULL), "gather"); break;
    case 1: status_ok(ew_gather_walk_f32(in, out, pick_n(), (size_t)pick_stride(), NULL), "walk"); break;
    case 2:
        status_ok(ew_copy2d_f32(in, pick_stride(), pick_stride(), out, below(2) ? pick_n() : below(300),
                                below(2) ? pick_n() : below(300), NULL), "copy2d");
        break;
    default:
        status_ok(ew_bias_relu_f32(in, (const float *)pick_ptr(), out, below(2) ? pick_n() : below(300),
                                   below(2) ? pick_n() : below(300), NULL), "bias_relu");
        break;
    }
}

static void plan_calls(void)
{
    ew_plan_t p;
    const int cus = below(4) ? 256 : (int)below(2000) - 2;
    const size_t n = pick_n();
    ew_status_t st;
    const int which = (int)below(3);
    if (which == 0) {
        st = ew_make_plan(pick_op(), (const void *)pick_ptr(), (const void *)pick_ptr(),
                          (const void *)pick_ptr(), n, cus, &p);
    } else if (which == 1) {
        st = ew_make_gather_plan((const void *)pick_ptr(), (const void *)pick_ptr(), n,
                                 (size_t)pick_stride(), cus, &p);
    } else {
        const size_t rows = below(2) ? pick_n() : below(300), cols = below(2) ? pick_n() : below(300);
        st = ew_make_copy2d_plan((const void *)pick_ptr(), pick_stride(), pick_stride(),
                                 (const void *)pick_ptr(), rows, cols, cus, &p);
    }
    status_ok(st, "plan");
    if (st != EW_OK) return;
    if (p.path < EW_PATH_STREAM || p.path > EW_PATH_GATHER_TILES) fail("plan path", p.path, which);
    if (which == 0 && p.n > 0) {
        if (p.vec_elems <= 0 || p.head + p.vectors * (size_t)p.vec_elems + p.tail != p.n)
            fail("plan split", (long long)p.n, (long long)p.head);
        if (p.tail >= (size_t)p.vec_elems) fail("plan tail", (long long)p.tail, p.vec_elems);
    }
    if (p.n > 0 && cus > 0 && p.grid < 1) fail("plan grid", p.grid, which);
    if (p.n > 0 && (p.block < 1 || p.block > 1024 || p.unroll < 1))
        fail("plan shape", p.block, p.unroll);
}

static void batch_calls(void)
{
    ew_batch_item_t items[48];
    const size_t count = (size_t)below(49);
    const char *op = pick_op();
    for (size_t i = 0; i < count; ++i) {
        items[i].out = (void *)pick_ptr();
        items[i].in0 = (const void *)pick_ptr();
        items[i].in1 = (const void *)pick_ptr();
        items[i].n = below(3) ? (size_t)below(3000) : pick_n();
    }
    const ew_batch_item_t *it = (count || below(2)) ? items : NULL;
    ew_batch_plan_t plan;
    ew_status_t st = ew_batch_build(op, it, count, NULL, 0, &plan);
    status_ok(st, "batch size query");
    const ew_status_t host = ew_batch(op, 1.5f, it, count, NULL);
    status_ok(host, "batch");
    if (st != EW_OK) {
        if (host == EW_OK || host == EW_ERR_NO_DEVICE) fail("build failed, batch passed", st, host);
        return;
    }
    if (host != EW_OK && host != EW_ERR_NO_DEVICE) fail("build passed, batch failed", st, host);
    if (plan.bytes == 0 || plan.bytes > ((uint64_t)16 << 20)) return;
    uint64_t *image = (uint64_t *)malloc((size_t)plan.bytes);
    if (!image) return;
    if (below(8) == 0) {   /* too small, then misaligned */
        status_ok(ew_batch_build(op, it, count, image, (size_t)plan.bytes - 8, &plan), "small image");
        status_ok(ew_batch_build(op, it, count, (char *)image + 4, (size_t)plan.bytes - 8, &plan),
                  "misaligned image");
        ew_batch_build(op, it, count, NULL, 0, &plan);
    }
    st = ew_batch_build(op, it, count, image, (size_t)plan.bytes, &plan);
    status_ok(st, "batch build");
    if (st == EW_OK) {
        /* records: in0, in1, out, n, first tile (five 8-byte words) */
        uint64_t k = 0, next_tile = 0;
        for (size_t i = 0; i < count; ++i) {
            if (items[i].n == 0) continue;
            const uint64_t *r = image + 5 * k;
            if (r[0] != (uint64_t)(uintptr_t)items[i].in0 || r[2] != (uint64_t)(uintptr_t)items[i].out ||
                r[3] != (uint64_t)items[i].n || r[4] != next_tile)
                fail("table record", (long long)k, (long long)r[4]);
            next_tile = (k + 1 < plan.items) ? image[5 * (k + 1) + 4] : plan.tiles;
            if (next_tile <= r[4]) fail("table tiles", (long long)k, (long long)next_tile);
            const uint32_t *ti = (const uint32_t *)(image + 5 * plan.items);
            for (uint64_t t = r[4]; t < next_tile && t < plan.tiles; ++t)
                if (ti[t] != (uint32_t)k) fail("tile item", (long long)t, (long long)ti[t]);
            ++k;
        }
        if (k != plan.items) fail("table items", (long long)k, (long long)plan.items);
        /* a consistent plan runs as far as the device check */
        status_ok(ew_batch_run(&plan, 1.0f, (const void *)((uintptr_t)1 << 40), NULL), "run");
        status_ok(ew_batch_run_static(&plan, 1.0f, image, NULL), "run static");
    }
    free(image);
    /* plans that were not built */
    ew_batch_plan_t bad = plan;
    switch (below(6)) {
    case 0: bad.block = (int32_t)below(2048) - 1; break;
    case 1: bad.unroll = (int32_t)below(16) - 1; break;
    case 2: bad.items = rnd(); break;
    case 3: bad.tiles = rnd(); break;
    case 4: bad.bytes = rnd(); break;
    default: bad.op = (int32_t)below(80) - 10; break;
    }
    status_ok(ew_batch_run(&bad, 1.0f, (const void *)((uintptr_t)1 << 40 | below(9)), NULL), "bad run");
    status_ok(ew_batch_run_static(&bad, 1.0f, below(2) ? NULL : &bad, NULL), "bad run static");
    status_ok(ew_batch_run(NULL, 1.0f, NULL, NULL), "null plan");
}

static void row_calls(void)
{
    static const int blocks[] = {-64, 0, 1, 63, 64, 65, 128, 256, 320, 512, 1024, 1088, 2048};
    const char *op = pick_op();
    const int block = blocks[below(sizeof blocks / sizeof blocks[0])];
    const int bpc = (int)below(2100) - 2, unroll = (int)below(12) - 1;
    int b = 0, k = 0, u = 0, g = 0;
    switch (below(4)) {
    case 0: status_ok(ew_set_launch_row(op, pick_n(), block, bpc, unroll), "set row"); break;
    case 1: status_ok(ew_get_launch_row(op, pick_n(), &b, &k, &u), "get row"); break;
    case 2: status_ok(ew_set_launch_config(op, block, bpc, unroll), "set config"); break;
    default: status_ok(ew_get_launch_config(op, pick_n(), &b, &g, &u), "get config"); break;
    }
    if (below(50) == 0) ew_reset_launch_config();
}

static void table_file_calls(const char *path)
{
    static const char *const words[] = {"add_f32", "gather_f32", "relu_f16", "bogus", "#", "0",
                                        "1024", "256", "-1", "4294967296", "18446744073709551616",
                                        "1e3", "0x10", "\t", "  ", "8", "2", "65536", "# note"};
    FILE *f = fopen(path, "w");
    if (!f) return;
    const int lines = (int)below(12);
    for (int i = 0; i < lines; ++i) {
        const int w = (int)below(7);
        for (int j = 0; j < w; ++j)
            fprintf(f, "%s%s", words[below(sizeof words / sizeof words[0])], below(5) ? " " : "");
        if (below(10)) fputc('\n', f);
    }
    if (below(10) == 0) {
        for (int i = 0; i < 3000; ++i) fputc('a' + (int)below(26), f);   /* one very long line */
    }
    fclose(f);
    status_ok(ew_load_launch_table(path), "load table");
    ew_reset_launch_config();
}

int main(int argc, char **argv)
{
    if (argc != 4) {
        fprintf(stderr, "usage: %s ITERATIONS SEED SCRATCH_FILE\n", argv[0]);
        return 2;
    }
    int b = 0, g = 0, u = 0;
    if (ew_get_launch_config("add_f32", 1 << 20, &b, &g, &u) != EW_ERR_NO_DEVICE) {
        fprintf(stderr, "a GPU is visible: the fuzz passes fabricated addresses, not run\n");
        return 77;
    }
    const long iterations = atol(argv[1]);
    g_state = (uint64_t)strtoull(argv[2], NULL, 10);
    for (long i = 0; i < iterations; ++i) {
        switch (below(16)) {
        case 0: case 1: case 2: case 3: stream_calls(); break;
        case 4: case 5: strided_calls(); break;
        case 6: case 7: case 8: plan_calls(); break;
        case 9: case 10: case 11: batch_calls(); break;
        case 12: case 13: row_calls(); break;
        case 14:
            if (below(20) == 0) table_file_calls(argv[3]);
            break;
        default:   /* any int, defined or not, has a string */
            if (!ew_status_string((ew_status_t)((int)below(20) - 10)) ||
                !ew_status_string((ew_status_t)(int)(uint32_t)rnd()))
                fail("null status string", 0, 0);
            break;
        }
    }
    ew_reset_launch_config();
    printf("ew_fuzz: %ld iterations, %d failures; statuses OK %ld, INVALID_ARG %ld, "
           "MISALIGNED %ld, OVERLAP %ld, NO_DEVICE %ld, HIP %ld, TOO_LARGE %ld\n",
           iterations, g_failures, g_status_count[0], g_status_count[1], g_status_count[2],
           g_status_count[3], g_status_count[4], g_status_count[5], g_status_count[6]);
    return g_failures ? 1 : 0;
}
