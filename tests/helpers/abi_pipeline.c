/* The routing path run from C through the library's C ABI alone: device
 * memory, copies and one stream from the HIP runtime, then tk_route, tk_map,
 * tk_expand_quant (1x128 FP8 E4M3) and tk_reduce (or tk_reduce_dense), each
 * feeding the next on the device.  No Python and no torch: the GPU test
 * writes seeded inputs as raw little-endian files, runs this program and
 * compares what it writes with the oracle.
 *
 * usage: abi_pipeline DIR T E k H score n_groups topk_groups group_topn
 *                     route_scale local_begin local_end has_bias dense
 * reads  DIR/logits  fp32 (T, E)
 *        DIR/bias    fp32 (E), when has_bias is 1
 *        DIR/x       bf16 (T, H)
 *        DIR/y       bf16 (T*k, H): expert outputs, one row per possible route
 * writes DIR/idx, DIR/w (T, k); DIR/counts (n_local); DIR/offsets (n_local+1);
 *        DIR/pos (T, k); DIR/row_src (T*k); DIR/xq (T*k, H) E4M3;
 *        DIR/scales fp32 (T*k, H/128); DIR/out bf16 (T, H)
 * Rows past the routed count (offsets[n_local]) are left as the device
 * allocation held them.  Exit status: 0 done; 1 usage or file error; 2 a
 * library or HIP call failed (its message on stderr). */
#include "tk.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static char g_dir[4096];

static int io_file(const char* name, void* data, size_t bytes, int write)
{
    char path[4200];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE* f = fopen(path, write ? "wb" : "rb");
    if (f == NULL) {
        fprintf(stderr, "abi_pipeline: cannot open %s\n", path);
        return 1;
    }
    const size_t n = write ? fwrite(data, 1, bytes, f) : fread(data, 1, bytes, f);
    fclose(f);
    if (n != bytes) {
        fprintf(stderr, "abi_pipeline: %s: %zu of %zu bytes\n", path, n, bytes);
        return 1;
    }
    return 0;
}

#define HIP_OK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "abi_pipeline: %s: %s\n", #call, hipGetErrorString(e_));     \
            return 2;                                                                    \
        }                                                                                \
    } while (0)

#define TK_OK_(call)                                                                     \
    do {                                                                                 \
        tk_status s_ = (call);                                                           \
        if (s_ != TK_OK) {                                                               \
            fprintf(stderr, "abi_pipeline: %s -> %d: %s\n", #call, (int)s_,              \
                    tk_last_error());                                                    \
            return 2;                                                                    \
        }                                                                                \
    } while (0)

/* one host buffer and its device copy */
typedef struct {
    void* h;
    void* d;
    size_t bytes;
} buf;

static int buf_alloc(buf* b, size_t bytes)
{
    b->bytes = bytes;
    b->h = malloc(bytes > 0 ? bytes : 1);
    b->d = NULL;
    if (b->h == NULL) return 1;
    return hipMalloc(&b->d, bytes > 0 ? bytes : 16) == hipSuccess ? 0 : 2;
}

static int run(int argc, char** argv)
{
    if (argc != 15) {
        fprintf(stderr, "usage: abi_pipeline DIR T E k H score n_groups topk_groups group_topn "
                        "route_scale local_begin local_end has_bias dense\n");
        return 1;
    }
    snprintf(g_dir, sizeof g_dir, "%s", argv[1]);
    const int32_t T = atoi(argv[2]), E = atoi(argv[3]), k = atoi(argv[4]), H = atoi(argv[5]);
    tk_route_opts opts;
    opts.score = atoi(argv[6]);
    opts.n_groups = atoi(argv[7]);
    opts.topk_groups = atoi(argv[8]);
    opts.group_topn = atoi(argv[9]);
    opts.renormalize = 1;
    opts.route_scale = (float)atof(argv[10]);
    const int32_t lo = atoi(argv[11]), hi = atoi(argv[12]);
    const int has_bias = atoi(argv[13]), dense = atoi(argv[14]);
    if (T < 1 || E < 1 || k < 1 || H < 128 || H % 128 != 0 || lo < 0 || hi > E || lo >= hi) {
        fprintf(stderr, "abi_pipeline: bad sizes\n");
        return 1;
    }
    const int32_t n_local = hi - lo;
    const size_t routes = (size_t)T * (size_t)k, cap = routes;

    buf logits, bias, x, y, idx, w, counts, offsets, pos, row_src, xq, scales, out, ws;
    int rc = 0;
    rc |= buf_alloc(&logits, (size_t)T * E * 4);
    rc |= buf_alloc(&bias, has_bias ? (size_t)E * 4 : 0);
    rc |= buf_alloc(&x, (size_t)T * H * 2);
    rc |= buf_alloc(&y, cap * H * 2);
    rc |= buf_alloc(&idx, routes * 4);
    rc |= buf_alloc(&w, routes * 4);
    rc |= buf_alloc(&counts, (size_t)n_local * 4);
    rc |= buf_alloc(&offsets, ((size_t)n_local + 1) * 4);
    rc |= buf_alloc(&pos, routes * 4);
    rc |= buf_alloc(&row_src, cap * 4);
    rc |= buf_alloc(&xq, cap * H);
    rc |= buf_alloc(&scales, cap * (H / 128) * 4);
    rc |= buf_alloc(&out, (size_t)T * H * 2);
    rc |= buf_alloc(&ws, tk_map_workspace_bytes(T, k, n_local));
    if (rc != 0) {
        fprintf(stderr, "abi_pipeline: allocation failed\n");
        return 2;
    }

    if (io_file("logits", logits.h, logits.bytes, 0) || io_file("x", x.h, x.bytes, 0) ||
        io_file("y", y.h, y.bytes, 0) || (has_bias && io_file("bias", bias.h, bias.bytes, 0)))
        return 1;
    HIP_OK(hipMemcpy(logits.d, logits.h, logits.bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(x.d, x.h, x.bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(y.d, y.h, y.bytes, hipMemcpyHostToDevice));
    if (has_bias) HIP_OK(hipMemcpy(bias.d, bias.h, bias.bytes, hipMemcpyHostToDevice));

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    TK_OK_(tk_route((const float*)logits.d, has_bias ? (const float*)bias.d : NULL, T, E, k,
                    &opts, (int32_t*)idx.d, (float*)w.d, s));
    TK_OK_(tk_map((const int32_t*)idx.d, T, k, E, lo, hi, (int32_t*)counts.d,
                  (int32_t*)offsets.d, (int32_t*)pos.d, (int32_t*)row_src.d, ws.d, ws.bytes, s));
    TK_OK_(tk_expand_quant(x.d, T, H, k, (const int32_t*)pos.d, TK_EXPAND_FP8_E4M3_1X128, xq.d,
                           (float*)scales.d, (int64_t)cap, s));
    if (dense)
        TK_OK_(tk_reduce_dense(y.d, (int64_t)cap, (const int32_t*)pos.d, (const float*)w.d, T, k,
                               H, out.d, s));
    else
        TK_OK_(tk_reduce(y.d, (int64_t)cap, (const int32_t*)pos.d, (const float*)w.d, T, k, H,
                         out.d, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipStreamDestroy(s));

    buf* outs[] = {&idx, &w, &counts, &offsets, &pos, &row_src, &xq, &scales, &out};
    const char* names[] = {"idx", "w", "counts", "offsets", "pos", "row_src", "xq", "scales", "out"};
    for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
        HIP_OK(hipMemcpy(outs[i]->h, outs[i]->d, outs[i]->bytes, hipMemcpyDeviceToHost));
        if (io_file(names[i], outs[i]->h, outs[i]->bytes, 1)) return 1;
    }
    buf* all[] = {&logits, &bias, &x, &y, &idx, &w, &counts, &offsets, &pos, &row_src, &xq,
                  &scales, &out, &ws};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) {
        HIP_OK(hipFree(all[i]->d));
        free(all[i]->h);
    }
    return 0;
}

int main(int argc, char** argv)
{
    const int rc = run(argc, argv);
    if (rc == 0) printf("abi_pipeline: done\n");
    return rc;
}
