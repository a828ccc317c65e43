/*
 * pe_client.c -- a C caller of libpe.so through include/pe.h only (no Python, no torch): reads
 * bf16 frames, weight and bias from files, runs pe_create / pe_forward / pe_layernorm /
 * pe_destroy on the current HIP device and writes the outputs to files. The test that builds
 * and runs it compares the outputs with the oracle.
 *
 * usage: pe_client <dir>   (dir holds frames.bin, weight.bin, bias.bin, gamma.bin, beta.bin as
 *                           raw bf16, and meta.txt: P E t h w F; writes out.bin and ln.bin)
 *        pe_client <dir> rows   (dir holds rows.bin: N pre-flattened patch rows [N, K] in
 *                           in_dtype, weight.bin, bias.bin, and rows_meta.txt: P E N in_dtype;
 *                           the rows go to a device buffer of exactly N*K elements, so the
 *                           last row ends at the end of the allocation; writes rows_out.bin)
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pe.h"

static void *read_file(const char *dir, const char *name, size_t *bytes) {
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    fseek(f, 0, SEEK_END);
    *bytes = (size_t)ftell(f);
    fseek(f, 0, SEEK_SET);
    void *p = malloc(*bytes);
    if (!p || fread(p, 1, *bytes, f) != *bytes) { fprintf(stderr, "cannot read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t bytes) {
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

static void *to_device(const void *h, size_t bytes) {
    void *d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "device copy failed\n");
        exit(3);
    }
    return d;
}

#define CHECK(call)                                                                   \
    do {                                                                              \
        int rc_ = (call);                                                             \
        if (rc_ != PE_OK) {                                                           \
            fprintf(stderr, "%s -> %d: %s\n", #call, rc_, pe_last_error());           \
            return 4;                                                                 \
        }                                                                             \
    } while (0)

static int run_rows(const char *dir) {
    char path[1024];
    snprintf(path, sizeof path, "%s/rows_meta.txt", dir);
    FILE *m = fopen(path, "r");
    int P, E, N, in_dtype;
    if (!m || fscanf(m, "%d %d %d %d", &P, &E, &N, &in_dtype) != 4) { fprintf(stderr, "bad rows meta\n"); return 1; }
    fclose(m);
    size_t nx, nw, nb;
    void *x = read_file(dir, "rows.bin", &nx), *wt = read_file(dir, "weight.bin", &nw);
    void *b = read_file(dir, "bias.bin", &nb);
    const size_t K = (size_t)3 * 2 * P * P, isz = in_dtype == PE_BF16 ? 2 : 4;
    if (nx != (size_t)N * K * isz) { fprintf(stderr, "rows.bin holds %zu bytes, not N*K*%zu\n", nx, isz); return 1; }
    void *dx = to_device(x, nx), *dw = to_device(wt, nw), *db = to_device(b, nb);   /* exactly N*K elements */
    pe_config cfg = {3, 2, P, E, 2, PE_BF16, PE_BF16, PE_ORDER_RASTER, 0, 0};
    pe_handle hd = NULL;
    CHECK(pe_create(&cfg, dw, db, NULL, &hd));
    const int32_t grid[3] = {1, 1, N};
    const size_t out_bytes = (size_t)N * (size_t)E * 2;
    void *dout = NULL;
    if (hipMalloc(&dout, out_bytes) != hipSuccess) return 3;
    CHECK(pe_forward(hd, PE_INPUT_PATCHES, dx, in_dtype, grid, NULL, 1, dout, NULL));
    if (hipDeviceSynchronize() != hipSuccess) return 3;
    void *out = malloc(out_bytes);
    if (hipMemcpy(out, dout, out_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 3;
    write_file(dir, "rows_out.bin", out, out_bytes);
    CHECK(pe_destroy(hd));
    hipFree(dx); hipFree(dw); hipFree(db); hipFree(dout);
    free(x); free(wt); free(b); free(out);
    printf("pe_client: %d patch rows x %d written\n", N, E);
    return 0;
}

int main(int argc, char **argv) {
    if (argc == 3 && strcmp(argv[2], "rows") == 0) return run_rows(argv[1]);
    if (argc != 2) { fprintf(stderr, "usage: %s <dir> [rows]\n", argv[0]); return 1; }
    const char *dir = argv[1];
    char path[1024];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE *m = fopen(path, "r");
    int P, E, t, h, w, F;
    if (!m || fscanf(m, "%d %d %d %d %d %d", &P, &E, &t, &h, &w, &F) != 6) { fprintf(stderr, "bad meta\n"); return 1; }
    fclose(m);

    size_t nx, nw, nb, ng, nbe;
    void *x = read_file(dir, "frames.bin", &nx), *wt = read_file(dir, "weight.bin", &nw);
    void *b = read_file(dir, "bias.bin", &nb), *g = read_file(dir, "gamma.bin", &ng);
    void *be = read_file(dir, "beta.bin", &nbe);
    void *dx = to_device(x, nx), *dw = to_device(wt, nw), *db = to_device(b, nb);
    void *dg = to_device(g, ng), *dbe = to_device(be, nbe);

    pe_config cfg = {3, 2, P, E, 2, PE_BF16, PE_BF16, PE_ORDER_MERGE_WINDOW, 0, 0};
    pe_handle hd = NULL;
    CHECK(pe_create(&cfg, dw, db, NULL, &hd));
    const int32_t grid[3] = {t, h, w};
    const int32_t frames[1] = {F};
    const int64_t n = pe_num_rows(grid, 1);
    if (n <= 0) { fprintf(stderr, "bad grid\n"); return 1; }
    const size_t out_bytes = (size_t)n * (size_t)E * 2;
    void *dout = NULL, *dln = NULL;
    if (hipMalloc(&dout, out_bytes) != hipSuccess || hipMalloc(&dln, out_bytes) != hipSuccess) return 3;
    CHECK(pe_forward(hd, PE_INPUT_FRAMES, dx, PE_BF16, grid, frames, 1, dout, NULL));
    CHECK(pe_layernorm(dout, PE_BF16, dg, dbe, PE_BF16, 1e-6f, n, E, dln, NULL));
    if (hipDeviceSynchronize() != hipSuccess) return 3;
    void *out = malloc(out_bytes), *ln = malloc(out_bytes);
    if (hipMemcpy(out, dout, out_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(ln, dln, out_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 3;
    write_file(dir, "out.bin", out, out_bytes);
    write_file(dir, "ln.bin", ln, out_bytes);
    CHECK(pe_destroy(hd));
    hipFree(dx); hipFree(dw); hipFree(db); hipFree(dg); hipFree(dbe); hipFree(dout); hipFree(dln);
    free(x); free(wt); free(b); free(g); free(be); free(out); free(ln);
    printf("pe_client: %lld rows x %d written\n", (long long)n, E);
    return 0;
}
