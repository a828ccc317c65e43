/*
 * pe_oracle.c -- the oracle for the vision PatchEmbed.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load, link or call this file:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it. It shares
 * no code, header, table or constant with the HIP library.
 *
 * What it computes (plain definition, fp64, no blocking, no reordering of any sum):
 *
 *   The PatchEmbed of Qwen2/2.5/3-VL is a Conv3d with C input channels, E output channels and
 *   kernel = stride = (Tp, P, P), no padding, dilation 1 ("Qwen2.5VL-Vision Encode-PatchEmbed",
 *   the bullet list on the convolution; "Optimize VLM PatchEmbed", the Qwen3VLVisionPatchEmbed
 *   class; "patch详解" section 4.3, the PatchEmbed class).  For each item (an image or a video)
 *   with patch grid (t, h, w) and F frames of size [C, h*P, w*P], the oracle
 *
 *     1. forms the temporally completed volume V[c][tau][y][x] for tau < t*Tp, taking frame
 *        min(tau, F-1): a single image frame is repeated to fill the temporal pair (the page
 *        "patch详解" section 4.5 rounds 1/2 up to one temporal patch; repeating the frame is
 *        the reading taken for that round-up);
 *     2. evaluates the textbook Conv3d sum at every output position (to, ho, wo):
 *          out[e] = b[e] + sum_c sum_kt sum_ky sum_kx
 *                     W[e][c][kt][ky][kx] * V[c][to*Tp+kt][ho*P+ky][wo*P+kx]
 *        as five nested loops, e outermost, in that order;
 *     3. places the result at the output row given by the row order:
 *          raster:        r = (to*h + ho)*w + wo
 *          merge window:  r = (((to*(h/m) + ho/m)*(w/m) + wo/m)*m + ho%m)*m + wo%m
 *        (windows of m x m neighbouring patches are concatenated by the PatchMerger, page
 *        "freechatgpt/mytransformer" section 3.2; the windows follow the merged grid in raster
 *        order, as the vision-token position ids on the "Qwen2.5VL语言模型" page show), plus
 *        the item's first row (items are concatenated in order).
 *
 *   Pre-flattened patch rows x[N, C*Tp*P*P] (the [N,1176] hidden states of the pages) are the
 *   same convolution on a single patch volume: row n viewed as [C][Tp][P][P]; out row n.
 *
 *   All inputs arrive as fp64 copies of the exact bf16/fp32 values the GPU receives; no
 *   rounding happens here. Output is fp64.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_SHAPE (-2)
#define ORACLE_ERR_OOM (-5)

/* ---- problem ------------------------------------------------------------------------ */

typedef struct {
    int C, Tp, P, E;
    int kind;   /* 0: patch rows, 1: frames */
    int order;  /* 0: raster, 1: merge window */
    int m;      /* merge size */
    int n_items;
    const int32_t *grid;    /* n_items * 3 */
    const int32_t *frames;  /* n_items, frames kind */
    const double *x, *w, *b;
    int64_t *item_row0;     /* n_items + 1 */
    int64_t *item_x0;       /* n_items, element offset of the item's first frame */
} problem;

/* Value of the temporally completed volume of item i at (c, tau, y, x). */
static double volume_at(const problem *pb, int i, int c, int tau, int y, int x) {
    int F = pb->frames[i];
    int H = pb->grid[3 * i + 1] * pb->P;
    int W = pb->grid[3 * i + 2] * pb->P;
    int f = tau < F ? tau : F - 1;
    const double *X = pb->x + pb->item_x0[i];
    return X[(((int64_t)f * pb->C + c) * H + y) * (int64_t)W + x];
}

/* Output row, inside item i, of the patch at (to, ho, wo). */
static int64_t row_in_item(const problem *pb, int i, int to, int ho, int wo) {
    int64_t h = pb->grid[3 * i + 1], w = pb->grid[3 * i + 2];
    if (pb->order == 0) return ((int64_t)to * h + ho) * w + wo;
    int64_t m = pb->m;
    int64_t window = ((int64_t)to * (h / m) + ho / m) * (w / m) + wo / m;
    return (window * m + ho % m) * m + wo % m;
}

/* One output row of a frames item: the direct Conv3d at (to, ho, wo). */
static void conv_frames(const problem *pb, int i, int to, int ho, int wo, double *out) {
    const int C = pb->C, Tp = pb->Tp, P = pb->P;
    const int64_t K = (int64_t)C * Tp * P * P;
    for (int e = 0; e < pb->E; ++e) {
        double acc = 0.0;
        const double *We = pb->w + (int64_t)e * K;
        for (int c = 0; c < C; ++c)
            for (int kt = 0; kt < Tp; ++kt)
                for (int ky = 0; ky < P; ++ky)
                    for (int kx = 0; kx < P; ++kx)
                        acc += We[((c * Tp + kt) * P + ky) * P + kx] *
                               volume_at(pb, i, c, to * Tp + kt, ho * P + ky, wo * P + kx);
        out[e] = (pb->b ? pb->b[e] : 0.0) + acc;
    }
}

/* One output row of patch-row input: row n viewed as a [C][Tp][P][P] volume. */
static void conv_patch_row(const problem *pb, int64_t n, double *out) {
    const int C = pb->C, Tp = pb->Tp, P = pb->P;
    const int64_t K = (int64_t)C * Tp * P * P;
    const double *V = pb->x + n * K;
    for (int e = 0; e < pb->E; ++e) {
        double acc = 0.0;
        const double *We = pb->w + (int64_t)e * K;
        for (int c = 0; c < C; ++c)
            for (int kt = 0; kt < Tp; ++kt)
                for (int ky = 0; ky < P; ++ky)
                    for (int kx = 0; kx < P; ++kx) {
                        int64_t k = ((int64_t)(c * Tp + kt) * P + ky) * P + kx;
                        acc += We[k] * V[k];
                    }
        out[e] = (pb->b ? pb->b[e] : 0.0) + acc;
    }
}

/* ---- row bookkeeping ----------------------------------------------------------------- */

/* For every output row, the position it comes from: item, to, ho, wo. Built by walking every
 * position and applying the forward row formula, so the formula above stays the definition. */
typedef struct { int32_t item, to, ho, wo; } position;

static int validate(problem *pb, int64_t *n_rows_out) {
    if (pb->C <= 0 || pb->Tp <= 0 || pb->P <= 0 || pb->E <= 0 || pb->n_items <= 0) return ORACLE_ERR_ARG;
    if (!pb->grid || !pb->x || !pb->w) return ORACLE_ERR_ARG;
    if (pb->kind == 1 && !pb->frames) return ORACLE_ERR_ARG;
    if (pb->order == 1 && pb->m <= 0) return ORACLE_ERR_ARG;
    int64_t rows = 0, xoff = 0;
    for (int i = 0; i < pb->n_items; ++i) {
        int t = pb->grid[3 * i], h = pb->grid[3 * i + 1], w = pb->grid[3 * i + 2];
        if (t <= 0 || h <= 0 || w <= 0) return ORACLE_ERR_SHAPE;
        if (pb->kind == 1) {
            int F = pb->frames[i];
            if (F <= 0 || (F + pb->Tp - 1) / pb->Tp != t) return ORACLE_ERR_SHAPE;
            if (pb->order == 1 && (h % pb->m || w % pb->m)) return ORACLE_ERR_SHAPE;
            pb->item_x0[i] = xoff;
            xoff += (int64_t)F * pb->C * h * pb->P * (int64_t)w * pb->P;
        }
        pb->item_row0[i] = rows;
        rows += (int64_t)t * h * w;
    }
    pb->item_row0[pb->n_items] = rows;
    *n_rows_out = rows;
    return ORACLE_OK;
}

static void build_positions(const problem *pb, position *pos) {
    for (int i = 0; i < pb->n_items; ++i) {
        int t = pb->grid[3 * i], h = pb->grid[3 * i + 1], w = pb->grid[3 * i + 2];
        for (int to = 0; to < t; ++to)
            for (int ho = 0; ho < h; ++ho)
                for (int wo = 0; wo < w; ++wo) {
                    int64_t r = pb->item_row0[i] + row_in_item(pb, i, to, ho, wo);
                    pos[r].item = i; pos[r].to = to; pos[r].ho = ho; pos[r].wo = wo;
                }
    }
}

/* ---- threads --------------------------------------------------------------------------- */

typedef struct {
    const problem *pb;
    const position *pos;
    const int64_t *rows;
    int64_t n_rows, first, stride;
    double *out;
} job;

static void *worker(void *arg) {
    job *j = (job *)arg;
    for (int64_t q = j->first; q < j->n_rows; q += j->stride) {
        int64_t r = j->rows ? j->rows[q] : q;
        double *o = j->out + q * j->pb->E;
        if (j->pb->kind == 0) conv_patch_row(j->pb, r, o);
        else conv_frames(j->pb, j->pos[r].item, j->pos[r].to, j->pos[r].ho, j->pos[r].wo, o);
    }
    return NULL;
}

/* ---- public entry points ---------------------------------------------------------------- */

/* Number of output rows, sum over items of t*h*w; negative on a bad grid. */
int64_t pe_oracle_num_rows(const int32_t *grid, int n_items) {
    if (!grid || n_items <= 0) return ORACLE_ERR_ARG;
    int64_t n = 0;
    for (int i = 0; i < n_items; ++i) {
        if (grid[3 * i] <= 0 || grid[3 * i + 1] <= 0 || grid[3 * i + 2] <= 0) return ORACLE_ERR_SHAPE;
        n += (int64_t)grid[3 * i] * grid[3 * i + 1] * grid[3 * i + 2];
    }
    return n;
}

/* Row index -> source position (item, to, ho, wo), for all N rows (out: N*4 int32). */
int pe_oracle_row_positions(int kind, int order, int m, int C, int Tp, int P, int n_items,
                            const int32_t *grid, const int32_t *frames, int32_t *out) {
    problem pb;
    memset(&pb, 0, sizeof pb);
    pb.C = C; pb.Tp = Tp; pb.P = P; pb.E = 1; pb.kind = kind; pb.order = order; pb.m = m;
    pb.n_items = n_items; pb.grid = grid; pb.frames = frames;
    double dummy = 0.0;
    pb.x = &dummy; pb.w = &dummy;
    if (n_items <= 0 || !out) return ORACLE_ERR_ARG;
    pb.item_row0 = (int64_t *)malloc(sizeof(int64_t) * (n_items + 1));
    pb.item_x0 = (int64_t *)malloc(sizeof(int64_t) * n_items);
    if (!pb.item_row0 || !pb.item_x0) { free(pb.item_row0); free(pb.item_x0); return ORACLE_ERR_OOM; }
    int64_t n = 0;
    int rc = validate(&pb, &n);
    if (rc == ORACLE_OK) build_positions(&pb, (position *)out);
    free(pb.item_row0); free(pb.item_x0);
    return rc;
}

/*
 * Compute output rows of the PatchEmbed.
 *   kind      0 = patch rows x[N][C*Tp*P*P]; 1 = frames (item i: frames[i] frames of [C][h*P][w*P],
 *             items back to back in x)
 *   order     0 = raster, 1 = merge window of size m (frames kind only; patch rows keep their order)
 *   grid      n_items * (t, h, w); N = sum t*h*w
 *   x, w, b   fp64 inputs; w is [E][C][Tp][P][P]; b is [E] or NULL
 *   rows      the output rows wanted (n_rows of them), or NULL for all N rows in order
 *   out       n_rows * E fp64
 *   n_threads worker threads (>= 1)
 * Returns 0, or a negative code for a bad argument or an inconsistent shape.
 */
int pe_oracle_forward(int C, int Tp, int P, int E, int kind, int order, int m, int n_items,
                      const int32_t *grid, const int32_t *frames, const double *x,
                      const double *w, const double *b, const int64_t *rows, int64_t n_rows,
                      double *out, int n_threads) {
    if (!out || n_threads <= 0 || (kind != 0 && kind != 1) || (order != 0 && order != 1))
        return ORACLE_ERR_ARG;
    problem pb;
    memset(&pb, 0, sizeof pb);
    pb.C = C; pb.Tp = Tp; pb.P = P; pb.E = E; pb.kind = kind; pb.order = kind == 0 ? 0 : order;
    pb.m = m; pb.n_items = n_items; pb.grid = grid; pb.frames = frames; pb.x = x; pb.w = w; pb.b = b;
    if (n_items <= 0) return ORACLE_ERR_ARG;
    pb.item_row0 = (int64_t *)malloc(sizeof(int64_t) * (n_items + 1));
    pb.item_x0 = (int64_t *)malloc(sizeof(int64_t) * n_items);
    position *pos = NULL;
    int rc = ORACLE_OK;
    if (!pb.item_row0 || !pb.item_x0) { rc = ORACLE_ERR_OOM; goto done; }
    int64_t N = 0;
    rc = validate(&pb, &N);
    if (rc != ORACLE_OK) goto done;
    if (!rows) n_rows = N;
    for (int64_t q = 0; rows && q < n_rows; ++q)
        if (rows[q] < 0 || rows[q] >= N) { rc = ORACLE_ERR_ARG; goto done; }
    if (kind == 1) {
        pos = (position *)malloc(sizeof(position) * (size_t)(N > 0 ? N : 1));
        if (!pos) { rc = ORACLE_ERR_OOM; goto done; }
        build_positions(&pb, pos);
    }
    {
        if (n_threads > 256) n_threads = 256;
        pthread_t th[256];
        job jobs[256];
        int started = 0;
        for (int t = 0; t < n_threads; ++t) {
            jobs[t].pb = &pb; jobs[t].pos = pos; jobs[t].rows = rows; jobs[t].n_rows = n_rows;
            jobs[t].first = t; jobs[t].stride = n_threads; jobs[t].out = out;
        }
        for (int t = 1; t < n_threads; ++t)
            if (pthread_create(&th[t], NULL, worker, &jobs[t]) == 0) started = t; else break;
        /* threads that failed to start: run their share here */
        for (int t = started + 1; t < n_threads; ++t) worker(&jobs[t]);
        worker(&jobs[0]);
        for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    }
done:
    free(pos); free(pb.item_row0); free(pb.item_x0);
    return rc;
}
