// pe_plan.cpp -- launch plan of pe_forward (see pe_plan.h). Host-only: no HIP header, no device
// call, so it builds with g++ and runs under -fsanitize=address,undefined in the CPU tests.
#include "pe_plan.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "pe.h"

namespace pe {

namespace {

constexpr int kC = 3, kTp = 2;

int fail(std::string &err, int code, const char *fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(std::string &err, int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return code;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// columns of the packed weight: E rounded up to the matrix-core block (32 for bf16, 16 for fp32)
int64_t packed_cols(int E, int esz) {
    const int nb = esz == 2 ? 32 : 16;
    return cdiv(E, nb) * nb;
}

void set_tiles(Launch &L, const TileShape &t, int E) {
    L.tile = t;
    L.a.tiles = t.id;
    L.a.tiles_m = (int32_t)cdiv(L.a.n_rows, t.bm);
    L.a.tiles_n = (int32_t)cdiv(E, t.bn);
    L.workgroups = (int64_t)L.a.tiles_m * L.a.tiles_n;
}

}  // namespace

const char *kernel_name(int tile_id) {
    switch (tile_id) {
        case kTileLarge256:
        case kTileLarge128: return "pe_fwd32_kernel";
        case kTileSplitK: return "pe_fwd32_sk_kernel";
        case kTileF32: return "pe_fwd16_kernel";
        default: return "";
    }
}

// Tile choice. A launch runs in rounds of at most one workgroup per CU. The cost of a round was
// measured per bf16 tile shape (P = 14, 1k to 332k patches): 256 x 256 tiles ~30 us, 256 x 128
// ~18 us, split-k 32 x 160 ~8 us. The shape with the fewest (rounds x round cost) wins; ties go
// to the larger tile (better per area when the chip is full). An fp32 weight uses the 16x16
// kernel's small tiles: 32 x 160 where E allows (1024 x 1280 makes 256 of them, one round),
// else 32 x 128.
TileShape choose_tiles(int64_t n_rows, int E, int weight_esz, int num_cus) {
    const int skn = E % 160 == 0 ? 160 : 128;
    if (weight_esz == 4) return TileShape{kTileF32, 32, skn};
    const int64_t ncu = num_cus > 0 ? num_cus : 256;
    auto rounds = [&](int64_t tiles) { return cdiv(tiles, ncu); };
    const int64_t rt = cdiv(n_rows, 256);
    const int64_t c256 = rounds(rt * cdiv(E, 256)) * 30;
    const int64_t c128 = rounds(rt * cdiv(E, 128)) * 18;
    const int64_t csk = rounds(cdiv(n_rows, 32) * cdiv(E, skn)) * 8;
    if (c256 <= c128 && c256 <= csk) return TileShape{kTileLarge256, 256, 256};
    if (c128 <= csk) return TileShape{kTileLarge128, 256, 128};
    return TileShape{kTileSplitK, 32, skn};
}

int plan_forward(const PlanRequest &r, std::vector<Launch> &out, std::string &err) {
    out.clear();
    if (r.n_items < 0) return fail(err, PE_ERR_INVALID_ARG, "n_items must be >= 0 (got %d)", r.n_items);
    if (r.n_items == 0) return fail(err, PE_ERR_SHAPE, "no items: N = 0");
    if (!r.grid_thw) return fail(err, PE_ERR_INVALID_ARG, "grid_thw is NULL");
    if (r.input_kind != PE_INPUT_PATCHES && r.input_kind != PE_INPUT_FRAMES)
        return fail(err, PE_ERR_INVALID_ARG, "bad input_kind %d", r.input_kind);
    const int P = r.P, E = r.E, m = r.m, ies = r.in_esz;
    const int64_t K = (int64_t)kC * kTp * P * P;
    const bool frames_in = r.input_kind == PE_INPUT_FRAMES;
    const bool merge = frames_in && r.merge;
    const int32_t *g = r.grid_thw;
    const int n = r.n_items;

    // ---- validate every item before planning any launch
    std::vector<int32_t> F(n, 0);
    std::vector<int64_t> row0(n + 1), elems(n, 0);
    int64_t N = 0;
    for (int i = 0; i < n; ++i) {
        const int32_t t = g[3 * i], hh = g[3 * i + 1], ww = g[3 * i + 2];
        if (t <= 0 || hh <= 0 || ww <= 0)
            return fail(err, PE_ERR_SHAPE, "item %d: grid (%d, %d, %d) has a non-positive entry", i, t, hh, ww);
        // an item's rows, like N, stay below 2^31; checked before the products below can overflow
        if ((int64_t)t * hh >= ((int64_t)1 << 31) || (int64_t)t * hh * ww >= ((int64_t)1 << 31))
            return fail(err, PE_ERR_SHAPE, "item %d: grid (%d, %d, %d) makes 2^31 rows or more", i, t, hh, ww);
        if (frames_in) {
            const int64_t f = r.frames ? (int64_t)r.frames[i] : (t == 1 ? 1 : (int64_t)kTp * t);
            if (f <= 0 || (f + kTp - 1) / kTp != t)
                return fail(err, PE_ERR_SHAPE, "item %d: %lld frames do not make t = %d temporal patches", i,
                            (long long)f, t);
            if (merge && (hh % m || ww % m))
                return fail(err, PE_ERR_SHAPE, "item %d: grid %d x %d not divisible by merge size %d", i, hh, ww, m);
            elems[i] = f * kC * hh * P * (int64_t)ww * P;  // f <= 2t and t*hh*ww < 2^31: no overflow
            if ((uint64_t)elems[i] * ies > kMaxLaunchBytes)
                return fail(err, PE_ERR_UNSUPPORTED, "item %d: %lld bytes of frames exceed the 4 GiB launch range",
                            i, (long long)(elems[i] * ies));
            F[i] = (int32_t)f;  // < 2^31 after the byte check
        }
        row0[i] = N;
        N += (int64_t)t * hh * ww;
    }
    row0[n] = N;
    if (N >= ((int64_t)1 << 31)) return fail(err, PE_ERR_SHAPE, "N = %lld rows: must be < 2^31", (long long)N);

    Launch base;
    memset(&base, 0, sizeof base);
    base.a.E = E;
    base.a.m = m;
    base.a.order = merge ? 1 : 0;

    if (!frames_in) {
        // patch rows: launches of at most kMaxLaunchBytes of input, split at any row
        const int64_t rows_per = (int64_t)(kMaxLaunchBytes / (uint64_t)(K * ies));
        for (int64_t r0 = 0; r0 < N; r0 += rows_per) {
            const int64_t nr = (N - r0 < rows_per) ? N - r0 : rows_per;
            Launch L = base;
            L.a.kind = 0;
            L.weight_map = r.weight_esz == 2 ? kWeightRows : kWeightFrames;  // fp32: one map for both inputs
            L.a.plane = (uint32_t)(kTp * P * P);  // a row is [C][Tp][P][P]
            L.a.rstr = (uint32_t)P;
            L.in_off = (uint64_t)r0 * K * ies;
            L.a.in_bytes = (uint32_t)(nr * K * ies);
            L.row0 = r0;
            L.a.n_rows = (int32_t)nr;
            L.a.n_items = 0;
            L.a.colmajor = (uint64_t)nr * K * ies < (uint64_t)packed_cols(E, ies) * K * ies;
            set_tiles(L, choose_tiles(nr, E, r.weight_esz, r.num_cus), E);
            out.push_back(L);
        }
        return PE_OK;
    }

    // frames: launches of at most kMaxItems consecutive items (any number when they are all alike)
    // and at most kMaxLaunchBytes of input. A launch whose items are all single images loads an
    // image's shared temporal slots once; images mixed with videos run in the videos' launch (both
    // temporal slots read the image's one frame, which is exact), since a launch per run of images
    // or videos costs a launch and a partly idle last round each. With image_fold, single images
    // are kept apart: only their launches use the folded weight. Items of different frame sizes
    // share a launch (the kernels then take each item's strides per lane instead of one scalar
    // stride).
    const bool split_images = r.image_fold != 0;
    int64_t x0 = 0;  // element offset of item i0
    int i0 = 0;
    while (i0 < n) {
        int i1 = i0;
        int64_t span = 0;
        bool mixed = false, all_images = true, same = true;
        auto same_as_first = [&](int i) {
            return F[i] == F[i0] && g[3 * i] == g[3 * i0] && g[3 * i + 1] == g[3 * i0 + 1] && g[3 * i + 2] == g[3 * i0 + 2];
        };
        while (i1 < n && (!split_images || (F[i1] == 1) == (F[i0] == 1)) &&
               (uint64_t)(span + elems[i1]) * ies <= kMaxLaunchBytes) {
            const bool still_same = same && same_as_first(i1);
            // the item table holds kMaxItems entries; launches of identical items never read it
            // past the first (a row's item is a division), so they may hold more
            if (i1 - i0 >= kMaxItems && !still_same) break;
            span += elems[i1];
            mixed = mixed || g[3 * i1 + 1] != g[3 * i0 + 1] || g[3 * i1 + 2] != g[3 * i0 + 2];
            all_images = all_images && F[i1] == 1;
            same = still_same;
            ++i1;
        }
        Launch L = base;
        L.a.kind = 1;
        L.a.img = all_images ? 1 : 0;
        L.a.fold = L.a.img && r.image_fold ? 1 : 0;
        L.weight_map = L.a.fold ? kWeightFold : kWeightFrames;
        L.a.mixg = mixed ? 1 : 0;
        L.a.rstr = (uint32_t)g[3 * i0 + 2] * (uint32_t)P;
        L.a.plane = (uint32_t)g[3 * i0 + 1] * (uint32_t)P * L.a.rstr;
        L.in_off = (uint64_t)x0 * ies;
        L.a.in_bytes = (uint32_t)(span * ies);
        L.row0 = row0[i0];
        L.a.n_rows = (int32_t)(row0[i1] - row0[i0]);
        L.a.n_items = i1 - i0;
        L.a.colmajor = (uint64_t)span * ies < (uint64_t)packed_cols(E, ies) * K * ies;
        L.a.uni = same ? 1 : 0;
        L.a.u_rows = (int32_t)(row0[i0 + 1] - row0[i0]);
        L.a.u_elems = (uint32_t)elems[i0];
        int64_t off = 0;
        for (int i = i0; i < i1 && i - i0 < kMaxItems; ++i) {
            Item &it = L.a.items[i - i0];
            it.row0 = (int32_t)(row0[i] - row0[i0]);
            it.t = g[3 * i];
            it.h = g[3 * i + 1];
            it.w = g[3 * i + 2];
            it.F = F[i];
            it.x_off = (uint32_t)off;
            off += elems[i];
        }
        set_tiles(L, choose_tiles(L.a.n_rows, E, r.weight_esz, r.num_cus), E);
        // opt-in: single images of one frame size with bf16 input and weight, P = 14, on the large
        // tiles: the kernel stages the tile's pixel rows through LDS and reads the weight in the
        // grouped order
        L.a.staged = (r.stage_images && L.a.img && !L.a.fold && !L.a.mixg && P == 14 && r.weight_esz == 2 &&
                      ies == 2 && (L.tile.id == kTileLarge256 || L.tile.id == kTileLarge128)) ? 1 : 0;
        if (L.a.staged) L.weight_map = kWeightGrouped;
        out.push_back(L);
        x0 += span;
        i0 = i1;
    }
    return PE_OK;
}

}  // namespace pe
