// Host driver of the library's launch planner (vlm_vision_patch_amd/csrc/pe_plan.cpp), built with
// g++ and -fsanitize=address,undefined by tests/test_plan.py. No GPU, no HIP header.
//
// stdin: one request per line
//   P E m weight_esz in_esz out_esz merge fold stage num_cus input_kind n_items has_frames  t h w [F] ...
// stdout, per request:
//   R <status> <launches>
//   L row0 n_rows in_off in_bytes n_items tile_id bm bn workgroups tiles_m tiles_n img fold mixg uni
//     colmajor weight_map u_rows u_elems plane rstr kind order staged
//   I row0 t h w F x_off          (the launch's item table, first min(n_items, 64) entries)
#include <stdio.h>

#include <string>
#include <vector>

#include "pe_plan.h"

int main() {
    int P, E, m, wesz, iesz, oesz, merge, fold, stage, ncu, kind, n, hasf;
    while (scanf("%d %d %d %d %d %d %d %d %d %d %d %d %d", &P, &E, &m, &wesz, &iesz, &oesz, &merge, &fold, &stage,
                 &ncu, &kind, &n, &hasf) == 13) {
        // exact-size host arrays, so that any read past the item count is an ASan error
        std::vector<int32_t> g(3 * (size_t)(n > 0 ? n : 0)), f(hasf && n > 0 ? (size_t)n : 0);
        for (int i = 0; i < n; ++i) {
            if (scanf("%d %d %d", &g[3 * i], &g[3 * i + 1], &g[3 * i + 2]) != 3) return 2;
            if (hasf && scanf("%d", &f[i]) != 1) return 2;
        }
        pe::PlanRequest r;
        r.P = P; r.E = E; r.m = m;
        r.weight_esz = wesz; r.in_esz = iesz; r.out_esz = oesz;
        r.merge = merge; r.image_fold = fold; r.stage_images = stage; r.num_cus = ncu; r.input_kind = kind;
        r.grid_thw = n > 0 ? g.data() : nullptr;
        r.frames = hasf && n > 0 ? f.data() : nullptr;
        r.n_items = n;
        std::vector<pe::Launch> plan;
        std::string err;
        const int rc = pe::plan_forward(r, plan, err);
        printf("R %d %zu\n", rc, plan.size());
        for (const pe::Launch &L : plan) {
            const pe::FwdArgs &a = L.a;
            printf("L %lld %d %llu %u %d %d %d %d %lld %d %d %d %d %d %d %d %d %d %u %u %u %d %d %d\n", (long long)L.row0,
                   a.n_rows, (unsigned long long)L.in_off, a.in_bytes, a.n_items, L.tile.id, L.tile.bm, L.tile.bn,
                   (long long)L.workgroups, a.tiles_m, a.tiles_n, a.img, a.fold, a.mixg, a.uni, a.colmajor,
                   L.weight_map, a.u_rows, a.u_elems, a.plane, a.rstr, a.kind, a.order, a.staged);
            for (int i = 0; i < a.n_items && i < pe::kMaxItems; ++i) {
                const pe::Item &it = a.items[i];
                printf("I %d %d %d %d %d %u\n", it.row0, it.t, it.h, it.w, it.F, it.x_off);
            }
        }
    }
    return 0;
}
