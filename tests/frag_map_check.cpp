// Host check of the library's fragment map (pe_internal.h): for each supported patch size and
// element size, the (k-step, lane group, element) -> (pixel row, px) map must hit every patch
// element exactly once, keep each load inside its pixel row, and pad only the last fragments.
// Built and run by tests/test_abi.py; prints "OK" on success.
#include <cstdio>
#include <vector>

#include "pe_internal.h"

static int check(int P, int esz) {
    using namespace pe;
    const int rows = kC * kTp * P, epf = frag_elems(esz), first = split_first(P, esz);
    const int S = num_steps(P, esz), SF = full_steps(P, esz);
    std::vector<int> hits(rows * P, 0);
    int pads = 0;
    for (int s = 0; s < S; ++s)
        for (int g = 0; g < 4; ++g) {
            const Piece p = frag_piece(P, esz, s, g);
            if ((s < SF) != (p.kind == kFull)) { printf("kind/step mismatch P%d esz%d s%d\n", P, esz, s); return 1; }
            if (p.kind == kPad) { pads += epf; continue; }
            const int n1 = p.kind == kFull ? epf : first;
            if (p.x1 + n1 > P || p.r1 < 0 || p.r1 >= rows) { printf("piece 1 out of row\n"); return 1; }
            if (p.kind == kSplit && (p.x2 + (epf - first) > P || p.r2 < 0 || p.r2 >= rows)) { printf("piece 2 out of row\n"); return 1; }
            for (int j = 0; j < epf; ++j) {
                const int r = (p.kind == kFull || j < first) ? p.r1 : p.r2;
                const int x = (p.kind == kFull || j < first) ? p.x1 + j : p.x2 + j - first;
                hits[r * P + x]++;
            }
            // byte offsets of both pieces are 4-byte aligned within a row (row starts are)
            if ((p.x1 * esz) % 4 || (p.kind == kSplit && (p.x2 * esz) % 4)) { printf("misaligned piece\n"); return 1; }
        }
    for (int i = 0; i < rows * P; ++i)
        if (hits[i] != 1) { printf("P%d esz%d element %d hit %d times\n", P, esz, i, hits[i]); return 1; }
    if (pads != S * 4 * epf - rows * P) { printf("pad count\n"); return 1; }
    printf("P%d esz%d: %d steps (%d whole-fragment), %d pad elements\n", P, esz, S, SF, pads);
    return 0;
}

int main() {
    int bad = 0;
    for (int P : {14, 16})
        for (int esz : {2, 4}) bad |= check(P, esz);
    if (pe::num_steps(14, 2) != 37 || pe::num_steps(16, 2) != 48) { printf("step counts\n"); bad = 1; }
    if (!bad) printf("OK\n");
    return bad;
}
