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

// The temporal-split map of the bf16 32x32 kernel: fragment (s, g = 2j + tt) covers unique
// fragment uf = 2s + j of temporal slot tt; every element of each slot exactly once.
static int check_tt(int P) {
    using namespace pe;
    const int rows = kC * P, S = tt_steps(P);
    std::vector<int> hits(rows * P, 0);
    int pads = 0;
    for (int uf = 0; uf < 2 * S; ++uf) {
        const UFrag f = tt_frag(P, uf);
        for (int j = 0; j < 8; ++j) {
            int u = f.u1, x = f.x1 + j;
            if (f.kind == kUfSplit62 && j >= 6) { u = f.u2; x = f.x2 + j - 6; }
            if (f.kind == kUfTail4 && j >= 4) { ++pads; continue; }
            if (u < 0 || u >= rows || x < 0 || x >= P) { printf("tt map out of row\n"); return 1; }
            hits[u * P + x]++;
        }
        if ((f.x1 * 2) % 4 || (f.kind == kUfSplit62 && (f.x2 * 2) % 4)) { printf("misaligned\n"); return 1; }
        if (f.kind != kUfFull && f.x1 + (f.kind == kUfSplit62 ? 6 : 4) > P) { printf("piece 1 past row\n"); return 1; }
    }
    for (int i = 0; i < rows * P; ++i)
        if (hits[i] != 1) { printf("tt map P%d element %d hit %d times\n", P, i, hits[i]); return 1; }
    printf("tt map P%d: %d steps, %d pad elements per temporal slot\n", P, S, pads);
    return pads == 2 * S * 8 - rows * P ? 0 : 1;
}

// The patch-rows map: lane group g of k-step s takes elements [32s + 8g, +8) of the stored row,
// so each k-step covers 32 consecutive elements and only the tail past K is padding.
static int check_rows(int P) {
    using namespace pe;
    const int K = kC * kTp * P * P, S = rows_steps(P);
    std::vector<int> hits(K, 0);
    int pads = 0;
    for (int s = 0; s < S; ++s)
        for (int g = 0; g < 4; ++g)
            for (int j = 0; j < 8; ++j) {
                const int k = 32 * s + 8 * g + j;
                if (k >= K) ++pads; else hits[k]++;
            }
    for (int k = 0; k < K; ++k)
        if (hits[k] != 1) { printf("rows map P%d element %d hit %d times\n", P, k, hits[k]); return 1; }
    if (pads >= 32) { printf("rows map P%d: a whole padded k-step\n", P); return 1; }
    printf("rows map P%d: %d steps, %d pad elements\n", P, S, pads);
    return 0;
}

// The folded image map: fold pair p = 2s + j of k-step s; its halves are unique fragments of one
// load kind (or the second half empty); every element of one frame (C*P*P) exactly once.
static int check_fold(int P) {
    using namespace pe;
    const int rows = kC * P, S = fold_steps(P);
    std::vector<int> hits(rows * P, 0);
    int pads = 0;
    for (int p = 0; p < 2 * S; ++p) {
        const FoldPair fp = fold_pair(P, p);
        if (fp.uf0 < 0 || fp.uf0 >= 2 * tt_steps(P)) { printf("fold pair %d: bad first fragment\n", p); return 1; }
        if (fp.uf1 >= 0 && tt_frag(P, fp.uf1).kind != tt_frag(P, fp.uf0).kind) {
            printf("fold pair %d: two load kinds\n", p); return 1;
        }
        for (int half = 0; half < 2; ++half) {
            const int uf = half ? fp.uf1 : fp.uf0;
            if (uf < 0) { pads += 8; continue; }
            const UFrag f = tt_frag(P, uf);
            for (int j = 0; j < 8; ++j) {
                int u = f.u1, x = f.x1 + j;
                if (f.kind == kUfSplit62 && j >= 6) { u = f.u2; x = f.x2 + j - 6; }
                if (f.kind == kUfTail4 && j >= 4) { ++pads; continue; }
                if (u < 0 || u >= rows || x < 0 || x >= P) { printf("fold map out of row\n"); return 1; }
                hits[u * P + x]++;
            }
        }
    }
    for (int i = 0; i < rows * P; ++i)
        if (hits[i] != 1) { printf("fold map P%d element %d hit %d times\n", P, i, hits[i]); return 1; }
    printf("fold map P%d: %d steps, %d pad elements\n", P, S, pads);
    return pads == 2 * S * 16 - rows * P ? 0 : 1;
}

int main() {
    int bad = 0;
    for (int P : {14, 16}) bad |= check_rows(P);
    if (pe::rows_steps(14) != 37 || pe::rows_steps(16) != 48) { printf("rows step counts\n"); bad = 1; }
    for (int P : {14, 16})
        for (int esz : {2, 4}) bad |= check(P, esz);
    for (int P : {14, 16}) bad |= check_tt(P);
    if (pe::tt_steps(14) != 37 || pe::tt_steps(16) != 48) { printf("tt step counts\n"); bad = 1; }
    for (int P : {14, 16}) bad |= check_fold(P);
    if (pe::fold_steps(14) != 19 || pe::fold_steps(16) != 24) { printf("fold step counts\n"); bad = 1; }
    if (pe::num_steps(14, 2) != 37 || pe::num_steps(16, 2) != 48) { printf("step counts\n"); bad = 1; }
    if (!bad) printf("OK\n");
    return bad;
}
