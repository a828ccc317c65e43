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

// Load placement of the patch-rows map: a load's bytes [start, start + len) must lie inside its own
// row, for every lane half, sub-step and k-step, for bf16 (16-byte fragments) and fp32 input
// (the same 8 elements, 32 bytes) -- in particular for the last row of a buffer, where any byte
// past the row is past the caller's allocation. Every fragment that is not real must be one the
// kernel zeroes (rows_frag_real false). The same for the 16-byte parts of the 128-byte pieces
// that the large-tile kernel stages through LDS.
static int check_rows_loads(int P) {
    using namespace pe;
    const int K = kC * kTp * P * P, S = rows_steps(P);
    int relocated = 0;
    for (int isz : {2, 4}) {
        const int kb = K * isz;
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < 2; ++j) {
                if (!rows_frag_real(P, s, j, 0)) continue;   // not loaded at all
                for (int h = 0; h < 2; ++h) {
                    const int e0 = rows_load_elem(P, s, j, h);
                    const int b0 = e0 * isz, b1 = b0 + 8 * isz;
                    if (b0 < 0 || b1 > kb) { printf("rows load P%d isz%d s%d j%d h%d: bytes [%d, %d) leave a %d-byte row\n", P, isz, s, j, h, b0, b1, kb); return 1; }
                    const bool real = rows_frag_real(P, s, j, h);
                    if (real != (32 * s + 16 * j + 8 * h + 8 <= K)) { printf("rows fragment realness P%d\n", P); return 1; }
                    if (!real) ++relocated;
                }
            }
        const int nch = (kb + 127) / 128;
        for (int c = 0; c < nch; ++c)
            for (int q = 0; q < 8; ++q) {
                const int b0 = c * 128 + 16 * piece_load_part(kb, c, q);
                if (b0 < 0 || b0 + 16 > kb) { printf("piece load P%d isz%d c%d q%d: bytes [%d, %d) leave a %d-byte row\n", P, isz, c, q, b0, b0 + 16, kb); return 1; }
                if (piece_part_real(kb, c, q) != (c * 128 + 16 * q + 16 <= kb)) { printf("piece realness P%d\n", P); return 1; }
            }
    }
    printf("rows loads P%d: inside the row, %d fragments relocated\n", P, relocated);
    return 0;
}

// The grouped order and the LDS stage of single images (P = 14): ttg_uf is a permutation of the
// temporal-split fragments; staging every pixel row as sg_row says (half 0: px 0..7 to slot a;
// half 1: px 6..13 as d0..d3 to the slots of its kind, rows in increasing u) leaves each group's
// slots holding exactly the grouped fragments' elements (zeros in the tail); and the load/write
// schedule writes each row at least two k-steps before the first k-step that reads it (that
// fragment is read one k-step early), into a group buffer only after
// the last read of the group it held, through a ring of four registers that no row overwrites
// while it is still to be written.
static int check_staged() {
    using namespace pe;
    const int P = 14, S = tt_steps(P), NF = 2 * S, NU = kC * P;
    const int ZERO = -2, UNSET = -1;
    std::vector<int> seen(NF, 0);
    for (int g = 0; g < NF; ++g) {
        const int uf = ttg_uf(P, g);
        if (uf < 0 || uf >= NF || seen[uf]++) { printf("ttg_uf is not a permutation at %d\n", g); return 1; }
    }
    for (int g = 0; g < 2 * tt_steps(16); ++g)
        if (ttg_uf(16, g) != g) { printf("ttg_uf(16) is not the identity\n"); return 1; }
    // element id of (u, x): u * P + x
    const int NG = (NU + kSgRows - 1) / kSgRows;
    std::vector<int> slots(NG * 14 * 8, UNSET);
    auto put = [&](int G, int slot, int byte, int first_elem_id, int n, bool zero) {
        if (slot < 0 || slot >= 14 || byte % 4 || byte + 2 * n > 16) { printf("slot write out of range\n"); return false; }
        for (int i = 0; i < n; ++i) slots[(G * 14 + slot) * 8 + byte / 2 + i] = zero ? ZERO : first_elem_id + i;
        return true;
    };
    for (int u = 0; u < NU; ++u) {
        const SgRow w = sg_row(u);
        const int G = u / kSgRows, e = u * P;   // d_k of half 1 = elements (u, 6 + 2k), (u, 7 + 2k)
        bool ok = put(G, w.slot_a, 0, e + 0, 8, false);
        if (w.kind == 0) {
            ok = ok && put(G, w.slot_b, 0, e + 8, 6, false);
            ok = ok && put(G, w.slot_b, 12, e + 12, 2, false);                 // junk: d3 again
        } else if (w.kind == 1) {
            for (int k = 0; k < 3; ++k) ok = ok && put(G, w.slot_b + k, 12, e + 8 + 2 * k, 2, false);
        } else if (w.kind == 2) {
            ok = ok && put(G, w.slot_b, 12, e + 8, 2, false);
            ok = ok && put(G, w.slot_b + 1, 0, e + 10, 4, false);
            ok = ok && put(G, w.slot_b + 1, 8, 0, 4, true);
        } else {
            ok = false;
        }
        if (!ok) { printf("staged write of row %d\n", u); return 1; }
    }
    std::vector<int> first_read(NU, 1 << 30);
    for (int g = 0; g < NF; ++g) {
        const UFrag f = tt_frag(P, ttg_uf(P, g));
        const int G = g / 14, slot = g % 14;
        for (int j = 0; j < 8; ++j) {
            int want;
            if (f.kind == kUfTail4 && j >= 4) want = ZERO;
            else if (f.kind == kUfSplit62 && j >= 6) want = f.u2 * P + f.x2 + j - 6;
            else want = f.u1 * P + f.x1 + j;
            const int got = slots[(G * 14 + slot) * 8 + j];
            if (got != want) { printf("staged fragment %d element %d: %d, want %d\n", g, j, got, want); return 1; }
            if (want >= 0 && g / 2 < first_read[want / P]) first_read[want / P] = g / 2;
        }
    }
    for (int u = kSgRows; u < NU; ++u) {
        const int G = u / kSgRows, ld = sg_load_step(u), wr = ld + kSgLag;
        // the kernel reads k-step s's fragment during k-step s - 1, after that step's writes of
        // the step before: a row must be written at least two k-steps before its first read
        if (ld < 0 || wr > first_read[u] - 2) { printf("row %d written at step %d, read at %d\n", u, wr, first_read[u]); return 1; }
        // group G - 2's last fragment is read during k-step 7(G - 2) + 5 (one ahead)
        if (G >= 2 && wr < kSgSteps * (G - 2) + kSgSteps - 1) { printf("row %d overwrites group %d early\n", u, G - 2); return 1; }
        for (int v = u + 1; v < NU; ++v)
            if (v % 4 == u % 4 && sg_load_step(v) <= wr) { printf("rows %d and %d share a register\n", u, v); return 1; }
        if (u > kSgRows && sg_load_step(u) < sg_load_step(u - 1)) { printf("loads out of order\n"); return 1; }
    }
    for (int u = 0; u < kSgRows; ++u)
        if (first_read[u] < 0) return 1;
    printf("staged images P14: %d fragments in %d groups, schedule ok\n", NF, NG);
    return 0;
}

int main() {
    int bad = 0;
    bad |= check_staged();
    for (int P : {14, 16}) bad |= check_rows(P);
    for (int P : {14, 16}) bad |= check_rows_loads(P);
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
