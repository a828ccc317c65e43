// pe_internal.h -- types shared by the C ABI (pe_api.cpp) and the gfx950 kernels (pe_device.h,
// pe_gather.h, the kernel headers and the .hip units that instantiate them). Not installed; the
// public interface is include/pe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pe_plan.h"  // FwdArgs, Item, kMaxItems, TileId

namespace pe {

constexpr int kC = 3;          // input channels
constexpr int kTp = 2;         // temporal patch size

// Fragment map: which patch elements the lane group g (0..3) of k-step s feeds to the matrix
// core. A fragment is 16 bytes: 8 bf16 or 4 fp32 elements. Pixel rows are indexed
// r = (tt*C + c)*P + py, elements within a row by px.
enum PieceKind { kFull = 0, kSplit = 1, kPad = 2 };
struct Piece {
    int kind;
    int r1, x1;  // first piece: row, first px (whole fragment if kFull)
    int r2, x2;  // second piece (kSplit)
};

__host__ __device__ constexpr int frag_elems(int esz) { return 16 / esz; }
// elements of the first piece of a split fragment: bf16 P=14 -> 6 (+2), fp32 P=14 -> 2 (+2)
__host__ __device__ constexpr int split_first(int P, int esz) { return P % frag_elems(esz); }
__host__ __device__ constexpr int full_steps(int P, int esz) {
    return kC * kTp * P * (P / frag_elems(esz)) / 4;
}
__host__ __device__ constexpr int split_frags(int P, int esz) {
    // remainder 6 (bf16): 4 rows -> 3 fragments; remainder 2 (fp32): 2 rows -> 1 fragment;
    // remainder 0: none
    return split_first(P, esz) == 0 ? 0
         : (esz == 2 ? kC * kTp * P / 4 * 3 : kC * kTp * P / 2);
}
__host__ __device__ constexpr int num_steps(int P, int esz) {
    return full_steps(P, esz) + (split_frags(P, esz) + 3) / 4;
}
// Packed weight layout: [step][column block of NB][lane group g][NB columns][16 bytes], NB = 32
// for bf16 (32x32 matrix-core blocks) and 16 for fp32 (16x16 blocks); E is padded with zero
// columns up to a multiple of NB.
__host__ __device__ constexpr int pack_block(int esz) { return esz == 2 ? 32 : 16; }
__host__ __device__ constexpr int packed_cols(int E, int esz) {
    return (E + pack_block(esz) - 1) / pack_block(esz) * pack_block(esz);
}
// P values the fragment map covers: P % 8 == 0 (all whole fragments) or P == 14.
__host__ __device__ constexpr bool patch_supported(int P) { return P == 14 || P == 16; }

__host__ __device__ inline Piece frag_piece(int P, int esz, int s, int g) {
    Piece p{kPad, 0, 0, 0, 0};
    const int epf = frag_elems(esz);
    const int per = P / epf;   // whole fragments per pixel row
    const int sfull = full_steps(P, esz);
    if (s < sfull) {
        const int f = 4 * s + g;
        p.kind = kFull;
        p.r1 = f / per;
        p.x1 = (f % per) * epf;
        return p;
    }
    const int j = 4 * (s - sfull) + g;
    if (j >= split_frags(P, esz)) return p;
    p.kind = kSplit;
    if (esz == 2) {  // rows a, b, c, d -> (a[8:14], d[8:10]), (b[8:14], d[10:12]), (c[8:14], d[12:14])
        const int q = j / 3, i = j % 3;
        p.r1 = 4 * q + i;
        p.x1 = per * epf;
        p.r2 = 4 * q + 3;
        p.x2 = per * epf + 2 * i;
    } else {         // rows a, b -> (a[12:14], b[12:14])
        p.r1 = 2 * j;
        p.x1 = per * epf;
        p.r2 = 2 * j + 1;
        p.x2 = per * epf;
    }
    return p;
}

// bf16 fragment map of the 32x32x16 kernel. A k-step holds four 8-element fragments
// g = 2j + h: h is the temporal slot tt (the two lane halves of a 32x32x16 product read the two
// frames of a temporal patch, or the same frame twice for an image), j picks one of the step's
// two "unique" fragments uf = 2s + j over the C*P pixel rows u = c*P + py of one temporal slot.
//   P % 8 == 0: row u = uf / (P/8), px 8*(uf % (P/8)) .. +7 (one 16-byte load).
//   P == 14:    uf < 42: row uf, px 0..7;
//               42 <= uf < 72: rows a..d = 4q..4q+3, q = (uf-42)/3, i = (uf-42)%3:
//                              row a+i px 8..13 (12 bytes) + row d px 8+2i..9+2i (4 bytes);
//               uf == 72:      row 40 px 8..13 + row 41 px 8..9;
//               uf == 73:      row 41 px 10..13 (8 bytes) + 4 zero elements.
// 37 steps for P = 14 (1184 = 1176 + 8 zero k), 48 for P = 16.
enum UfKind { kUfFull = 0, kUfSplit62 = 1, kUfTail4 = 2 };
struct UFrag {
    int kind;
    int u1, x1;  // first piece: pixel row within the temporal slot, first px
    int u2, x2;  // second piece (kUfSplit62)
};
__host__ __device__ constexpr int tt_steps(int P) {
    return P % 8 == 0 ? kC * P * (P / 8) / 2 : (P == 14 ? 37 : 0);
}
__host__ __device__ constexpr UFrag tt_frag(int P, int uf) {
    UFrag f{kUfFull, 0, 0, 0, 0};
    if (P % 8 == 0) {
        f.u1 = uf / (P / 8);
        f.x1 = 8 * (uf % (P / 8));
        return f;
    }
    if (uf < kC * P) {            // 42 whole fragments
        f.u1 = uf;
        return f;
    }
    if (uf < 72) {
        const int q = (uf - 42) / 3, i = (uf - 42) % 3;
        f.kind = kUfSplit62;
        f.u1 = 4 * q + i; f.x1 = 8;
        f.u2 = 4 * q + 3; f.x2 = 8 + 2 * i;
        return f;
    }
    if (uf == 72) {
        f.kind = kUfSplit62;
        f.u1 = 40; f.x1 = 8;
        f.u2 = 41; f.x2 = 8;
        return f;
    }
    f.kind = kUfTail4;
    f.u1 = 41; f.x1 = 10;
    return f;
}

// Grouped order of the same unique fragments, for single images staged through LDS (P = 14): the
// fragments of each 4 pixel rows a..d = 4q..4q+3 are consecutive, ufg = 7q + k:
//   k = 0..3: row 4q+k px 0..7 (tt uf 4q+k);  k = 4..6: the split fragment of row 4q+k-4 (tt uf
//   42 + 3q + k-4);  then ufg 70, 71 = rows 40, 41 px 0..7 and ufg 72, 73 = tt uf 72, 73.
// So 8 pixel rows fill 14 fragments (7 k-steps) and a group of 8 rows can be staged, used and
// replaced while the next is loaded. P % 8 == 0 keeps the temporal-split order.
__host__ __device__ constexpr int ttg_uf(int P, int ufg) {
    if (P % 8 == 0 || ufg >= 72) return ufg;
    if (ufg >= 70) return ufg - 30;
    return ufg % 7 < 4 ? 4 * (ufg / 7) + ufg % 7 : 42 + 3 * (ufg / 7) + ufg % 7 - 4;
}
// LDS stage of the grouped order (P = 14): group G = u / 8 of pixel rows u, its fragments
// ufg = 14G + slot. A lane loads 16 bytes of one pixel row of a patch: part 0 px 0..7 (dwords
// d0..d3), part 1 px 6..13 (d1..d3 = px 8..13; px 6..7 again, so no load leaves the patch's 28
// bytes). Where they go, as 16-byte slots of the patch's group:
//   kind 0: part 0 -> slot a; part 1 -> (d1, d2, d3, junk) at slot b (the junk dword is
//           overwritten by the later row that owns it)
//   kind 1: part 0 -> slot a; part 1 -> d1, d2, d3 at byte 12 of slots b, b+1, b+2 (row d)
//   kind 2: part 0 -> slot a; part 1 -> d1 at byte 12 of slot b, (d2, d3, 0, 0) at slot b+1
// Rows are written in increasing u.
struct SgRow { int kind, slot_a, slot_b; };
__host__ __device__ constexpr SgRow sg_row(int u) {
    if (u == 40) return SgRow{0, 0, 2};
    if (u == 41) return SgRow{2, 1, 2};
    const int b = (u / 4) % 2, i = u % 4;
    return i < 3 ? SgRow{0, 7 * b + i, 7 * b + 4 + i} : SgRow{1, 7 * b + 3, 7 * b + 4};
}
constexpr int kSgRows = 8;   // pixel rows per group
constexpr int kSgSteps = 7;  // k-steps per group
// k-step during which pixel row u (u >= 8) is loaded: the rows of group G over the k-steps of
// group G - 1, two at its first step; each is written to LDS kSgLag steps later (after that
// step's products). Rows 0..7 are loaded and written before the k loop.
constexpr int kSgLag = 2;
__host__ __device__ constexpr int sg_load_step(int u) {
    return kSgSteps * (u / kSgRows - 1) + (u % kSgRows == 0 ? 0 : u % kSgRows - 1);
}

// bf16 patch-rows map: a patch row is stored in (c, t, py, px) order, so k-step s and lane
// group g take its elements [32s + 8g, 32s + 8g + 8): every load is 16 contiguous bytes and a
// k-step reads 64 contiguous bytes of each row. Elements at K and beyond are zero in the packed
// weight (P = 14: the last lane group of step 36).
__host__ __device__ constexpr int rows_steps(int P) { return (kC * kTp * P * P + 31) / 32; }
// Where the loads of the rows map go. The raw buffer loads take the per-step part of the address
// as a scalar offset, which the hardware's range check does not cover, so no load may rely on
// the range check to stay inside the row: a fragment past the row's K elements (P = 14: lane
// half 1 of the last sub-step) loads lane half 0's elements instead, which lie inside the row,
// and the kernel zeroes it.
//   rows_frag_real: elements [32s + 16j + 8h, +8) are elements of the row (K is a multiple of 8)
//   rows_load_elem: first element that lane half h actually loads for (s, j)
__host__ __device__ constexpr bool rows_frag_real(int P, int s, int j, int h) {
    return 32 * s + 16 * j + 8 * h < kC * kTp * P * P;
}
__host__ __device__ constexpr int rows_load_elem(int P, int s, int j, int h) {
    return rows_frag_real(P, s, j, h) ? 32 * s + 16 * j + 8 * h : 32 * s + 16 * j;
}
// The large-tile kernel stages patch rows through LDS in 128-byte pieces, each loaded as eight
// 16-byte parts. Part q of piece c lies at bytes c*128 + 16q of a row of kb bytes (kb a multiple
// of 16); a part past the row end loads part 0 of the same piece instead (inside the row, since
// a piece exists only if it starts inside the row) and is zeroed.
__host__ __device__ constexpr bool piece_part_real(int kb, int c, int q) { return c * 128 + 16 * q < kb; }
__host__ __device__ constexpr int piece_load_part(int kb, int c, int q) { return piece_part_real(kb, c, q) ? q : 0; }

// bf16 folded map for single-frame items (opt-in, approximate): both temporal slots of an image read
// the same frame, so out = x . (W[:, :, 0] + W[:, :, 1]) over the C*P*P elements of one frame. The
// folded weight is rounded to bf16 once. k-step s has four fragments g = 2j + h: lane half h of the
// j-th 32x32x16 product reads fold pair p = 2s + j, half h. A pair is two unique fragments of the
// same load kind (tt_frag's kinds), loaded by one instruction, or one fragment and a zero half:
//   P % 8 == 0: p -> (2p, 2p + 1)                        (C*P*P/8 fragments, C*P*P/32 steps)
//   P == 14:    p < 36 -> (2p, 2p + 1); p == 36 -> (72, none); p == 37 -> (73, none)   (19 steps)
__host__ __device__ constexpr int fold_steps(int P) {
    return P % 8 == 0 ? kC * P * (P / 8) / 4 : (P == 14 ? 19 : 0);
}
struct FoldPair { int uf0, uf1; };  // uf1 < 0: lanes 32-63 hold zeros
__host__ __device__ constexpr FoldPair fold_pair(int P, int p) {
    if (P % 8 != 0 && p >= 36) return FoldPair{36 + p, -1};
    return FoldPair{2 * p, 2 * p + 1};
}

// k-steps of the packed weight: the temporal-split map for bf16, frag_piece's map for fp32
__host__ __device__ constexpr int packed_steps(int P, int esz) {
    return esz == 2 ? tt_steps(P) : num_steps(P, esz);
}

// How the bf16 kernels read A: frames with two temporal slots, frames that are all single images
// (both slots the same pixels), pre-flattened patch rows (the rows map above), single images
// against the folded weight (the fold map above), or single images whose pixel rows are staged
// through LDS in the grouped order (P = 14, bf16 input, large tiles).
enum AMode { kAFrames = 0, kAImage = 1, kARows = 2, kAFold = 3, kAStaged = 4 };
// packed weight maps (kPackTTG: the temporal-split map in the grouped order)
enum PackMap { kPackTT = 0, kPackRows = 1, kPackFold = 2, kPackTTG = 3 };

// Launchers (pe_pack.hip and pe_fwd_p*.hip). Return the launch status.
// map: PackMap (kPackRows and kPackFold are bf16 only)
hipError_t launch_pack(const void *w, int w_esz, void *wpk, int P, int E, int map, hipStream_t st);
hipError_t launch_bias(const void *b, int b_esz, float *bias32, int E, hipStream_t st);
hipError_t launch_forward(const FwdArgs &a, int P, int w_esz, int in_esz, int out_esz, hipStream_t st);
// the forward kernels, one translation unit per patch size and input dtype (pe_fwd_p*.hip)
hipError_t launch_forward_p14_bf16in(const FwdArgs &a, int out_esz, hipStream_t st);
hipError_t launch_forward_p16_bf16in(const FwdArgs &a, int out_esz, hipStream_t st);
hipError_t launch_forward_p14_f32in(const FwdArgs &a, int w_esz, int out_esz, hipStream_t st);
hipError_t launch_forward_p16_f32in(const FwdArgs &a, int w_esz, int out_esz, hipStream_t st);

// LayerNorm over the last dimension of [n_rows, dim] (pe_norm.hip). esz: bytes of an x / y element
// (2 bf16, 4 fp32), psz: of a gamma / beta element; gamma / beta may be null (1 / 0).
constexpr int kNormMaxDim = 4096;
hipError_t launch_layernorm(const void *x, int esz, void *y, const void *gamma, const void *beta, int psz,
                            float eps, int64_t n_rows, int dim, hipStream_t st);

}  // namespace pe
