// pe_internal.h -- types shared by the C ABI (pe_api.cpp) and the gfx950 kernels
// (pe_kernels.hip). Not installed; the public interface is include/pe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

constexpr int kC = 3;          // input channels
constexpr int kTp = 2;         // temporal patch size
constexpr int kMaxItems = 64;  // items per launch (the item table travels in the kernel arguments)

// One item (image or video) of a frames launch. Offsets are in input elements relative to the
// launch's input pointer; rows are relative to the launch's first output row.
struct Item {
    int32_t row0;     // first output row of the item
    int32_t t, h, w;  // patch grid
    int32_t F;        // frame count
    uint32_t x_off;   // element offset of the item's first frame
};

struct FwdArgs {
    const void *in;      // launch input base
    const void *wpk;     // packed weight
    const float *bias;   // fp32 [E] or null
    void *out;           // launch output base (row 0 of the launch)
    uint32_t in_bytes;   // bytes addressable from `in` (buffer range; loads beyond read 0)
    int32_t n_rows;      // output rows in this launch
    int32_t E;
    int32_t kind;        // 0 patch rows, 1 frames
    int32_t order;       // 0 raster, 1 merge window
    int32_t m;           // merge size
    int32_t n_items;
    int32_t tiles_m, tiles_n;
    int32_t pad_;
    Item items[kMaxItems];
};

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

// Launchers (pe_kernels.hip). Return the launch status.
hipError_t launch_pack(const void *w, int w_esz, void *wpk, int P, int E, hipStream_t st);
hipError_t launch_bias(const void *b, int b_esz, float *bias32, int E, hipStream_t st);
hipError_t launch_forward(const FwdArgs &a, int P, int in_esz, int out_esz, hipStream_t st);

}  // namespace pe
