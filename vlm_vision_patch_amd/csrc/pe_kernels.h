// pe_kernels.h -- gfx950 forward kernels of the vision PatchEmbed and their launchers. Included
// by the translation units that instantiate them, pe_fwd_p{14,16}_{bf16,f32}in.hip (one per
// patch size and input dtype, built in parallel). The kernels live in pe_fwd32.h, pe_fwd32_sk.h
// and pe_fwd16.h; the patch gather they share in pe_gather.h; the weight pack in pe_pack.hip.
//
// The operation ("Qwen2.5VL-Vision Encode-PatchEmbed", the bullet list on the convolution):
// a Conv3d whose kernel equals its stride meets each patch once, so it is a matrix product
//   out[r, e] = sum_k A[r, k] * W[e, k] (+ b[e]),  K = C*Tp*P*P,
// where A[r, :] is the patch behind output row r, flattened. Nothing materialises A: the
// forward kernels read each patch's pixels straight from the frames (or patch rows) into the
// registers that feed the matrix cores.
//
// K order. Any permutation of k applied to both A and W leaves the sum unchanged, so the
// kernels use ones that suit 16-byte fragments (pe_internal.h holds the maps; the weight is
// packed once in the same order by pe_pack_kernel):
//  - bf16 frames, tt_frag: the two lane halves of a 32x32x16 product read the two temporal slots
//    of the patch, each fragment one of the C*P pixel rows' 8-element pieces (P = 14: a whole
//    px 0..7 piece, or a 6-element rest joined with 2 elements of a fourth row), 37 k-steps for
//    P = 14 (1184 = 1176 + 8), 48 for P = 16;
//  - bf16 patch rows, rows_steps: the stored (c, t, py, px) order, 32 contiguous elements a step;
//  - bf16 single images with the opt-in fold, fold_pair: one frame's fragments against
//    W[:, :, 0] + W[:, :, 1] (19 k-steps for P = 14);
//  - fp32, frag_piece: 4-element fragments (P = 14: 3 whole + pairs of 2-element rests).
//
// bf16 kernel (pe_fwd32_kernel): v_mfma_f32_32x32x16_bf16, fp32 accumulate. (Measured on this
// chip: the 32x32x16 form keeps the matrix pipe ~87% busy from a single wave per SIMD; the
// 16x16x32 form reaches only ~54% from one wave.) A k-step of four fragments is two 32x32x16
// products: lane l supplies row (or column) l % 32 and fragment g = 2j + l / 32 in sub-step j.
// A workgroup computes a BM x BN tile with WM x WN waves, each wave TM x TN blocks of 32 x 32.
// For frames each wave loads its own A fragments with raw buffer loads (32-bit offsets; reads
// past the range return 0) straight into registers; patch rows are staged through LDS in whole
// 128-byte pieces. The packed weight for one k-step and the tile's columns is one contiguous
// run, staged in LDS (KS k-steps per buffer, two buffers) and read as one conflict-free 1 KB
// ds_read_b128 per sub-step and 32-column block.
//
// bf16 split-k kernel (pe_fwd32_sk_kernel), for few rows: four waves share a 32 x 160 (or 128)
// tile, each over a quarter of the k-steps, partial tiles summed through LDS.
//
// fp32 kernel (pe_fwd16_kernel): split-k like the bf16 split-k kernel, with 16x16 blocks and
// v_mfma_f32_16x16x4_f32: four waves share a 32 x 160 (or 128) tile, each over a quarter of the
// k-steps, the weight straight from global memory into registers.
//
// Rows of a tile are output rows in output order; each lane maps its row back to the patch
// (item, tp, hp, wp) through the raster or merge-window order, so the order costs only index
// arithmetic and the stores stay row-contiguous.
#pragma once

#include "pe_fwd16.h"
#include "pe_fwd32.h"
#include "pe_fwd32_sk.h"

namespace pe {

// ----------------------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------------------
template <int P, int ESZ, int OSZ, int TM, int TN, int AD>
inline hipError_t launch16(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = TM * 16, BN = TN * 16;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
    if (a.staged) return hipErrorInvalidValue;
    hipLaunchKernelGGL((pe_fwd16_kernel<P, ESZ, OSZ, TM, TN, AD>), dim3(a.tiles_m * a.tiles_n), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int P, int ISZ, int OSZ, int TM, int TN, int WM, int WN, int KS, int PF, int AD, int BD>
inline hipError_t launch32(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
    const dim3 grid(a.tiles_m * a.tiles_n), block(WM * WN * 64);
    if (a.staged) return hipErrorInvalidValue;  // launch32_staged
    if (a.kind == 0)
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kARows, false>), grid, block, 0, st, a);
    else if (a.img && a.fold && a.mixg)
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAFold, true>), grid, block, 0, st, a);
    else if (a.img && a.fold)
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAFold, false>), grid, block, 0, st, a);
    else if (a.img && a.mixg)
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAImage, true>), grid, block, 0, st, a);
    else if (a.img)
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAImage, false>), grid, block, 0, st, a);
    else if (a.mixg)
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAFrames, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAFrames, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

// Single images staged through LDS (opt-in; bf16 input, P = 14, one frame size): the tile's pixel
// rows are shared by the waves, so a wave takes TM = 2 row blocks and reads half the weight
// fragments per product.
template <int P, int ISZ, int OSZ, int TM, int TN, int WM, int WN, int KS, int PF, int AD, int BD>
inline hipError_t launch32_staged(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
    if (!a.staged || !a.img || a.fold || a.kind != 1) return hipErrorInvalidValue;
    if constexpr (P == 14 && ISZ == 2) {
        if (a.mixg) return hipErrorInvalidValue;  // one frame geometry per staged launch
        hipLaunchKernelGGL((pe_fwd32_kernel<P, ISZ, OSZ, TM, TN, WM, WN, KS, PF, AD, BD, kAStaged, false>),
                           dim3(a.tiles_m * a.tiles_n), dim3(WM * WN * 64), 0, st, a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int P, int ISZ, int OSZ, int TM, int TN, int AD>
inline hipError_t launch_sk(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = TM * 32, BN = TN * 32;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
    if (a.staged) return hipErrorInvalidValue;  // the LDS-staged image path is the large-tile kernel's
    const dim3 grid(a.tiles_m * a.tiles_n), block(256);
    if (a.kind == 0)
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kARows, false>), grid, block, 0, st, a);
    else if (a.img && a.fold && a.mixg)
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kAFold, true>), grid, block, 0, st, a);
    else if (a.img && a.fold)
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kAFold, false>), grid, block, 0, st, a);
    else if (a.img && a.mixg)
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kAImage, true>), grid, block, 0, st, a);
    else if (a.img)
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kAImage, false>), grid, block, 0, st, a);
    else if (a.mixg)
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kAFrames, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((pe_fwd32_sk_kernel<P, ISZ, OSZ, TM, TN, AD, kAFrames, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

// ESZ: weight element size; ISZ: input element size (fp32 input meets a bf16 weight by rounding
// on load)
template <int P, int ESZ, int ISZ, int OSZ>
inline hipError_t launch_p(const FwdArgs &a, hipStream_t st) {
    // the plan (pe_plan.cpp) chose the kernel and its tile; the launchers recompute the tile
    // counts from their own template shapes and refuse a launch whose shape differs
    const int skn = a.E % 160 == 0 ? 160 : 128;
    if constexpr (ESZ == 4) {
        // fp32 I/O: 16x16 blocks, split-k over four waves, small tiles; 32 x 160 tiles where E
        // allows (1024 x 1280 makes 256 of them: one round, where 32 x 128 tiles take 1.25),
        // loads two k-steps ahead
        if (a.tiles != kTileF32) return hipErrorInvalidValue;
        if (skn == 160) return launch16<P, ESZ, OSZ, 2, 10, 2>(a, st);
        return launch16<P, ESZ, OSZ, 2, 8, 2>(a, st);
    } else {
        // 8 waves of 32 x BN (two per SIMD), one weight k-step per LDS buffer (a barrier per k-step
        // measured ~2% faster than two), eight weight fragments read ahead
        if (a.staged) {
            // staged single images: 8 waves of 64 x 128 (or 64 x 64), all of a k-step's weight
            // fragments read ahead
            switch (a.tiles) {
                case kTileLarge256: return launch32_staged<P, ISZ, OSZ, 2, 4, 4, 2, 1, 8, 2, 3>(a, st);
                case kTileLarge128: return launch32_staged<P, ISZ, OSZ, 2, 2, 4, 2, 1, 4, 2, 3>(a, st);
                default: return hipErrorInvalidValue;
            }
        }
        switch (a.tiles) {
            case kTileLarge256: return launch32<P, ISZ, OSZ, 1, 8, 8, 1, 1, 8, 2, 3>(a, st);
            case kTileLarge128: return launch32<P, ISZ, OSZ, 1, 4, 8, 1, 1, 8, 2, 3>(a, st);
            case kTileSplitK:
                // few rows: split-K workgroups, 32 rows by 160 (or 128) columns
                if (skn == 160) return launch_sk<P, ISZ, OSZ, 1, 5, 2>(a, st);
                return launch_sk<P, ISZ, OSZ, 1, 4, 2>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
}

}  // namespace pe
