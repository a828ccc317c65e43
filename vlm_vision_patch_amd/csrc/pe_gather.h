// pe_gather.h -- the A operand of the forward kernels: output row -> patch, and the loads of a
// patch's pixels (frames or patch rows, bf16 or fp32) into the registers that feed the matrix
// cores, in the k orders of pe_internal.h. Nothing materialises the patch matrix.
#pragma once

#include "pe_device.h"

namespace pe {

// ----------------------------------------------------------------------------------------
// Forward kernel
// ----------------------------------------------------------------------------------------
struct PatchRef {
    uint32_t base;   // element offset of (tt=0, c=0, py=0, px=0)
    uint32_t tstr;   // element offset of temporal slot 1 relative to slot 0 (0: repeated frame)
    uint32_t plane;  // channel stride
    uint32_t rstr;   // pixel-row stride
};

// Output row -> the patch it comes from (see pe.h for the orders).
template <int P>
__device__ __forceinline__ PatchRef patch_of_row(const FwdArgs &a, int row) {
    PatchRef pr{0u, 0u, 0u, 0u};
    if (row < 0 || row >= a.n_rows) return pr;  // tail rows: harmless in-range reads
    if (a.kind == 0) {
        pr.base = (uint32_t)row * (uint32_t)(kC * kTp * P * P);
        pr.tstr = P * P;
        pr.plane = kTp * P * P;
        pr.rstr = P;
        return pr;
    }
    Item it;
    uint32_t q;
    if (a.uni) {
        // identical items: the item index is a division, and every field but the offset is item 0's
        // (scalar loads of the kernel arguments at fixed offsets, no dependent table reads)
        const uint32_t idx = (uint32_t)row / (uint32_t)a.u_rows;
        it = a.items[0];
        it.x_off = idx * a.u_elems;
        q = (uint32_t)row - idx * (uint32_t)a.u_rows;
    } else {
        int lo = 0, hi = a.n_items - 1;
        while (lo < hi) {  // last item whose first row <= row
            const int mid = (lo + hi + 1) >> 1;
            if (row >= a.items[mid].row0) lo = mid; else hi = mid - 1;
        }
        it = a.items[lo];
        q = (uint32_t)(row - it.row0);
    }
    uint32_t tp, hp, wp;
    if (a.order == 0) {
        wp = q % (uint32_t)it.w;
        const uint32_t r2 = q / (uint32_t)it.w;
        hp = r2 % (uint32_t)it.h;
        tp = r2 / (uint32_t)it.h;
    } else {
        const uint32_t m = (uint32_t)a.m;
        const uint32_t dw = q % m, r1 = q / m;
        const uint32_t dh = r1 % m, win = r1 / m;
        const uint32_t mw = (uint32_t)it.w / m, mh = (uint32_t)it.h / m;
        const uint32_t wm = win % mw, r3 = win / mw;
        const uint32_t hm = r3 % mh;
        tp = r3 / mh;
        hp = hm * m + dh;
        wp = wm * m + dw;
    }
    const uint32_t Wpx = (uint32_t)it.w * P, Hpx = (uint32_t)it.h * P;
    const uint32_t plane = Hpx * Wpx, fe = kC * plane;
    pr.base = it.x_off + (tp * kTp) * fe + hp * P * Wpx + wp * P;
    pr.tstr = (tp * kTp + 1 < (uint32_t)it.F) ? fe : 0u;
    pr.plane = plane;
    pr.rstr = Wpx;
    return pr;
}


// ---- A fragments of the 32x32x16 kernels (temporal-split map, see pe_internal.h).
// The input is bf16 (ISZ = 2) or fp32 (ISZ = 4; rounded to bf16, nearest-even, when the products
// use it). A fragment as loaded: one 16-byte register of 8 bf16, or two of 8 fp32.
template <int ISZ> struct AFrag { u32x4 d[ISZ / 2]; };

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}
template <int ISZ>
__device__ __forceinline__ u32x4 frag_bf16(const AFrag<ISZ> &f) {
    if constexpr (ISZ == 2) {
        return f.d[0];
    } else {
        const f32x4 a = __builtin_bit_cast(f32x4, f.d[0]), b = __builtin_bit_cast(f32x4, f.d[1]);
        return u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
    }
}
// loads of 8 consecutive elements; of 6 + 2 elements from two places; of 4 elements + 4 zeros
template <int ISZ>
__device__ __forceinline__ void ld_whole(__amdgpu_buffer_rsrc_t r, uint32_t v, int so, AFrag<ISZ> &f) {
    f.d[0] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, so, 0);
    if constexpr (ISZ == 4) f.d[1] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, so + 16, 0);
}
template <int ISZ>
__device__ __forceinline__ void ld_split62(__amdgpu_buffer_rsrc_t r, uint32_t v1, int so1, uint32_t v2, int so2,
                                           AFrag<ISZ> &f) {
    if constexpr (ISZ == 2) {
        const u32x3 m3 = __builtin_amdgcn_raw_buffer_load_b96(r, (int)v1, so1, 0);
        const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b32(r, (int)v2, so2, 0);
        f.d[0] = u32x4{m3.x, m3.y, m3.z, e1};
    } else {
        f.d[0] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)v1, so1, 0);
        const u32x2 m2 = __builtin_amdgcn_raw_buffer_load_b64(r, (int)v1, so1 + 16, 0);
        const u32x2 e2 = __builtin_amdgcn_raw_buffer_load_b64(r, (int)v2, so2, 0);
        f.d[1] = u32x4{m2.x, m2.y, e2.x, e2.y};
    }
}
template <int ISZ>
__device__ __forceinline__ void ld_tail4(__amdgpu_buffer_rsrc_t r, uint32_t v, int so, AFrag<ISZ> &f) {
    if constexpr (ISZ == 2) {
        const u32x2 m2 = __builtin_amdgcn_raw_buffer_load_b64(r, (int)v, so, 0);
        f.d[0] = u32x4{m2.x, m2.y, 0u, 0u};
    } else {
        f.d[0] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, so, 0);
        f.d[1] = u32x4{0u, 0u, 0u, 0u};
    }
}
template <int ISZ>
__device__ __forceinline__ void zero_frag(AFrag<ISZ> &f) {
#pragma unroll
    for (int i = 0; i < ISZ / 2; ++i) f.d[i] = u32x4{0u, 0u, 0u, 0u};
}

// Byte offset of element x of pixel row u (u = c*P + py) of one temporal slot.
template <int P, int ISZ>
__device__ __forceinline__ uint32_t frag_off(int u, int x, uint32_t plane, uint32_t rstr) {
    return ((uint32_t)(u / P) * plane + (uint32_t)(u % P) * rstr + (uint32_t)x) * (uint32_t)ISZ;
}
// Image launches (every item one frame): both temporal slots read the same pixels, so the two
// lane halves of a k-step would load the same bytes twice. Instead one load brings unique fragment
// uf = 2s to lanes 0-31 and uf = 2s + 1 to lanes 32-63, and v_permlane32_swap then copies each
// into both halves: half the load instructions and half the bytes. This needs the two fragments
// to be the same kind of load; P = 14's last step (a split fragment and the 8-byte tail) is not.
template <int P, int s>
__device__ constexpr bool img_paired() {
    constexpr UFrag f0 = tt_frag(P, 2 * s), f1 = tt_frag(P, 2 * s + 1);
    return f0.kind == f1.kind && f0.kind != kUfTail4;
}
// Issue the A loads of k-step s for TM 32-row blocks (vb: per-lane byte offset of the lane's
// patch and temporal slot, or of its patch row plus 8 elements for lanes 32-63). Paired image
// steps leave their two fragments in dst[rb][0]. With one frame geometry per launch (MG false) the
// per-step part of every address is one scalar for the whole launch; with items of different
// frame sizes in one launch (MG true) each lane adds its own item's channel plane and pixel-row
// stride (vpl, vrs) instead: two multiply-adds per fragment.
// k-steps of a bf16 kernel for A mode AM
template <int P, int AM>
__host__ __device__ constexpr int a_steps() {
    return AM == kARows ? rows_steps(P) : (AM == kAFold ? fold_steps(P) : tt_steps(P));
}

template <int P, int TM, int AM, int ISZ, int s, bool MG = false>
__device__ __forceinline__ void load_a_step(__amdgpu_buffer_rsrc_t rsrc, const uint32_t (&vb)[TM],
                                            uint32_t plane, uint32_t rstr, int h, AFrag<ISZ> (&dst)[TM][2],
                                            const uint32_t (&vpl)[TM], const uint32_t (&vrs)[TM]) {
    // byte offset of (u, x) for block rb: uniform scalar, or per lane
    auto off = [&](int rb, int u, int x) -> uint32_t {
        return MG ? frag_off<P, ISZ>(u, x, vpl[rb], vrs[rb]) : frag_off<P, ISZ>(u, x, plane, rstr);
    };
    if constexpr (AM == kARows) {
        static_assert((kC * kTp * P * P) % 8 == 0, "a fragment lies wholly inside or outside the row");
        static_for<2>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int k0 = 32 * s + 16 * j;  // first element of lane half 0
            // vb already holds lane half 1's +8 elements; a half-1 fragment past the row loads
            // half 0's elements (rows_load_elem) and is zeroed: the bytes past a row belong to the
            // next row (non-finite values there would poison the products even against the zero
            // weight) or lie past the end of the caller's buffer
            constexpr bool h1_real = rows_frag_real(P, s, j, 1);
            static_assert(rows_load_elem(P, s, j, 1) == (h1_real ? k0 + 8 : k0), "rows map placement");
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                if constexpr (!rows_frag_real(P, s, j, 0)) {
                    zero_frag(dst[rb][j]);
                } else if constexpr (h1_real) {
                    ld_whole<ISZ>(rsrc, vb[rb], ISZ * k0, dst[rb][j]);
                } else {
                    ld_whole<ISZ>(rsrc, h ? vb[rb] - 8u * ISZ : vb[rb], ISZ * k0, dst[rb][j]);
                    if (h) zero_frag(dst[rb][j]);
                }
            }
        });
    } else if constexpr (AM == kAFold) {
        // folded images: lane half h of sub-step j loads fragment fold_pair(2s + j) half h with
        // one instruction (both halves have the same load kind); a pair without a second
        // fragment loads the first twice and a_operands zeroes lanes 32-63
        static_for<2>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr FoldPair fp = fold_pair(P, 2 * s + j);
            constexpr bool two = fp.uf1 >= 0;
            constexpr UFrag f0 = tt_frag(P, fp.uf0), f1 = tt_frag(P, two ? fp.uf1 : fp.uf0);
            static_assert(f0.kind == f1.kind, "a fold pair is one load kind");
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                uint32_t v1, v2 = 0u;
                int so1 = 0, so2 = 0;
                if constexpr (!MG) {
                    so1 = (int)off(0, f0.u1, f0.x1);
                    v1 = vb[rb] + ((two && h) ? off(0, f1.u1, f1.x1) - (uint32_t)so1 : 0u);
                    if constexpr (f0.kind == kUfSplit62) {
                        so2 = (int)off(0, f0.u2, f0.x2);
                        v2 = vb[rb] + ((two && h) ? off(0, f1.u2, f1.x2) - (uint32_t)so2 : 0u);
                    }
                } else {
                    v1 = vb[rb] + ((two && h) ? off(rb, f1.u1, f1.x1) : off(rb, f0.u1, f0.x1));
                    if constexpr (f0.kind == kUfSplit62)
                        v2 = vb[rb] + ((two && h) ? off(rb, f1.u2, f1.x2) : off(rb, f0.u2, f0.x2));
                }
                if constexpr (f0.kind == kUfFull) ld_whole<ISZ>(rsrc, v1, so1, dst[rb][j]);
                else if constexpr (f0.kind == kUfSplit62) ld_split62<ISZ>(rsrc, v1, so1, v2, so2, dst[rb][j]);
                else ld_tail4<ISZ>(rsrc, v1, so1, dst[rb][j]);
            }
        });
    } else if constexpr (AM == kAImage && img_paired<P, s>()) {
        constexpr UFrag f0 = tt_frag(P, 2 * s), f1 = tt_frag(P, 2 * s + 1);
        if constexpr (!MG) {
            const uint32_t o0 = off(0, f0.u1, f0.x1);
            const uint32_t hd = h ? off(0, f1.u1, f1.x1) - o0 : 0u;
            if constexpr (f0.kind == kUfFull) {
#pragma unroll
                for (int rb = 0; rb < TM; ++rb) ld_whole<ISZ>(rsrc, vb[rb] + hd, (int)o0, dst[rb][0]);
            } else {
                const uint32_t p0 = off(0, f0.u2, f0.x2);
                const uint32_t hd2 = h ? off(0, f1.u2, f1.x2) - p0 : 0u;
#pragma unroll
                for (int rb = 0; rb < TM; ++rb)
                    ld_split62<ISZ>(rsrc, vb[rb] + hd, (int)o0, vb[rb] + hd2, (int)p0, dst[rb][0]);
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                const uint32_t v1 = vb[rb] + (h ? off(rb, f1.u1, f1.x1) : off(rb, f0.u1, f0.x1));
                if constexpr (f0.kind == kUfFull) {
                    ld_whole<ISZ>(rsrc, v1, 0, dst[rb][0]);
                } else {
                    const uint32_t v2 = vb[rb] + (h ? off(rb, f1.u2, f1.x2) : off(rb, f0.u2, f0.x2));
                    ld_split62<ISZ>(rsrc, v1, 0, v2, 0, dst[rb][0]);
                }
            }
        }
    } else {
        static_for<2>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr UFrag f = tt_frag(P, 2 * s + j);
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                // (vector, scalar) offsets of the two pieces
                const uint32_t v1 = MG ? vb[rb] + off(rb, f.u1, f.x1) : vb[rb];
                const int so1 = MG ? 0 : (int)off(0, f.u1, f.x1);
                if constexpr (f.kind == kUfFull) {
                    ld_whole<ISZ>(rsrc, v1, so1, dst[rb][j]);
                } else if constexpr (f.kind == kUfSplit62) {
                    const uint32_t v2 = MG ? vb[rb] + off(rb, f.u2, f.x2) : vb[rb];
                    const int so2 = MG ? 0 : (int)off(0, f.u2, f.x2);
                    ld_split62<ISZ>(rsrc, v1, so1, v2, so2, dst[rb][j]);
                } else {
                    ld_tail4<ISZ>(rsrc, v1, so1, dst[rb][j]);
                }
            }
        });
    }
}
// The matrix-core operands of k-step s from what load_a_step loaded (rounded to bf16 here, where
// they are used, so a load's wait is not pulled forward): for a paired image step, or a staged
// image step (lane half h read grouped fragment 2s + h from LDS), (lanes 0-31 of x, twice) and
// (lanes 32-63 of x, twice); otherwise the loads as they are.
__device__ __forceinline__ void swap_halves(const u32x4 &x, u32x4 &lo, u32x4 &hi) {
    const auto r0 = __builtin_amdgcn_permlane32_swap(x.x, x.x, false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(x.y, x.y, false, false);
    const auto r2 = __builtin_amdgcn_permlane32_swap(x.z, x.z, false, false);
    const auto r3 = __builtin_amdgcn_permlane32_swap(x.w, x.w, false, false);
    lo = u32x4{r0[0], r1[0], r2[0], r3[0]};
    hi = u32x4{r0[1], r1[1], r2[1], r3[1]};
}
template <int P, int TM, int AM, int ISZ, int s>
__device__ __forceinline__ void a_operands(const AFrag<ISZ> (&src)[TM][2], u32x4 (&dst)[TM][2], int h) {
#pragma unroll
    for (int rb = 0; rb < TM; ++rb) {
        if constexpr ((AM == kAImage && img_paired<P, s>()) || AM == kAStaged) {
            swap_halves(frag_bf16<ISZ>(src[rb][0]), dst[rb][0], dst[rb][1]);
        } else {
            dst[rb][0] = frag_bf16<ISZ>(src[rb][0]);
            dst[rb][1] = frag_bf16<ISZ>(src[rb][1]);
            if constexpr (AM == kAFold) {
                // a fold pair without a second fragment: lanes 32-63 take zeros
                if constexpr (fold_pair(P, 2 * s).uf1 < 0) dst[rb][0] = h ? u32x4{0u, 0u, 0u, 0u} : dst[rb][0];
                if constexpr (fold_pair(P, 2 * s + 1).uf1 < 0) dst[rb][1] = h ? u32x4{0u, 0u, 0u, 0u} : dst[rb][1];
            }
        }
    }
}

}  // namespace pe
