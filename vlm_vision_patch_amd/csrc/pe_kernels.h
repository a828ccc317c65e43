// pe_kernels.h -- gfx950 kernels of the vision PatchEmbed (templates). Included by the
// translation units that instantiate them: pe_pack.hip (weight pack, bias, dispatch) and
// pe_fwd_p{14,16}_{bf16,f32}in.hip (the forward kernels per patch size and input dtype),
// which build in parallel.
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
// fp32 kernel (pe_fwd16_kernel): the same structure with 16x16 blocks and v_mfma_f32_16x16x4_f32.
//
// Rows of a tile are output rows in output order; each lane maps its row back to the patch
// (item, tp, hp, wp) through the raster or merge-window order, so the order costs only index
// arithmetic and the stores stay row-contiguous.
#pragma once

#include <type_traits>
#include <utility>

#include "pe_internal.h"

namespace pe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// gfx9 buffer descriptor word 3: 32-bit data format, raw (untyped) access.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <int OSZ>
__device__ __forceinline__ void store_out(void *out, int64_t idx, float v) {
    if constexpr (OSZ == 2) {
        static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(v);
    } else {
        static_cast<float *>(out)[idx] = v;
    }
}

// One 16-byte output chunk at element `elem` of out (16/OSZ values, fp32, bias included): with a
// fused addend (an [N, E] tensor in the output dtype and row order, e.g. the position embeddings
// that follow PatchEmbed) its chunk at the same position is added in fp32 first; then one
// round-to-nearest-even cast and a non-temporal store.
template <int OSZ>
__device__ __forceinline__ void store_chunk_r(void *out, bool add, const u32x4 &ad, int64_t elem, float (&v)[16 / OSZ]) {
    if (add) {
        if constexpr (OSZ == 2) {
            const uint32_t d[4] = {ad.x, ad.y, ad.z, ad.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] += __builtin_bit_cast(float, d[i] << 16);
                v[2 * i + 1] += __builtin_bit_cast(float, d[i] & 0xffff0000u);
            }
        } else {
            const f32x4 af = __builtin_bit_cast(f32x4, ad);
            v[0] += af.x; v[1] += af.y; v[2] += af.z; v[3] += af.w;
        }
    }
    char *dst = static_cast<char *>(out) + elem * OSZ;
    if constexpr (OSZ == 2) {
        u32x4 o;
        o.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        o.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        o.z = (uint32_t)f32_to_bf16_rne(v[4]) | ((uint32_t)f32_to_bf16_rne(v[5]) << 16);
        o.w = (uint32_t)f32_to_bf16_rne(v[6]) | ((uint32_t)f32_to_bf16_rne(v[7]) << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(dst));
    } else {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(dst));
    }
}
template <int OSZ>
__device__ __forceinline__ void store_chunk(void *out, const void *addend, int64_t elem, float (&v)[16 / OSZ]) {
    u32x4 ad = u32x4{0u, 0u, 0u, 0u};
    if (addend) ad = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(addend) + elem * OSZ);
    store_chunk_r<OSZ>(out, addend != nullptr, ad, elem, v);
}

// ----------------------------------------------------------------------------------------
// Weight pre-pack: W[E][C][Tp][P][P] -> packed[s][E'/NB][g][NB][16 bytes] in the fragment order
// (NB = 32 for bf16, 16 for fp32; columns e >= E are zero). One thread writes one 16-byte
// fragment (k-step s, column e = NB*cb + n, lane group g).
// ----------------------------------------------------------------------------------------
template <typename TW>
__global__ void pe_pack_kernel(const TW *__restrict__ w, TW *__restrict__ wpk, int P, int E,
                               int S, int map) {
    constexpr int esz = sizeof(TW);
    constexpr int epf = 16 / esz;
    constexpr int NB = pack_block(esz);
    const int Ep = packed_cols(E, esz);
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)S * Ep * 4;
    if (idx >= total) return;
    const int n = (int)(idx % NB);
    int64_t t = idx / NB;
    const int g = (int)(t % 4);
    t /= 4;
    const int ncb = Ep / NB;
    const int cb = (int)(t % ncb);
    const int s = (int)(t / ncb);
    const int e = cb * NB + n;
    TW vals[epf];
    if constexpr (esz == 2) {
        if (map == kPackFold) {
            // folded map: fold pair p = 2s + j, half h of lane group g = 2j + h; each element is
            // W[e, c, 0, py, px] + W[e, c, 1, py, px] (exact in fp32 for bf16 inputs within 2^16
            // of each other in magnitude), rounded to bf16 once
            const FoldPair fp = fold_pair(P, 2 * s + (g >> 1));
            const int uf = (g & 1) ? fp.uf1 : fp.uf0;
            uint16_t out[8];
            const UFrag f = tt_frag(P, uf < 0 ? 0 : uf);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int u = f.u1, x = f.x1 + j;
                bool pad = e >= E || uf < 0;
                if (f.kind == kUfSplit62 && j >= 6) { u = f.u2; x = f.x2 + (j - 6); }
                if (f.kind == kUfTail4 && j >= 4) pad = true;
                float v = 0.f;
                if (!pad) {
                    const int64_t i0 = ((((int64_t)e * kC + u / P) * kTp + 0) * P + u % P) * P + x;
                    const int64_t i1 = i0 + (int64_t)P * P;
                    const uint16_t b0 = reinterpret_cast<const uint16_t *>(w)[i0];
                    const uint16_t b1 = reinterpret_cast<const uint16_t *>(w)[i1];
                    v = __builtin_bit_cast(float, (uint32_t)b0 << 16) + __builtin_bit_cast(float, (uint32_t)b1 << 16);
                }
                out[j] = f32_to_bf16_rne(v);
            }
            uint16_t *dst = reinterpret_cast<uint16_t *>(wpk) + idx * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = out[j];
            return;
        }
    }
    if (esz == 2 && map == kPackRows) {
        // patch-rows map: elements [32s + 8g, +8) of the flattened (c, t, py, px) filter
        const int K = kC * kTp * P * P;
#pragma unroll
        for (int j = 0; j < epf; ++j) {
            const int k = 32 * s + 8 * g + j;
            vals[j] = (e < E && k < K) ? w[(int64_t)e * K + k] : TW(0);
        }
        TW *dst = wpk + idx * epf;
#pragma unroll
        for (int j = 0; j < epf; ++j) dst[j] = vals[j];
        return;
    }
    if constexpr (esz == 2) {
        // temporal-split map: g = 2j + tt, unique fragment uf = 2s + j
        const int tt = g & 1;
        const UFrag f = tt_frag(P, 2 * s + (g >> 1));
#pragma unroll
        for (int j = 0; j < epf; ++j) {
            int u = f.u1, x = f.x1 + j;
            bool pad = e >= E;
            if (f.kind == kUfSplit62 && j >= 6) { u = f.u2; x = f.x2 + (j - 6); }
            if (f.kind == kUfTail4 && j >= 4) pad = true;
            vals[j] = pad ? TW(0) : w[((((int64_t)e * kC + u / P) * kTp + tt) * P + u % P) * P + x];
        }
        TW *dst = wpk + idx * epf;
#pragma unroll
        for (int j = 0; j < epf; ++j) dst[j] = vals[j];
        return;
    }
    const Piece pc = frag_piece(P, esz, s, g);
    const int first = split_first(P, esz);
#pragma unroll
    for (int j = 0; j < epf; ++j) {
        int r = 0, x = 0;
        bool pad = e >= E;
        if (pc.kind == kFull) {
            r = pc.r1; x = pc.x1 + j;
        } else if (pc.kind == kSplit) {
            if (j < first) { r = pc.r1; x = pc.x1 + j; }
            else { r = pc.r2; x = pc.x2 + (j - first); }
        } else {
            pad = true;
        }
        if (pad) {
            vals[j] = TW(0);
        } else {
            const int tt = r / (kC * P), c = (r / P) % kC, py = r % P;
            vals[j] = w[((((int64_t)e * kC + c) * kTp + tt) * P + py) * P + x];
        }
    }
    TW *dst = wpk + idx * epf;
#pragma unroll
    for (int j = 0; j < epf; ++j) dst[j] = vals[j];
}

template <typename TB>
__global__ void pe_bias_kernel(const TB *__restrict__ b, float *__restrict__ b32, int E) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < E) b32[i] = static_cast<float>(b[i]);
}

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

// Compile-time loop: f(IC<0>{}), f(IC<1>{}), ..., f(IC<N-1>{}).
template <int N> using IC = std::integral_constant<int, N>;
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(IC<Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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
// they are used, so a load's wait is not pulled forward): for a paired image step, (lanes 0-31 of
// x, twice) and (lanes 32-63 of x, twice); otherwise the loads as they are.
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
        if constexpr (AM == kAImage && img_paired<P, s>()) {
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

template <int P, int ESZ, int OSZ, int TM, int TN, int WM, int WN, int KS, int PF, int AD>
__global__ void __launch_bounds__(WM *WN * 64, 1) pe_fwd16_kernel(const FwdArgs a) {
    constexpr int NT = WM * WN * 64;
    constexpr int BM = WM * TM * 16;
    constexpr int BN = WN * TN * 16;
    constexpr int S = num_steps(P, ESZ);
    constexpr int SF = full_steps(P, ESZ);
    constexpr int NSPLIT = split_frags(P, ESZ);
    constexpr int STAGE = BN * 64;              // packed-weight bytes of one k-step
    constexpr int CH = (STAGE / 16 + NT - 1) / NT;  // 16-byte chunks per thread per k-step
    constexpr bool CH_EVEN = (STAGE / 16) % NT == 0;
    constexpr int FIRST = split_first(P, ESZ);  // elements in the first piece of a split fragment
    // epilogue staging: one 16-row block of a wave's tile, fp32; a row pitch of 4 mod 16 dwords
    // puts the four lane groups (rows 4 apart) on disjoint banks
    constexpr int EP_PITCH = TN * 16 + 4;       // dwords
    constexpr int EP_WAVE = 16 * EP_PITCH * 4;  // bytes per wave
    constexpr int KBUF = KS * STAGE;            // one LDS buffer: KS k-steps of packed weight
    constexpr int LDS_BYTES = (2 * KBUF > EP_WAVE * WM * WN) ? 2 * KBUF : EP_WAVE * WM * WN;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    // ---- tile: blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous run of
    // tiles so the tiles that share rows (same tm) run on one XCD, close in time.
    const int G = a.tiles_m * a.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, loc = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    // row-major runs share rows (A) within an XCD; column-major runs share weight columns, for
    // launches whose input is smaller than the weight
    const int tm = a.colmajor ? L % a.tiles_m : L / a.tiles_n;
    const int tn = a.colmajor ? L / a.tiles_m : L % a.tiles_n;
    const int row0 = tm * BM, col0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;
    const int g = lane >> 4, l16 = lane & 15;
    const int ncb = a.E >> 4;

    PatchRef pr[TM];
#pragma unroll
    for (int rb = 0; rb < TM; ++rb) pr[rb] = patch_of_row<P>(a, row0 + (wm * TM + rb) * 16 + l16);

    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.in), (short)0, (int)a.in_bytes, kBufWord3);

    auto elem_off = [&](const PatchRef &p, int r, int x) -> uint32_t {
        const int tt = r / (kC * P), c = (r / P) % kC, py = r % P;
        return p.base + (tt ? p.tstr : 0u) + (uint32_t)c * p.plane + (uint32_t)py * p.rstr + (uint32_t)x;
    };

    // A fragments of k-step s for this lane's TM rows (no use of the data here: the loads stay
    // in flight until the step's matrix products).
    auto load_a = [&](auto sc, u32x4 (&dst)[TM]) {
        constexpr int s = decltype(sc)::value;
        const Piece pc = frag_piece(P, ESZ, s, g);
        if constexpr (s < SF) {
#pragma unroll
            for (int rb = 0; rb < TM; ++rb)
                dst[rb] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(elem_off(pr[rb], pc.r1, pc.x1) * ESZ), 0, 0);
        } else {
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                const int o1 = (int)(elem_off(pr[rb], pc.r1, pc.x1) * ESZ);
                const int o2 = (int)(elem_off(pr[rb], pc.r2, pc.x2) * ESZ);
                if constexpr (FIRST * ESZ == 12) {
                    const u32x3 m3 = __builtin_amdgcn_raw_buffer_load_b96(rsrc, o1, 0, 0);
                    const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b32(rsrc, o2, 0, 0);
                    dst[rb] = u32x4{m3.x, m3.y, m3.z, e1};
                } else {
                    static_assert(FIRST * ESZ == 8, "split fragments are 12+4 or 8+8 bytes");
                    const u32x2 m2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, o1, 0, 0);
                    const u32x2 e2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, o2, 0, 0);
                    dst[rb] = u32x4{m2.x, m2.y, e2.x, e2.y};
                }
            }
        }
    };

    // Packed weight of k-step s for the tile's columns: BN*64 contiguous bytes. Chunks past the
    // last column block (or past the stage) get an offset beyond the buffer range and read 0, so
    // the loads need no branches (branches would make the wait counts conservative).
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.wpk), (short)0, (int)((uint32_t)S * (uint32_t)packed_cols(a.E, ESZ) * 64u), kBufWord3);
    uint32_t boff[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = c * NT + tid;
        const bool ok = (CH_EVEN || idx < STAGE / 16) && (col0 >> 4) + (idx >> 6) < ncb;
        boff[c] = ok ? ((uint32_t)(col0 >> 4) * 1024u + (uint32_t)idx * 16u) : 0x80000000u;
    }
    auto load_b = [&](int s, u32x4 (&dst)[CH]) {
        const uint32_t soff = (uint32_t)s * (uint32_t)ncb * 1024u;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            dst[c] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(boff[c] + soff), 0, 0);
    };
    // LDS position of k-step s: buffer (s / KS) & 1, slot s % KS
    auto store_b = [&](int s, const u32x4 (&src)[CH]) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(lds + ((s / KS) & 1) * KBUF + (s % KS) * STAGE);
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (CH_EVEN || c * NT + tid < STAGE / 16) dst[c * NT + tid] = src[c];
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](auto sc, const u32x4 (&af_in)[TM]) {
        constexpr int s = decltype(sc)::value;
        u32x4 af[TM];
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) af[rb] = af_in[rb];
        if constexpr (s >= SF && 4 * (s - SF) + 4 > NSPLIT) {
            // the last split step holds zero (padding) fragments in its top lane groups
            const bool pad = 4 * (s - SF) + g >= NSPLIT;
#pragma unroll
            for (int rb = 0; rb < TM; ++rb)
                if (pad) af[rb] = u32x4{0u, 0u, 0u, 0u};
        }
        const u32x4 *bs = reinterpret_cast<const u32x4 *>(lds + ((s / KS) & 1) * KBUF + (s % KS) * STAGE) +
                          wn * TN * 64 + lane;
        // weight fragments are read PF column blocks ahead of their matrix products
        u32x4 bq[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) bq[i] = bs[(i < TN ? i : 0) * 64];
#pragma unroll
        for (int cb = 0; cb < TN; ++cb) {
            const u32x4 bf = bq[cb % PF];
            if (cb + PF < TN) bq[cb % PF] = bs[(cb + PF) * 64];
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                if constexpr (ESZ == 2) {
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[rb]), __builtin_bit_cast(bf16x8, bf), acc[rb][cb], 0, 0, 0);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // copy the element out first: bit-casting an ext-vector element lvalue
                        // directly reads element 0
                        const uint32_t ai = af[rb][i], bi = bf[i];
                        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            __builtin_bit_cast(float, ai), __builtin_bit_cast(float, bi), acc[rb][cb], 0, 0, 0);
                    }
                }
            }
        }
    };

    // ---- k loop, fully unrolled. A runs AD k-steps ahead in an (AD+1)-deep register ring. The packed
    // weight sits in two LDS buffers of KS k-steps each (one barrier per KS k-steps); while the
    // waves compute from one buffer they fill the other, one k-step at a time, from a 2-deep
    // register ring loaded one k-step before it is stored.
    u32x4 Ar[AD + 1][TM], Br[2][CH];
    {
        u32x4 tmp[CH];
#pragma unroll
        for (int j = 0; j < (KS < S ? KS : S); ++j) {
            load_b(j, tmp);
            store_b(j, tmp);
        }
    }
    if constexpr (KS < S) load_b(KS, Br[KS & 1]);
    static_for<(AD < S ? AD : S)>([&](auto jc) { load_a(jc, Ar[decltype(jc)::value]); });
    __syncthreads();
    static_for<S>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int t = s + KS;            // the weight k-step this step moves to LDS
        if constexpr (t + 1 < S) load_b(t + 1, Br[(t + 1) & 1]);
        if constexpr (s + AD < S) load_a(IC<s + AD>{}, Ar[(s + AD) % (AD + 1)]);
        compute(sc, Ar[s % (AD + 1)]);
        if constexpr (t < S) store_b(t, Br[t & 1]);
        if constexpr (s % KS == KS - 1 && s + 1 < S) __syncthreads();
        // keep each step's instructions inside the step: bounds register live ranges
        __builtin_amdgcn_sched_barrier(0);
    });

    // ---- epilogue: + bias (fp32), one RNE cast, 16-byte row-contiguous stores. Each wave
    // stages one 16-row block of its tile at a time through its own LDS region.
    __syncthreads();  // every wave is done reading the weight stages
    float *ep = reinterpret_cast<float *>(lds + wave * EP_WAVE);
    float bv[TN];
#pragma unroll
    for (int cb = 0; cb < TN; ++cb) {
        const int col = col0 + (wn * TN + cb) * 16 + l16;
        bv[cb] = (a.bias && col < a.E) ? a.bias[col] : 0.f;
    }
    constexpr int VPC = 16 / OSZ;                 // output values per 16-byte chunk
    constexpr int CHUNKS = 16 * TN * 16 / VPC;    // chunks in a 16-row block
    const int wcol0 = col0 + wn * TN * 16;
#pragma unroll
    for (int rb = 0; rb < TM; ++rb) {
#pragma unroll
        for (int cb = 0; cb < TN; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ep[(4 * g + i) * EP_PITCH + cb * 16 + l16] = acc[rb][cb][i] + bv[cb];
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's writes are in LDS
        __builtin_amdgcn_wave_barrier();
        const int rbase = row0 + (wm * TM + rb) * 16;
#pragma unroll
        for (int j = 0; j < (CHUNKS + 63) / 64; ++j) {
            const int c = j * 64 + lane;
            if (CHUNKS % 64 != 0 && c >= CHUNKS) break;
            const int r = c / (TN * 16 / VPC), q = c % (TN * 16 / VPC);
            const float *src = ep + r * EP_PITCH + q * VPC;
            const int row = rbase + r, col = wcol0 + q * VPC;
            if (row < a.n_rows && col < a.E) {
                float v[VPC];
#pragma unroll
                for (int e = 0; e < VPC; ++e) v[e] = src[e];
                store_chunk<OSZ>(a.out, a.addend, (int64_t)row * a.E + col, v);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    }
}

// ----------------------------------------------------------------------------------------
// bf16 forward kernel: 32x32x16 matrix-core blocks (see the file header)
// ----------------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int P, int ISZ, int OSZ, int TM, int TN, int WM, int WN, int KS, int PF, int AD, int BD, int AM, bool MG>
__global__ void __launch_bounds__(WM *WN * 64, 1) pe_fwd32_kernel(const FwdArgs a) {
    constexpr int ESZ = 2;
    constexpr int NT = WM * WN * 64;
    constexpr int BM = WM * TM * 32;
    constexpr int BN = WN * TN * 32;
    constexpr int S = a_steps<P, AM>();
    constexpr int STAGE = BN * 64;                  // packed-weight bytes of one k-step
    constexpr int CH = (STAGE / 16 + NT - 1) / NT;  // 16-byte chunks per thread per k-step
    constexpr bool CH_EVEN = (STAGE / 16) % NT == 0;
    // epilogue staging: 16 rows of a wave's tile at a time, fp32; a pitch of 8 mod 16 dwords
    // puts the two lane halves (rows 4 apart) on disjoint banks
    constexpr int EP_PITCH = TN * 32 + 8;           // dwords
    constexpr int EP_WAVE = 16 * EP_PITCH * 4;      // bytes per wave
    constexpr int KBUF = KS * STAGE;
    // Patch rows stage A through LDS as well: each row's k-steps are 128-byte pieces of one
    // contiguous row, loaded by consecutive threads (eight rows per load instruction, every
    // cache line fetched whole) into two LDS stages of BM rows (pitch 144 bytes: the 16 lanes of
    // a 16-byte read land on distinct banks), and read back as the matrix-core fragments.
    constexpr bool AST = AM == kARows;
    static_assert(!AST || KS == 1, "patch rows: one weight k-step per LDS buffer");
    constexpr int AC = ISZ == 2 ? 2 : 1;           // k-steps per 128-byte A piece
    constexpr int NCH = (S + AC - 1) / AC;         // A pieces per row
    constexpr int APITCH = 144;
    constexpr int ASTAGE = BM * APITCH;
    constexpr int AL = BM * 8 / NT;                // 16-byte A loads per thread per piece
    static_assert(!AST || (BM * 8) % NT == 0, "A piece loads");
    constexpr int AOFF = 2 * KBUF;                 // A stages after the weight buffers
    constexpr int MAIN_BYTES = 2 * KBUF + (AST ? 2 * ASTAGE : 0);
    constexpr int LDS_BYTES = (MAIN_BYTES > EP_WAVE * WM * WN) ? MAIN_BYTES : EP_WAVE * WM * WN;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    // ---- tile: blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous run of
    // tiles so the tiles that share rows (same tm) run on one XCD, close in time.
    const int G = a.tiles_m * a.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, loc = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    // row-major runs share rows (A) within an XCD; column-major runs share weight columns, for
    // launches whose input is smaller than the weight
    const int tm = a.colmajor ? L % a.tiles_m : L / a.tiles_n;
    const int tn = a.colmajor ? L / a.tiles_m : L % a.tiles_n;
    const int row0 = tm * BM, col0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;
    const int h = lane >> 5, l32 = lane & 31;
    const int ncb = packed_cols(a.E, ESZ) >> 5;  // 32-column blocks of the packed weight

    // Per lane and 32-row block: byte offset of its patch's temporal slot h (the two lane halves
    // read the two frames of the temporal patch: tstr = 0 for a repeated image frame), or for
    // patch rows the row plus 8 elements for lanes 32-63. The per-step part of each address is the
    // same for every row of the launch (one frame geometry per launch), so it is a scalar offset
    // and the loads cost no vector arithmetic. Computed once the first weight k-step's loads are in
    // flight (they depend only on the tile's columns).
    uint32_t vb[TM], vpl[TM], vrs[TM];
    auto rows_setup = [&]() {
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) {
            const PatchRef p = patch_of_row<P>(a, row0 + (wm * TM + rb) * 32 + l32);
            vb[rb] = AM == kARows ? (p.base + (h ? 8u : 0u)) * (uint32_t)ISZ : (p.base + (h ? p.tstr : 0u)) * (uint32_t)ISZ;
            vpl[rb] = p.plane;
            vrs[rb] = p.rstr;
        }
    };

    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.in), (short)0, (int)a.in_bytes, kBufWord3);
    const uint32_t plane = a.plane, rstr = a.rstr;

    // A fragments of k-step s (sub-steps j = 0, 1). Loads only; the data is first used by the
    // step's matrix products.
    auto load_a = [&](auto sc, AFrag<ISZ> (&dst)[TM][2]) {
        load_a_step<P, TM, AM, ISZ, decltype(sc)::value, MG>(rsrc, vb, plane, rstr, h, dst, vpl, vrs);
    };

    // Patch rows: thread piece loads. Load i of a piece: row (i*NT + tid) / 8 of the tile, its
    // 16-byte part (i*NT + tid) % 8; rows past the end read row 0 of the launch (never stored).
    constexpr int KB = kC * kTp * P * P * ISZ;     // bytes of one patch row
    static_assert(KB % 16 == 0, "a 16-byte part lies wholly inside or outside the row");
    uint32_t av[AST ? AL : 1];
    int apart[AST ? AL : 1];
    if constexpr (AST) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int q = i * NT + tid, r = q >> 3;
            apart[i] = q & 7;
            const int row = row0 + r;
            av[i] = (row < a.n_rows ? (uint32_t)row * (uint32_t)KB : 0u) + (uint32_t)apart[i] * 16u;
        }
    }
    auto load_piece = [&](auto cc, u32x4 (&dst)[AST ? AL : 1]) {
        constexpr int c = decltype(cc)::value;
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            if constexpr (c * 128 + 128 > KB) {
                // the last piece: a part past the row loads the piece's part 0 (piece_load_part,
                // inside the row; the bytes past a row belong to the next row or lie past the
                // caller's buffer) and is zeroed
                const bool real = piece_part_real(KB, c, apart[i]);
                dst[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(real ? av[i] : av[i] - (uint32_t)apart[i] * 16u),
                                                               c * 128, 0);
                if (!real) dst[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                dst[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)av[i], c * 128, 0);
            }
        }
    };
    auto store_piece = [&](int c, const u32x4 (&src)[AST ? AL : 1]) {
        unsigned char *st = lds + AOFF + (c & 1) * ASTAGE;
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int q = i * NT + tid;
            *reinterpret_cast<u32x4 *>(st + (q >> 3) * APITCH + (q & 7) * 16) = src[i];
        }
    };
    // fragments of k-step s for this lane from the A stage: row (wm*TM + rb)*32 + l32, elements
    // 32*(s % AC)... of the piece: bytes (s % AC)*64 + (2j + h)*16*ISZ/2
    auto read_a = [&](int s, AFrag<ISZ> (&dst)[TM][2]) {
        const unsigned char *st = lds + AOFF + ((s / AC) & 1) * ASTAGE;
#pragma unroll
        for (int rb = 0; rb < TM; ++rb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const unsigned char *src = st + ((wm * TM + rb) * 32 + l32) * APITCH + (s % AC) * 64 + (2 * j + h) * 8 * ISZ;
#pragma unroll
                for (int d = 0; d < ISZ / 2; ++d) dst[rb][j].d[d] = *reinterpret_cast<const u32x4 *>(src + 16 * d);
            }
    };

    // Packed weight of k-step s for the tile's columns: BN*64 contiguous bytes. Chunks past the
    // last column block get an offset beyond the buffer range and read 0 (no branches: branches
    // would make the wait counts conservative).
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.wpk), (short)0, (int)((uint32_t)S * (uint32_t)ncb * 2048u), kBufWord3);
    uint32_t boff[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = c * NT + tid;
        const bool ok = (CH_EVEN || idx < STAGE / 16) && (col0 >> 5) + (idx >> 7) < ncb;
        boff[c] = ok ? ((uint32_t)(col0 >> 5) * 2048u + (uint32_t)idx * 16u) : 0x80000000u;
    }
    auto load_b = [&](int s, u32x4 (&dst)[CH]) {
        const uint32_t soff = (uint32_t)s * (uint32_t)ncb * 2048u;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            dst[c] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(boff[c] + soff), 0, 0);
    };
    auto store_b = [&](int s, const u32x4 (&src)[CH]) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(lds + ((s / KS) & 1) * KBUF + (s % KS) * STAGE);
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (CH_EVEN || c * NT + tid < STAGE / 16) dst[c * NT + tid] = src[c];
    };

    // accumulators start at the bias (fp32): out = bias + sum of products
    f32x16 acc[TM][TN];
#pragma unroll
    for (int cb = 0; cb < TN; ++cb) {
        const int col = col0 + (wn * TN + cb) * 32 + l32;
        const float bv = (a.bias && col < a.E) ? a.bias[col] : 0.f;
        f32x16 b16;
#pragma unroll
        for (int i = 0; i < 16; ++i) b16[i] = bv;
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) acc[rb][cb] = b16;
    }

    auto compute = [&](auto sc, const AFrag<ISZ> (&ald_regs)[TM][2]) {
        constexpr int s = decltype(sc)::value;
        AFrag<ISZ> ald_lds[TM][2];
        if constexpr (AST) read_a(s, ald_lds);
        const AFrag<ISZ>(&ald)[TM][2] = AST ? ald_lds : ald_regs;
        u32x4 af[TM][2];
        a_operands<P, TM, AM, ISZ, s>(ald, af, h);
        // fragment (j, cb) of this step: 1 KB at stage + (wn*TN + cb)*2 KB + j*1 KB
        const u32x4 *bs = reinterpret_cast<const u32x4 *>(lds + ((s / KS) & 1) * KBUF + (s % KS) * STAGE) +
                          wn * TN * 128 + lane;
        constexpr int NF = 2 * TN;
        u32x4 bq[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int f = i < NF ? i : 0;
            bq[i] = bs[(f % TN) * 128 + (f / TN) * 64];
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int j = f / TN, cb = f % TN;
            const u32x4 bf = bq[f % PF];
            if (f + PF < NF) bq[f % PF] = bs[((f + PF) % TN) * 128 + ((f + PF) / TN) * 64];
#pragma unroll
            for (int rb = 0; rb < TM; ++rb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, af[rb][j]), __builtin_bit_cast(bf16x8, bf), acc[rb][cb], 0, 0, 0);
        }
        // Pin the interleave: PF fragment reads first, then per fragment its TM products and the
        // read PF fragments ahead (left alone, the scheduler sinks each read next to its use).
        __builtin_amdgcn_sched_group_barrier(0x100, (PF < NF ? PF : NF) + (AST ? TM * 2 * (ISZ / 2) : 0), 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x008, TM, 0);
            if (f + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    // ---- k loop, fully unrolled. A runs AD k-steps ahead in a register ring. Patch rows load
    // A two k-steps at a time (the 128 bytes of each row that two k-steps read are one cache
    // line, fetched once). The packed weight sits in two LDS buffers of KS k-steps each (one
    // barrier per KS k-steps); while the waves compute from one buffer they fill the other one
    // k-step at a time from a BD-deep register ring (each weight k-step is loaded BD-1 k-steps
    // before it is stored).
    // Patch rows: A piece c (k-steps AC*c ..) is loaded at k-step AC*c - 3 and stored into stage
    // c & 1 at the end of k-step AC*c - 1 (its barrier publishes it); at most three pieces are in
    // registers at once.
    constexpr int RD = AST ? 1 : AD + 1;                 // A ring depth (frames)
    constexpr int PRE = AST ? 0 : AD;                    // A k-steps loaded before the loop (frames)
    AFrag<ISZ> Ar[RD][TM][2];
    u32x4 Apc[AST ? 3 : 1][AST ? AL : 1];
    u32x4 Br[BD][CH];
    if constexpr (AST) {
        load_piece(IC<0>{}, Apc[0]);
        store_piece(0, Apc[0]);
        static_for<NCH>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            if constexpr (c >= 1 && AC * c - 3 < 0) load_piece(cc, Apc[c % 3]);
        });
    }
    {
        u32x4 tmp[CH];
#pragma unroll
        for (int j = 0; j < (KS < S ? KS : S); ++j) {
            load_b(j, tmp);
            if (j == 0 && !AST) rows_setup();
            store_b(j, tmp);
        }
    }
    static_for<BD - 1>([&](auto ic) {
        constexpr int t = KS + decltype(ic)::value;
        if constexpr (t < S) load_b(t, Br[t % BD]);
    });
    static_for<(PRE < S ? PRE : S)>([&](auto jc) { load_a(jc, Ar[decltype(jc)::value]); });
    __syncthreads();
    static_for<S>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int t = s + KS;
        if constexpr (t + BD - 1 < S) load_b(t + BD - 1, Br[(t + BD - 1) % BD]);
        if constexpr (AST) {
            // piece c with AC*c - 3 == s
            if constexpr ((s + 3) % AC == 0 && (s + 3) / AC < NCH && (s + 3) / AC >= 1)
                load_piece(IC<(s + 3) / AC>{}, Apc[((s + 3) / AC) % 3]);
        } else if constexpr (s + AD < S) {
            load_a(IC<s + AD>{}, Ar[(s + AD) % RD]);
        }
        compute(sc, Ar[s % RD]);
        if constexpr (t < S) store_b(t, Br[t % BD]);
        if constexpr (AST) {
            // piece c with AC*c - 1 == s
            if constexpr ((s + 1) % AC == 0 && (s + 1) / AC < NCH) store_piece((s + 1) / AC, Apc[((s + 1) / AC) % 3]);
        }
        if constexpr (s % KS == KS - 1 && s + 1 < S) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    });

    // ---- epilogue: one RNE cast, 16-byte row-contiguous non-temporal stores (the output is
    // not read again here; keeping it out of L2 leaves room for the weight). Lane l holds column l % 32
    // and, in accumulator element i, row 8*(i/4) + 4*(l/32) + i%4 of its block.
    __syncthreads();
    float *ep = reinterpret_cast<float *>(lds + wave * EP_WAVE);
    constexpr int VPC = 16 / OSZ;                 // output values per 16-byte chunk
    constexpr int RCH = TN * 32 / VPC;            // chunks per row
    constexpr int CHUNKS = 16 * RCH;              // chunks in 16 rows
    const int wcol0 = col0 + wn * TN * 32;
    // A fused bf16 addend is read one 16-row block ahead, so its latency overlaps the staging and
    // the stores of the block before; an fp32 one (twice the registers) is read at the start of its
    // own block and overlaps that block's staging. Chunks outside the output read the addend's
    // first chunk.
    constexpr int CPL = (CHUNKS + 63) / 64;       // chunks per lane in 16 rows
    constexpr int NBLK = 2 * TM;                  // 16-row blocks per wave
    constexpr int NBUF = OSZ == 2 ? 2 : 1;
    const bool has_add = a.addend != nullptr;
    auto add_load = [&](int it, u32x4 (&dst)[CPL]) {
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) {
            const int c = jj * 64 + lane;
            const int r = c / RCH, qq = c % RCH;
            const int row = row0 + (wm * TM + it / 2) * 32 + (it % 2) * 16 + r, col = wcol0 + qq * VPC;
            const bool ok = (CHUNKS % 64 == 0 || c < CHUNKS) && row < a.n_rows && col < a.E;
            dst[jj] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.addend) +
                                                       (ok ? ((int64_t)row * a.E + col) * OSZ : 0));
        }
    };
    u32x4 adq[NBUF][CPL];
    if (NBUF == 2 && has_add) add_load(0, adq[0]);
#pragma unroll
    for (int it = 0; it < NBLK; ++it) {
        const int rb = it / 2, half = it % 2;
        if (has_add) {
            if (NBUF == 1) add_load(it, adq[0]);
            else if (it + 1 < NBLK) add_load(it + 1, adq[(it + 1) % NBUF]);
        }
#pragma unroll
        for (int cb = 0; cb < TN; ++cb)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = half * 8 + q;
                const int rl = 8 * (q / 4) + 4 * h + (q % 4);   // row within these 16
                ep[rl * EP_PITCH + cb * 32 + l32] = acc[rb][cb][i];
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's writes are in LDS
        __builtin_amdgcn_wave_barrier();
        const int rbase = row0 + (wm * TM + rb) * 32 + half * 16;
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) {
            const int c = jj * 64 + lane;
            if (CHUNKS % 64 != 0 && c >= CHUNKS) break;
            const int r = c / RCH, qq = c % RCH;
            const float *src = ep + r * EP_PITCH + qq * VPC;
            const int row = rbase + r, col = wcol0 + qq * VPC;
            if (row < a.n_rows && col < a.E) {
                float v[VPC];
#pragma unroll
                for (int e = 0; e < VPC; ++e) v[e] = src[e];
                store_chunk_r<OSZ>(a.out, has_add, adq[it % NBUF][jj], (int64_t)row * a.E + col, v);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    }
}

// ----------------------------------------------------------------------------------------
// bf16 split-K kernel for few rows: the four waves of a workgroup share one BM x BN tile and
// each takes a contiguous quarter of the k-steps, so each wave's chain of dependent k-steps is a
// quarter as long. A wave's weight fragments are its own (no other wave uses that k range): they
// go from global memory straight to registers, with no LDS stage and no barrier in the k loop.
// The four fp32 partial tiles meet in LDS at the end and are summed in a fixed order.
// ----------------------------------------------------------------------------------------
template <int P, int ISZ, int OSZ, int TM, int TN, int AD, int AM, bool MG>
__global__ void __launch_bounds__(256, 1) pe_fwd32_sk_kernel(const FwdArgs a) {
    constexpr int NW = 4;
    constexpr int BM = TM * 32, BN = TN * 32;
    constexpr int S = a_steps<P, AM>();
    constexpr int PITCH = BN + 8;                   // dwords per partial-tile row (8 mod 16)
    constexpr int PART = BM * PITCH * 4;            // bytes per wave's partial tile
    __shared__ __attribute__((aligned(16))) unsigned char lds[NW * PART];

    const int G = a.tiles_m * a.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, loc = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    // row-major runs share rows (A) within an XCD; column-major runs share weight columns, for
    // launches whose input is smaller than the weight
    const int tm = a.colmajor ? L % a.tiles_m : L / a.tiles_n;
    const int tn = a.colmajor ? L / a.tiles_m : L % a.tiles_n;
    const int row0 = tm * BM, col0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int ncb = packed_cols(a.E, 2) >> 5;

    // per lane and 32-row block: the patch's byte offset (item lookup); filled once this wave's
    // first weight loads are in flight (they depend only on the tile's columns)
    uint32_t vb[TM], vpl[TM], vrs[TM];
    auto rows_setup = [&]() {
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) {
            const PatchRef p = patch_of_row<P>(a, row0 + rb * 32 + l32);
            vb[rb] = AM == kARows ? (p.base + (h ? 8u : 0u)) * (uint32_t)ISZ : (p.base + (h ? p.tstr : 0u)) * (uint32_t)ISZ;
            vpl[rb] = p.plane;
            vrs[rb] = p.rstr;
        }
    };
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.in), (short)0, (int)a.in_bytes, kBufWord3);
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.wpk), (short)0, (int)((uint32_t)S * (uint32_t)ncb * 2048u), kBufWord3);
    const uint32_t plane = a.plane, rstr = a.rstr;
    // weight fragment (s, j, cb): 1 KB at ((s*ncb + cb)*2 + j) KB; column blocks past E read 0
    uint32_t wb[TN];
#pragma unroll
    for (int cb = 0; cb < TN; ++cb)
        wb[cb] = ((col0 >> 5) + cb < ncb) ? ((uint32_t)((col0 >> 5) + cb) * 2048u + (uint32_t)lane * 16u) : 0x80000000u;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int cb = 0; cb < TN; ++cb) {
        const int col = col0 + cb * 32 + l32;
        const float bv = (wave == 0 && a.bias && col < a.E) ? a.bias[col] : 0.f;
        f32x16 b16;
#pragma unroll
        for (int i = 0; i < 16; ++i) b16[i] = bv;
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) acc[rb][cb] = b16;
    }

    struct Frags { AFrag<ISZ> a[TM][2]; u32x4 b[TN][2]; };
    auto load_b = [&](auto sc, Frags &d) {
        constexpr int s = decltype(sc)::value;
        static_for<2>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int sw = (int)(((uint32_t)s * (uint32_t)ncb * 2u + j) * 1024u);
#pragma unroll
            for (int cb = 0; cb < TN; ++cb) d.b[cb][j] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)wb[cb], sw, 0);
        });
    };
    auto load = [&](auto sc, Frags &d) {
        load_a_step<P, TM, AM, ISZ, decltype(sc)::value, MG>(rsrc, vb, plane, rstr, h, d.a, vpl, vrs);
        load_b(sc, d);
    };
    auto mma = [&](auto sc, const Frags &d) {
        u32x4 af[TM][2];
        a_operands<P, TM, AM, ISZ, decltype(sc)::value>(d.a, af, h);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int cb = 0; cb < TN; ++cb)
#pragma unroll
                for (int rb = 0; rb < TM; ++rb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, af[rb][j]), __builtin_bit_cast(bf16x8, d.b[cb][j]), acc[rb][cb], 0, 0, 0);
    };
    // wave W: k-steps [W*S/NW, (W+1)*S/NW), loads AD steps ahead in an (AD+1)-deep ring
    auto run = [&](auto wc) {
        constexpr int W = decltype(wc)::value;
        constexpr int lo = W * S / NW, hi = (W + 1) * S / NW, n = hi - lo;
        Frags ring[AD + 1];
        static_for<(AD < n ? AD : n)>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            load_b(IC<lo + i>{}, ring[i]);
        });
        rows_setup();
        static_for<(AD < n ? AD : n)>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            load_a_step<P, TM, AM, ISZ, lo + i, MG>(rsrc, vb, plane, rstr, h, ring[i].a, vpl, vrs);
        });
        static_for<n>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i + AD < n) load(IC<lo + i + AD>{}, ring[(i + AD) % (AD + 1)]);
            mma(IC<lo + i>{}, ring[i % (AD + 1)]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    switch (wave) {
        case 0: run(IC<0>{}); break;
        case 1: run(IC<1>{}); break;
        case 2: run(IC<2>{}); break;
        default: run(IC<3>{}); break;
    }

    // ---- partial tiles to LDS, then each wave sums BM/NW rows of the four partials (fixed
    // order), one RNE cast, 16-byte row-contiguous stores
    float *part = reinterpret_cast<float *>(lds + wave * PART);
#pragma unroll
    for (int rb = 0; rb < TM; ++rb)
#pragma unroll
        for (int cb = 0; cb < TN; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = rb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
                part[r * PITCH + cb * 32 + l32] = acc[rb][cb][i];
            }
    __syncthreads();
    constexpr int VPC = 16 / OSZ;                   // output values per 16-byte chunk
    constexpr int RCH = BN / VPC;                   // chunks per row
    constexpr int ROWS = BM / NW;                   // rows per wave
    constexpr int CHUNKS = ROWS * RCH;
    const float *p0 = reinterpret_cast<const float *>(lds);
#pragma unroll
    for (int jj = 0; jj < (CHUNKS + 63) / 64; ++jj) {
        const int c = jj * 64 + lane;
        if (CHUNKS % 64 != 0 && c >= CHUNKS) break;
        const int r = wave * ROWS + c / RCH, q = c % RCH;
        const int row = row0 + r, col = col0 + q * VPC;
        if (row < a.n_rows && col < a.E) {
            float v[VPC];
#pragma unroll
            for (int e4 = 0; e4 < VPC; e4 += 4) {
                f32x4 t = *reinterpret_cast<const f32x4 *>(p0 + r * PITCH + q * VPC + e4);
#pragma unroll
                for (int w = 1; w < NW; ++w)
                    t += *reinterpret_cast<const f32x4 *>(p0 + w * (PART / 4) + r * PITCH + q * VPC + e4);
                v[e4] = t.x; v[e4 + 1] = t.y; v[e4 + 2] = t.z; v[e4 + 3] = t.w;
            }
            store_chunk<OSZ>(a.out, a.addend, (int64_t)row * a.E + col, v);
        }
    }
}

// ----------------------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------------------
template <int P, int ESZ, int OSZ, int TM, int TN, int WM, int WN, int KS, int PF, int AD>
inline hipError_t launch16(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
    hipLaunchKernelGGL((pe_fwd16_kernel<P, ESZ, OSZ, TM, TN, WM, WN, KS, PF, AD>), dim3(a.tiles_m * a.tiles_n),
                       dim3(WM * WN * 64), 0, st, a);
    return hipGetLastError();
}

template <int P, int ISZ, int OSZ, int TM, int TN, int WM, int WN, int KS, int PF, int AD, int BD>
inline hipError_t launch32(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
    const dim3 grid(a.tiles_m * a.tiles_n), block(WM * WN * 64);
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

template <int P, int ISZ, int OSZ, int TM, int TN, int AD>
inline hipError_t launch_sk(const FwdArgs &a, hipStream_t st) {
    constexpr int BM = TM * 32, BN = TN * 32;
    if (a.tiles_m != (a.n_rows + BM - 1) / BM || a.tiles_n != (a.E + BN - 1) / BN) return hipErrorInvalidValue;
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
        // fp32 I/O: 16x16 blocks, small tiles (its fully unrolled k loop has 74 steps); 32 x 160
        // tiles where E allows (1024 x 1280 makes 256 of them: one round, where 32 x 128 tiles
        // take 1.25; measured 38 us against 45-47 us), one weight k-step per LDS buffer
        if (a.tiles != kTileF32) return hipErrorInvalidValue;
        if (skn == 160) return launch16<P, ESZ, OSZ, 1, 5, 2, 2, 1, 2, 2>(a, st);
        return launch16<P, ESZ, OSZ, 1, 4, 2, 2, 2, 2, 2>(a, st);
    } else {
        // 8 waves of 32 x BN (two per SIMD), one weight k-step per LDS buffer (a barrier per k-step
        // measured ~2% faster than two), eight weight fragments read ahead
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
