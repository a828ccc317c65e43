// pe_device.h -- device helpers shared by the gfx950 kernels: 16-byte vector types, the raw
// buffer descriptor word, the LDS sentinel fill of the debug build, bf16 rounding, the output
// stores (with the optional fused addend), the XCD-aware tile order, the split-k epilogue and a
// compile-time loop.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));

// gfx9 buffer descriptor word 3: 32-bit data format, raw (untyped) access.
constexpr int kBufWord3 = 0x00020000;

// LDS sentinel debug build (compiled with -DPE_LDS_SENTINEL=1 into libpe_sentinel.so; the shipped
// libpe.so has it off and its machine code does not change): every kernel that uses LDS first
// fills all of it with all-ones bytes, which are NaN as bf16 and as fp32, and waits at a barrier.
// LDS keeps whatever an earlier workgroup left there, so a read of a slot that this workgroup
// has not written yet (a missing write, or a read that runs ahead of its write) would otherwise
// give a stale finite value; with the fill it puts a NaN into the output, which the parity
// checks catch.
#ifndef PE_LDS_SENTINEL
#define PE_LDS_SENTINEL 0
#endif
template <int BYTES, int NT>
__device__ __forceinline__ void lds_sentinel_fill(unsigned char *lds) {
    if constexpr (PE_LDS_SENTINEL != 0) {
        static_assert(BYTES % 16 == 0, "the fill writes 16-byte chunks");
        for (int i = (int)threadIdx.x; i < BYTES / 16; i += NT)
            reinterpret_cast<u32x4 *>(lds)[i] = u32x4{~0u, ~0u, ~0u, ~0u};
        __syncthreads();
    }
}

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

// Tile of workgroup blockIdx.x: blocks are dealt to the 8 XCDs round-robin, so each XCD gets a
// contiguous run of the launch's tiles. Row-major runs (row tiles outermost) keep the column
// tiles that share a row tile's pixels on one XCD, close in time; column-major runs (a.colmajor,
// for launches whose input is smaller than the weight) keep tiles that share weight columns
// together instead.
struct TileIdx { int tm, tn; };
__device__ __forceinline__ TileIdx xcd_tile(const FwdArgs &a) {
    const int G = a.tiles_m * a.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, loc = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    return TileIdx{a.colmajor ? L % a.tiles_m : L / a.tiles_n, a.colmajor ? L / a.tiles_m : L % a.tiles_n};
}

// Split-k epilogue: each of the NW waves left a BM x BN fp32 partial tile in LDS (wave w's at
// byte w*PART, rows PITCH dwords apart). Wave `wave` sums rows [wave*BM/NW, (wave+1)*BM/NW) of
// the NW partials in a fixed order (deterministic), adds `bias` (fp32 [E]) when it is given, and
// stores 16-byte row-contiguous chunks: one RNE cast, the fused addend (if any) added first.
template <int OSZ, int BM, int BN, int NW, int PITCH, int PART>
__device__ __forceinline__ void sum_partials_store(const unsigned char *lds, const FwdArgs &a, int row0, int col0,
                                                   int wave, int lane, const float *bias) {
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
            if (bias) {
#pragma unroll
                for (int e = 0; e < VPC; ++e) v[e] += bias[col + e];
            }
            store_chunk<OSZ>(a.out, a.addend, (int64_t)row * a.E + col, v);
        }
    }
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

}  // namespace pe
