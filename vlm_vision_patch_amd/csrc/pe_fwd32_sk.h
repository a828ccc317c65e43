// pe_fwd32_sk.h -- bf16 split-k forward kernel for few rows (see pe_kernels.h).
#pragma once

#include "pe_gather.h"

namespace pe {

// bf16 split-K kernel for few rows: the four waves of a workgroup share one BM x BN tile and
// each takes a contiguous quarter of the k-steps, so each wave's chain of dependent k-steps is a
// quarter as long. A wave's weight fragments are its own (no other wave uses that k range): they
// go from global memory straight to registers, with no LDS stage and no barrier in the k loop.
// The four fp32 partial tiles meet in LDS at the end and are summed in a fixed order.
template <int P, int ISZ, int OSZ, int TM, int TN, int AD, int AM, bool MG>
__global__ void __launch_bounds__(256, 1) pe_fwd32_sk_kernel(const FwdArgs a) {
    constexpr int NW = 4;
    constexpr int BM = TM * 32, BN = TN * 32;
    constexpr int S = a_steps<P, AM>();
    constexpr int PITCH = BN + 8;                   // dwords per partial-tile row (8 mod 16)
    constexpr int PART = BM * PITCH * 4;            // bytes per wave's partial tile
    __shared__ __attribute__((aligned(16))) unsigned char lds[NW * PART];
    lds_sentinel_fill<NW * PART, NW * 64>(lds);

    const TileIdx tile = xcd_tile(a);   // XCD-aware tile order (pe_gather.h)
    const int row0 = tile.tm * BM, col0 = tile.tn * BN;

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
    sum_partials_store<OSZ, BM, BN, NW, PITCH, PART>(lds, a, row0, col0, wave, lane, nullptr);
}

}  // namespace pe
