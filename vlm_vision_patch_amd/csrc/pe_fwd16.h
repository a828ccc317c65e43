// pe_fwd16.h -- fp32 forward kernel: 16x16 blocks of v_mfma_f32_16x16x4_f32, split-k over the
// four waves of a workgroup (see pe_kernels.h).
#pragma once

#include "pe_gather.h"

namespace pe {

// fp32 weight (and fp32 input): fp32 products, 4-element fragments (frag_piece). The four waves
// of a workgroup share one BM x BN tile (TM x TN blocks of 16 x 16) and each takes a contiguous
// quarter of the k-steps. A wave loads its own weight fragments from global memory straight into
// registers (the packed weight of one k-step and 16-column block is the 1 KB its 64 lanes read),
// so the k loop has no LDS stage and no barrier, and each SIMD runs one wave whose products, 20
// independent accumulators per k-step for a 32 x 160 tile, keep the matrix pipe fed. The four
// fp32 partial tiles meet in LDS at the end and are summed in a fixed order (deterministic).
template <int P, int ESZ, int OSZ, int TM, int TN, int AD>
__global__ void __launch_bounds__(256, 1) pe_fwd16_kernel(const FwdArgs a) {
    static_assert(ESZ == 4, "the fp32 kernel takes an fp32 weight");
    constexpr int NW = 4;
    constexpr int BM = TM * 16, BN = TN * 16;
    constexpr int S = num_steps(P, ESZ);
    constexpr int SF = full_steps(P, ESZ);
    constexpr int NSPLIT = split_frags(P, ESZ);
    constexpr int FIRST = split_first(P, ESZ);  // elements in the first piece of a split fragment
    // partial tiles: a row pitch of 4 mod 16 dwords puts the four lane groups (rows 4 apart) on
    // disjoint banks
    constexpr int PITCH = BN + 4;               // dwords
    constexpr int PART = BM * PITCH * 4;        // bytes per wave's partial tile
    __shared__ __attribute__((aligned(16))) unsigned char lds[NW * PART];
    lds_sentinel_fill<NW * PART, NW * 64>(lds);

    const TileIdx tile = xcd_tile(a);   // XCD-aware tile order (pe_gather.h)
    const int row0 = tile.tm * BM, col0 = tile.tn * BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int ncb = a.E >> 4;   // 16-column blocks (E % 16 == 0)

    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.in), (short)0, (int)a.in_bytes, kBufWord3);
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.wpk), (short)0, (int)((uint32_t)S * (uint32_t)packed_cols(a.E, ESZ) * 64u), kBufWord3);
    // weight fragment (s, cb): 1 KB at (s*ncb + cb) KB, this lane's 16 bytes at lane*16; column
    // blocks past E get an offset beyond the buffer range and read 0 (no branches)
    uint32_t wb[TN];
#pragma unroll
    for (int cb = 0; cb < TN; ++cb)
        wb[cb] = ((col0 >> 4) + cb < ncb) ? ((uint32_t)((col0 >> 4) + cb) * 1024u + (uint32_t)lane * 16u) : 0x80000000u;

    // per lane and 16-row block: the patch (item lookup)
    PatchRef pr[TM];
#pragma unroll
    for (int rb = 0; rb < TM; ++rb) pr[rb] = patch_of_row<P>(a, row0 + rb * 16 + l16);
    auto elem_off = [&](const PatchRef &p, int r, int x) -> uint32_t {
        const int tt = r / (kC * P), c = (r / P) % kC, py = r % P;
        return p.base + (tt ? p.tstr : 0u) + (uint32_t)c * p.plane + (uint32_t)py * p.rstr + (uint32_t)x;
    };

    struct Frags { u32x4 a[TM]; u32x4 b[TN]; };
    auto load_b = [&](auto sc, Frags &d) {
        constexpr int s = decltype(sc)::value;
        const int sw = (int)((uint32_t)s * (uint32_t)ncb * 1024u);
#pragma unroll
        for (int cb = 0; cb < TN; ++cb) d.b[cb] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)wb[cb], sw, 0);
    };
    // A fragment of k-step s for this lane's TM rows: lane group g takes fragment frag_piece(s, g)
    auto load_a = [&](auto sc, Frags &d) {
        constexpr int s = decltype(sc)::value;
        const Piece pc = frag_piece(P, ESZ, s, g);
        if constexpr (s < SF) {
#pragma unroll
            for (int rb = 0; rb < TM; ++rb)
                d.a[rb] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(elem_off(pr[rb], pc.r1, pc.x1) * ESZ), 0, 0);
        } else {
            // split fragments; in the last step the top lane groups hold padding: their pieces
            // point at the patch's first elements (inside the patch) and are zeroed where the
            // products use them
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                const int o1 = (int)(elem_off(pr[rb], pc.r1, pc.x1) * ESZ);
                const int o2 = (int)(elem_off(pr[rb], pc.r2, pc.x2) * ESZ);
                if constexpr (FIRST * ESZ == 12) {
                    const u32x3 m3 = __builtin_amdgcn_raw_buffer_load_b96(rsrc, o1, 0, 0);
                    const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b32(rsrc, o2, 0, 0);
                    d.a[rb] = u32x4{m3.x, m3.y, m3.z, e1};
                } else {
                    static_assert(FIRST * ESZ == 8, "split fragments are 12+4 or 8+8 bytes");
                    const u32x2 m2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, o1, 0, 0);
                    const u32x2 e2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, o2, 0, 0);
                    d.a[rb] = u32x4{m2.x, m2.y, e2.x, e2.y};
                }
            }
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int rb = 0; rb < TM; ++rb)
#pragma unroll
        for (int cb = 0; cb < TN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mma = [&](auto sc, const Frags &d) {
        constexpr int s = decltype(sc)::value;
        u32x4 af[TM];
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) af[rb] = d.a[rb];
        if constexpr (s >= SF && 4 * (s - SF) + 4 > NSPLIT) {
            // padding fragments (frag_piece kind kPad) loaded real pixels; zero them so that no
            // pixel meets the zero weight (a non-finite one would make NaN)
            const bool pad = 4 * (s - SF) + g >= NSPLIT;
#pragma unroll
            for (int rb = 0; rb < TM; ++rb)
                if (pad) af[rb] = u32x4{0u, 0u, 0u, 0u};
        }
        // element i of every fragment first, so consecutive products use different accumulators
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int cb = 0; cb < TN; ++cb)
#pragma unroll
                for (int rb = 0; rb < TM; ++rb) {
                    // copy the elements out first: bit-casting an ext-vector element lvalue
                    // directly reads element 0
                    const uint32_t ai = af[rb][i], bi = d.b[cb][i];
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        __builtin_bit_cast(float, ai), __builtin_bit_cast(float, bi), acc[rb][cb], 0, 0, 0);
                }
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
        static_for<(AD < n ? AD : n)>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            load_a(IC<lo + i>{}, ring[i]);
        });
        static_for<n>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i + AD < n) {
                load_b(IC<lo + i + AD>{}, ring[(i + AD) % (AD + 1)]);
                load_a(IC<lo + i + AD>{}, ring[(i + AD) % (AD + 1)]);
            }
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

    // ---- partial tiles to LDS (lane (g, l16) of block (rb, cb) holds rows 4g..4g+3, column l16),
    // then each wave sums BM/NW rows of the four partials (fixed order), adds the bias, one RNE
    // cast, 16-byte row-contiguous stores
    float *part = reinterpret_cast<float *>(lds + wave * PART);
#pragma unroll
    for (int rb = 0; rb < TM; ++rb)
#pragma unroll
        for (int cb = 0; cb < TN; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[(rb * 16 + 4 * g + i) * PITCH + cb * 16 + l16] = acc[rb][cb][i];
    __syncthreads();
    sum_partials_store<OSZ, BM, BN, NW, PITCH, PART>(lds, a, row0, col0, wave, lane, a.bias);
}

}  // namespace pe
