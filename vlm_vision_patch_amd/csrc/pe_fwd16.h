// pe_fwd16.h -- fp32 forward kernel: 16x16 blocks of v_mfma_f32_16x16x4_f32 (see pe_kernels.h).
#pragma once

#include "pe_gather.h"

namespace pe {

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
    lds_sentinel_fill<LDS_BYTES, NT>(lds);

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

}  // namespace pe
