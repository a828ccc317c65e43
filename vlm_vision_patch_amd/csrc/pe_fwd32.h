// pe_fwd32.h -- bf16 forward kernel: 32x32x16 matrix-core blocks, the weight staged in LDS
// (see pe_kernels.h).
#pragma once

#include "pe_gather.h"

namespace pe {

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
    // Single images, P = 14 (AM == kAStaged): the tile's pixel rows are staged through LDS in the
    // grouped fragment order (pe_internal.h), 8 pixel rows (7 k-steps) per group, two group
    // buffers of BM patches. Wave w stages the 32-row slice w of the tile: a pixel row of its 32
    // patches is one load instruction, 16 bytes per lane, the 28 bytes of each patch in two lanes,
    // so the wave's bytes are contiguous runs of the image row (whole cache lines) instead of 16
    // bytes at a 28-byte stride per fragment. Shared A lets a wave take 64 rows (TM = 2) and half
    // the weight fragments per product. A row is written at least two k-steps before the first
    // read of it (the per-step barrier in between publishes it) and into a group buffer only
    // after the last read of the group it held. Patch pitch 240 bytes (14 fragments + 16): the 16
    // lanes of a 16-byte read land on distinct banks. Opt-in (pe_config.stage_images): on gfx950
    // these whole-row loads take more texture-data cycles per byte than the register gather's,
    // and the path measured 3-20 % slower.
    constexpr bool SG = AM == kAStaged;
    static_assert(!SG || (P == 14 && ISZ == 2 && S == 37 && BM == 32 * WM * WN && KS == 1 && !MG),
                  "LDS-staged images: bf16, P = 14, one frame geometry, one 32-row slice per wave, a barrier per k-step");
    constexpr int SG_PITCH = 240;
    constexpr int SG_BLOCK = BM * SG_PITCH;        // one group of the tile's patches
    constexpr int SGOFF = 2 * KBUF;                // after the weight buffers
    constexpr int MAIN_BYTES = 2 * KBUF + (AST ? 2 * ASTAGE : 0) + (SG ? 2 * SG_BLOCK : 0);
    constexpr int LDS_BYTES = (MAIN_BYTES > EP_WAVE * WM * WN) ? MAIN_BYTES : EP_WAVE * WM * WN;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    lds_sentinel_fill<LDS_BYTES, NT>(lds);

    const TileIdx tile = xcd_tile(a);   // XCD-aware tile order (pe_gather.h)
    const int row0 = tile.tm * BM, col0 = tile.tn * BN;

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

    // LDS-staged images: pixel row u of the lane's patch in the wave's slice (part 0: px 0..7,
    // part 1: px 6..13); the per-row part of the address is a scalar for one frame geometry.
    // Every byte read lies inside the patch's own pixel row (tail rows past the launch read
    // patch 0). Loading lane L takes part L & 1 of patch L >> 1 of the slice: a quad of lanes
    // reads two neighbouring patches' 56 contiguous bytes, and the two half-waves read different
    // patches (measured faster than each half-wave reading one part of all 32 patches).
    const int sgp = lane >> 1, sgh = lane & 1;
    uint32_t sgv = 0u;
    auto sg_setup = [&]() { sgv = patch_of_row<P>(a, row0 + wave * 32 + sgp).base * 2u + (sgh ? 12u : 0u); };
    auto sg_load = [&](auto uc) -> u32x4 {
        constexpr int u = decltype(uc)::value;
        return __builtin_amdgcn_raw_buffer_load_b128(
            rsrc, (int)sgv, (int)(((uint32_t)(u / P) * plane + (uint32_t)(u % P) * rstr) * 2u), 0);
    };
    // ... and its place in the group buffer (sg_row): the lane's patch slot
    const uint32_t sgw = SGOFF + (uint32_t)(wave * 32 + sgp) * SG_PITCH;
    auto sg_write = [&](auto uc, const u32x4 &v) {
        constexpr int u = decltype(uc)::value;
        constexpr SgRow w = sg_row(u);
        unsigned char *gb = lds + sgw + ((u / kSgRows) & 1) * SG_BLOCK;
        const bool h = sgh;   // the part this lane loaded
        if constexpr (w.kind == 0) {
            *reinterpret_cast<u32x4 *>(gb + (h ? 16 * w.slot_b : 16 * w.slot_a)) = h ? u32x4{v.y, v.z, v.w, v.w} : v;
        } else if constexpr (w.kind == 1) {
            // four dword writes in every lane (no branch): part 0 its 16 bytes at slot a, part 1
            // d1..d3 at byte 12 of slots b..b+2 and d3 there once more
            *reinterpret_cast<uint32_t *>(gb + (h ? 16 * w.slot_b + 12 : 16 * w.slot_a)) = h ? v.y : v.x;
            *reinterpret_cast<uint32_t *>(gb + (h ? 16 * (w.slot_b + 1) + 12 : 16 * w.slot_a + 4)) = h ? v.z : v.y;
            *reinterpret_cast<uint32_t *>(gb + (h ? 16 * (w.slot_b + 2) + 12 : 16 * w.slot_a + 8)) = h ? v.w : v.z;
            *reinterpret_cast<uint32_t *>(gb + (h ? 16 * (w.slot_b + 2) + 12 : 16 * w.slot_a + 12)) = v.w;
        } else {
            *reinterpret_cast<u32x4 *>(gb + (h ? 16 * (w.slot_b + 1) : 16 * w.slot_a)) = h ? u32x4{v.z, v.w, 0u, 0u} : v;
            // part 1: d1 at byte 12 of slot b; part 0 rewrites its own last dword
            *reinterpret_cast<uint32_t *>(gb + (h ? 16 * w.slot_b + 12 : 16 * w.slot_a + 12)) = h ? v.y : v.w;
        }
    };
    // grouped fragment 2s + h of the lane's row in 32-row block rb of the wave; each k-step reads
    // the next one's (sg_next)
    const uint32_t sgr = SGOFF + (uint32_t)(wm * TM * 32 + l32) * SG_PITCH + (h ? 16u : 0u);
    u32x4 sg_next[TM];
    auto sg_read = [&](int s, int rb) -> u32x4 {
        const int g = s / kSgSteps;
        return *reinterpret_cast<const u32x4 *>(lds + sgr + (g & 1) * SG_BLOCK + rb * 32 * SG_PITCH +
                                                (2 * s - 2 * kSgSteps * g) * 16);
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
        if constexpr (SG)
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) ald_lds[rb][0].d[0] = sg_next[rb];   // read during the previous k-step
        const AFrag<ISZ>(&ald)[TM][2] = (AST || SG) ? ald_lds : ald_regs;
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
            // staged images: the next k-step's fragment, half-way through this one's products
            if constexpr (SG && s + 1 < S)
                if (f == NF / 2 - 1)
#pragma unroll
                    for (int rb = 0; rb < TM; ++rb) sg_next[rb] = sg_read(s + 1, rb);
        }
        // Pin the interleave: PF fragment reads first, then per fragment its TM products and the
        // read PF fragments ahead (left alone, the scheduler sinks each read next to its use).
        __builtin_amdgcn_sched_group_barrier(0x100, (PF < NF ? PF : NF) + (AST ? TM * 2 * (ISZ / 2) : 0), 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x008, TM, 0);
            if (f + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (SG && s + 1 < S && f == NF / 2 - 1) __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);
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
    // LDS-staged images: rows 0..7 are staged before the loop; row u >= 8 is loaded at k-step
    // sg_load_step(u) into a ring of four and written kSgLag k-steps later (pe_internal.h; rows
    // are written before the k-step that first reads them, and into a group buffer only after
    // the reads of the group it held).
    constexpr int RD = (AST || SG) ? 1 : AD + 1;         // A ring depth (frames)
    constexpr int PRE = (AST || SG) ? 0 : AD;            // A k-steps loaded before the loop (frames)
    constexpr int NU = kC * P;                           // pixel rows of one frame's patch
    AFrag<ISZ> Ar[RD][TM][2];
    u32x4 Apc[AST ? 3 : 1][AST ? AL : 1];
    u32x4 Sr[SG ? 4 : 1];
    u32x4 Br[BD][CH];
    // staged images: rows 0..7 are loaded with the first weight k-step and written after it is
    // issued, so the tile's start waits for one round trip to memory, not two
    u32x4 first[SG ? kSgRows : 1];
    if constexpr (SG) {
        sg_setup();
        static_for<kSgRows>([&](auto uc) { first[decltype(uc)::value] = sg_load(uc); });
    }
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
            if (j == 0 && !AST && !SG) rows_setup();
            if constexpr (SG)
                if (j == 0) static_for<kSgRows>([&](auto uc) { sg_write(uc, first[decltype(uc)::value]); });
            store_b(j, tmp);
        }
    }
    static_for<BD - 1>([&](auto ic) {
        constexpr int t = KS + decltype(ic)::value;
        if constexpr (t < S) load_b(t, Br[t % BD]);
    });
    static_for<(PRE < S ? PRE : S)>([&](auto jc) { load_a(jc, Ar[decltype(jc)::value]); });
    __syncthreads();
    if constexpr (SG)
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) sg_next[rb] = sg_read(0, rb);
    static_for<S>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int t = s + KS;
        if constexpr (t + BD - 1 < S) load_b(t + BD - 1, Br[(t + BD - 1) % BD]);
        if constexpr (SG) {
            static_for<NU>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                if constexpr (u >= kSgRows && sg_load_step(u) == s) Sr[u % 4] = sg_load(uc);
            });
        } else if constexpr (AST) {
            // piece c with AC*c - 3 == s
            if constexpr ((s + 3) % AC == 0 && (s + 3) / AC < NCH && (s + 3) / AC >= 1)
                load_piece(IC<(s + 3) / AC>{}, Apc[((s + 3) / AC) % 3]);
        } else if constexpr (s + AD < S) {
            load_a(IC<s + AD>{}, Ar[(s + AD) % RD]);
        }
        compute(sc, Ar[s % RD]);
        if constexpr (t < S) store_b(t, Br[t % BD]);
        if constexpr (SG) {
            static_for<NU>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                if constexpr (u >= kSgRows && sg_load_step(u) + kSgLag == s) sg_write(uc, Sr[u % 4]);
            });
        }
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

}  // namespace pe
