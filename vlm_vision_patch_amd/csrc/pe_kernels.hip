// pe_kernels.hip -- gfx950 kernels of the vision PatchEmbed.
//
// The operation ("Qwen2.5VL-Vision Encode-PatchEmbed", the bullet list on the convolution):
// a Conv3d whose kernel equals its stride meets each patch once, so it is a matrix product
//   out[r, e] = sum_k A[r, k] * W[e, k] (+ b[e]),  K = C*Tp*P*P,
// where A[r, :] is the patch behind output row r, flattened. Nothing materialises A: the
// forward kernel reads each patch's pixels straight from the frames (or patch rows) into the
// registers that feed the matrix cores.
//
// K order. Any permutation of k applied to both A and W leaves the sum unchanged, so the
// kernels use one that suits 16-byte fragments. A patch is C*Tp*P pixel rows of P elements,
// r = (tt*C + c)*P + py. For bf16 and P = 14 each row gives one whole 8-element fragment
// (px 0..7, one 16-byte load) and a 6-element rest; the rests of rows a, b, c, d form three
// fragments (a[8:14] + d[8:10]), (b[8:14] + d[10:12]), (c[8:14] + d[12:14]), each a 12-byte
// and a 4-byte load. 84 rows give 84 + 63 fragments; one zero fragment pads them to 37
// k-steps of 32 (1184 = 1176 + 8). For P = 16 every row is two whole fragments (48 steps).
// fp32 uses 4-element fragments the same way (P = 14: 3 whole + pairs of 2-element rests).
// The weight is packed once in exactly this order (pe_pack_kernel).
//
// Forward kernel layout. A workgroup computes a BM x BN output tile with WM x WN waves; each
// wave owns TM x TN blocks of 16 x 16. The wave loads its own A fragments from global memory
// (raw buffer loads: 32-bit offsets, reads past the input range return 0), so A never passes
// through LDS. The packed weight for one k-step and the tile's BN columns is one contiguous
// BN*64-byte run; it is staged through a double-buffered LDS stage and read back as one
// conflict-free 16-byte ds_read per lane and 16-column block. Matrix core:
// v_mfma_f32_16x16x32_bf16 (fp32 accumulate) or v_mfma_f32_16x16x4_f32.
//
// Rows of the tile are output rows in output order; each lane maps its row back to the patch
// (item, tp, hp, wp) through the raster or merge-window order, so the order costs only index
// arithmetic and the stores stay row-contiguous.
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

// ----------------------------------------------------------------------------------------
// Weight pre-pack: W[E][C][Tp][P][P] -> packed[s][E/16][g][n][16 bytes] in the fragment order.
// One thread writes one 16-byte fragment (step s, column e = 16*cb + n, lane group g).
// ----------------------------------------------------------------------------------------
template <typename TW>
__global__ void pe_pack_kernel(const TW *__restrict__ w, TW *__restrict__ wpk, int P, int E,
                               int S) {
    constexpr int esz = sizeof(TW);
    constexpr int epf = 16 / esz;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)S * E * 4;
    if (idx >= total) return;
    const int n = (int)(idx % 16);
    int64_t t = idx / 16;
    const int g = (int)(t % 4);
    t /= 4;
    const int ncb = E / 16;
    const int cb = (int)(t % ncb);
    const int s = (int)(t / ncb);
    const int e = cb * 16 + n;
    const Piece pc = frag_piece(P, esz, s, g);
    const int first = split_first(P, esz);
    TW vals[epf];
#pragma unroll
    for (int j = 0; j < epf; ++j) {
        int r = 0, x = 0;
        bool pad = false;
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
    int lo = 0, hi = a.n_items - 1;
    while (lo < hi) {  // last item whose first row <= row
        const int mid = (lo + hi + 1) >> 1;
        if (row >= a.items[mid].row0) lo = mid; else hi = mid - 1;
    }
    const Item it = a.items[lo];
    const uint32_t q = (uint32_t)(row - it.row0);
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

template <int P, int ESZ, int OSZ, int TM, int TN, int WM, int WN>
__global__ void __launch_bounds__(WM *WN * 64, 1) pe_fwd_kernel(const FwdArgs a) {
    constexpr int NT = WM * WN * 64;
    constexpr int BM = WM * TM * 16;
    constexpr int BN = WN * TN * 16;
    constexpr int S = num_steps(P, ESZ);
    constexpr int SF = full_steps(P, ESZ);
    constexpr int STAGE = BN * 64;
    constexpr int CH = STAGE / (16 * NT);
    static_assert(STAGE % (16 * NT) == 0, "stage must split evenly over the threads");
    constexpr int FIRST = split_first(P, ESZ);  // elements in the first piece of a split fragment
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];

    // ---- tile: blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous run of
    // tiles so the tiles that share rows (same tm) run on one XCD, close in time.
    const int G = a.tiles_m * a.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, loc = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    const int tm = L / a.tiles_n, tn = L - tm * a.tiles_n;
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

    // A fragments of k-step s for this lane's TM rows.
    auto load_a = [&](int s, u32x4 (&dst)[TM]) {
        const Piece pc = frag_piece(P, ESZ, s, g);
        if (s < SF) {
#pragma unroll
            for (int rb = 0; rb < TM; ++rb)
                dst[rb] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(elem_off(pr[rb], pc.r1, pc.x1) * ESZ), 0, 0);
        } else {
            const bool pad = pc.kind == kPad;
#pragma unroll
            for (int rb = 0; rb < TM; ++rb) {
                const int o1 = (int)(elem_off(pr[rb], pc.r1, pc.x1) * ESZ);
                const int o2 = (int)(elem_off(pr[rb], pc.r2, pc.x2) * ESZ);
                u32x4 v;
                if constexpr (FIRST * ESZ == 12) {
                    const u32x3 m3 = __builtin_amdgcn_raw_buffer_load_b96(rsrc, o1, 0, 0);
                    const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b32(rsrc, o2, 0, 0);
                    v = u32x4{m3.x, m3.y, m3.z, e1};
                } else if constexpr (FIRST * ESZ == 8) {
                    const u32x2 m2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, o1, 0, 0);
                    const u32x2 e2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, o2, 0, 0);
                    v = u32x4{m2.x, m2.y, e2.x, e2.y};
                } else {
                    v = u32x4{0u, 0u, 0u, 0u};
                }
                dst[rb] = pad ? u32x4{0u, 0u, 0u, 0u} : v;
            }
        }
    };

    // Packed weight of k-step s for the tile's columns: BN*64 contiguous bytes.
    auto load_b = [&](int s, u32x4 (&dst)[CH]) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.wpk) + ((int64_t)s * ncb + (col0 >> 4)) * 64;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = c * NT + tid;
            dst[c] = ((col0 >> 4) + (idx >> 6) < ncb) ? src[idx] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_b = [&](int buf, const u32x4 (&src)[CH]) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(lds + buf * STAGE);
#pragma unroll
        for (int c = 0; c < CH; ++c) dst[c * NT + tid] = src[c];
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, const u32x4 (&af)[TM]) {
        const u32x4 *bs = reinterpret_cast<const u32x4 *>(lds + buf * STAGE) + wn * TN * 64 + lane;
#pragma unroll
        for (int cb = 0; cb < TN; ++cb) {
            const u32x4 bf = bs[cb * 64];
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

    u32x4 A0[TM], A1[TM], breg[CH];
    load_b(0, breg);
    load_a(0, A0);
    if (S > 1) load_a(1, A1);
    store_b(0, breg);
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
        if (s + 1 < S) load_b(s + 1, breg);
        compute(0, A0);
        if (s + 2 < S) load_a(s + 2, A0);
        if (s + 1 < S) store_b(1, breg);
        __syncthreads();
        if (s + 1 < S) {
            if (s + 2 < S) load_b(s + 2, breg);
            compute(1, A1);
            if (s + 3 < S) load_a(s + 3, A1);
            if (s + 2 < S) store_b(0, breg);
            __syncthreads();
        }
    }

    // ---- epilogue: + bias (fp32), one RNE cast, row-contiguous output
#pragma unroll
    for (int cb = 0; cb < TN; ++cb) {
        const int col = col0 + (wn * TN + cb) * 16 + l16;
        if (col >= a.E) continue;
        const float bv = a.bias ? a.bias[col] : 0.f;
#pragma unroll
        for (int rb = 0; rb < TM; ++rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + (wm * TM + rb) * 16 + 4 * g + i;
                if (row < a.n_rows) store_out<OSZ>(a.out, (int64_t)row * a.E + col, acc[rb][cb][i] + bv);
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------------------
hipError_t launch_pack(const void *w, int w_esz, void *wpk, int P, int E, hipStream_t st) {
    const int S = num_steps(P, w_esz);
    const int64_t total = (int64_t)S * E * 4;
    const int threads = 256;
    const int blocks = (int)((total + threads - 1) / threads);
    if (w_esz == 2)
        hipLaunchKernelGGL(pe_pack_kernel<uint16_t>, dim3(blocks), dim3(threads), 0, st,
                           static_cast<const uint16_t *>(w), static_cast<uint16_t *>(wpk), P, E, S);
    else
        hipLaunchKernelGGL(pe_pack_kernel<float>, dim3(blocks), dim3(threads), 0, st,
                           static_cast<const float *>(w), static_cast<float *>(wpk), P, E, S);
    return hipGetLastError();
}

hipError_t launch_bias(const void *b, int b_esz, float *bias32, int E, hipStream_t st) {
    const int threads = 256, blocks = (E + threads - 1) / threads;
    if (b_esz == 2)
        hipLaunchKernelGGL(pe_bias_kernel<__bf16>, dim3(blocks), dim3(threads), 0, st,
                           static_cast<const __bf16 *>(b), bias32, E);
    else
        hipLaunchKernelGGL(pe_bias_kernel<float>, dim3(blocks), dim3(threads), 0, st,
                           static_cast<const float *>(b), bias32, E);
    return hipGetLastError();
}

template <int P, int ESZ, int OSZ, int TM, int TN, int WM, int WN>
static hipError_t launch_cfg(FwdArgs a, hipStream_t st) {
    constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
    a.tiles_m = (a.n_rows + BM - 1) / BM;
    a.tiles_n = (a.E + BN - 1) / BN;
    const int blocks = a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((pe_fwd_kernel<P, ESZ, OSZ, TM, TN, WM, WN>), dim3(blocks), dim3(WM * WN * 64), 0, st, a);
    return hipGetLastError();
}

// Tile choice: the largest tile that still gives every CU work.
template <int P, int ESZ, int OSZ>
static hipError_t launch_p(const FwdArgs &a, hipStream_t st) {
    const int64_t big = ((int64_t)(a.n_rows + 255) / 256) * ((a.E + 255) / 256);
    const int64_t mid = ((int64_t)(a.n_rows + 63) / 64) * ((a.E + 255) / 256);
    if (big >= 512) return launch_cfg<P, ESZ, OSZ, 4, 8, 4, 2>(a, st);
    if (mid >= 256) return launch_cfg<P, ESZ, OSZ, 2, 8, 2, 2>(a, st);
    return launch_cfg<P, ESZ, OSZ, 1, 4, 2, 2>(a, st);
}

hipError_t launch_forward(const FwdArgs &a, int P, int in_esz, int out_esz, hipStream_t st) {
    if (P == 14) {
        if (in_esz == 2) return out_esz == 2 ? launch_p<14, 2, 2>(a, st) : launch_p<14, 2, 4>(a, st);
        return out_esz == 2 ? launch_p<14, 4, 2>(a, st) : launch_p<14, 4, 4>(a, st);
    }
    if (in_esz == 2) return out_esz == 2 ? launch_p<16, 2, 2>(a, st) : launch_p<16, 2, 4>(a, st);
    return out_esz == 2 ? launch_p<16, 4, 2>(a, st) : launch_p<16, 4, 4>(a, st);
}

}  // namespace pe
