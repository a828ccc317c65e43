// pe_pack.hip -- weight pre-pack and bias kernels, and the forward dispatch to the translation
// units that hold the forward kernels (one per patch size and input dtype).
#include "pe_device.h"

namespace pe {

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
        // temporal-split map: g = 2j + tt, unique fragment uf = 2s + j (kPackTTG: the grouped
        // order's fragment 2s + j)
        const int tt = g & 1;
        const int ufg = 2 * s + (g >> 1);
        const UFrag f = tt_frag(P, map == kPackTTG ? ttg_uf(P, ufg) : ufg);
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

hipError_t launch_pack(const void *w, int w_esz, void *wpk, int P, int E, int map, hipStream_t st) {
    if (w_esz != 2 && map != kPackTT) return hipErrorInvalidValue;
    const int S = map == kPackRows ? rows_steps(P) : (map == kPackFold ? fold_steps(P) : packed_steps(P, w_esz));
    const int64_t total = (int64_t)S * packed_cols(E, w_esz) * 4;
    const int threads = 256;
    const int blocks = (int)((total + threads - 1) / threads);
    if (w_esz == 2)
        hipLaunchKernelGGL(pe_pack_kernel<uint16_t>, dim3(blocks), dim3(threads), 0, st,
                           static_cast<const uint16_t *>(w), static_cast<uint16_t *>(wpk), P, E, S, map);
    else
        hipLaunchKernelGGL(pe_pack_kernel<float>, dim3(blocks), dim3(threads), 0, st,
                           static_cast<const float *>(w), static_cast<float *>(wpk), P, E, S, (int)kPackTT);
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

hipError_t launch_forward(const FwdArgs &a, int P, int w_esz, int in_esz, int out_esz, hipStream_t st) {
    if (w_esz == 4 && in_esz != 4) return hipErrorInvalidValue;  // fp32 weight: fp32 input
    if (P == 14) return in_esz == 2 ? launch_forward_p14_bf16in(a, out_esz, st) : launch_forward_p14_f32in(a, w_esz, out_esz, st);
    if (P == 16) return in_esz == 2 ? launch_forward_p16_bf16in(a, out_esz, st) : launch_forward_p16_f32in(a, w_esz, out_esz, st);
    return hipErrorInvalidValue;
}

}  // namespace pe
