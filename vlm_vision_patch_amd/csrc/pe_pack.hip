// pe_pack.hip -- weight pre-pack and bias kernels, and the forward dispatch to the translation
// units that hold the forward kernels (one per patch size and input dtype).
#include "pe_kernels.h"

namespace pe {

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
