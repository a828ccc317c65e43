// pe_fwd_p16_f32in.hip -- forward kernels for P = 16, fp32 input: on an fp32 weight, or on a bf16
// weight (the input rounded to bf16 as it is loaded).
#include "pe_kernels.h"

namespace pe {

hipError_t launch_forward_p16_f32in(const FwdArgs &a, int w_esz, int out_esz, hipStream_t st) {
    if (w_esz == 4) return out_esz == 2 ? launch_p<16, 4, 4, 2>(a, st) : launch_p<16, 4, 4, 4>(a, st);
    return out_esz == 2 ? launch_p<16, 2, 4, 2>(a, st) : launch_p<16, 2, 4, 4>(a, st);
}

}  // namespace pe
