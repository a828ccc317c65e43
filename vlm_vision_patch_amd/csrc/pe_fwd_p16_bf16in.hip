// pe_fwd_p16_bf16in.hip -- forward kernels for P = 16, bf16 input (bf16 weight).
#include "pe_kernels.h"

namespace pe {

hipError_t launch_forward_p16_bf16in(const FwdArgs &a, int out_esz, hipStream_t st) {
    return out_esz == 2 ? launch_p<16, 2, 2, 2>(a, st) : launch_p<16, 2, 2, 4>(a, st);
}

}  // namespace pe
