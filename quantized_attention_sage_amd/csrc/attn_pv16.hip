// Instantiations of the attention kernel with 16-bit P.V (attn_kernel.h).
#include "attn_kernel.h"

namespace sage {

hipError_t launch_attn_pv16(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out, hipStream_t s) {
    return dtype == 0 ? attn_dispatch_dp<__half, true>(a, Dp, causal, vec_out, s)
                      : attn_dispatch_dp<__hip_bfloat16, true>(a, Dp, causal, vec_out, s);
}

}  // namespace sage
