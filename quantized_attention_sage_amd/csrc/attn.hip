// Host launchers of the attention kernels (attn_kernel.h): the split merge,
// the int32-logit dump, and the dispatch to the P.V formats, whose kernel
// instantiations live in attn_fp8.hip and attn_pv16.hip (compiled apart).
#include "attn_kernel.h"

namespace sage {

hipError_t launch_combine(const AttnArgs& a, int Dp, int dtype, bool vec_out, bool pv16, hipStream_t s) {
    const float ps = pv16 ? 0.0f : 8.0f;
    if (dtype == 0)
        return Dp == 64 ? combine_dispatch<64, __half>(a, vec_out, ps, s)
                        : combine_dispatch<128, __half>(a, vec_out, ps, s);
    return Dp == 64 ? combine_dispatch<64, __hip_bfloat16>(a, vec_out, ps, s)
                    : combine_dispatch<128, __hip_bfloat16>(a, vec_out, ps, s);
}

hipError_t launch_attn(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out, bool pv16,
                       hipStream_t s) {
    return pv16 ? launch_attn_pv16(a, Dp, dtype, causal, vec_out, s)
                : launch_attn_fp8(a, Dp, dtype, causal, vec_out, s);
}

hipError_t launch_deal_tiles(const AttnArgs& a, int bq, int nqt, int full, hipStream_t s) {
    if (bq == 128)
        deal_tiles_kernel<128><<<8, 256, 0, s>>>(a, nqt, full);
    else
        deal_tiles_kernel<256><<<8, 256, 0, s>>>(a, nqt, full);
    return hipGetLastError();
}

hipError_t launch_attn_dump(const AttnArgs& a, int Dp, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>((a.m.Lq + kBQ - 1) / kBQ);
    if (Dp == 64)
        qk_dump_kernel<64><<<grid, 256, 0, s>>>(a);
    else
        qk_dump_kernel<128><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sage
