// Internal declarations shared by the host API and the gfx950 kernels.
// Not part of the public ABI (include/sage_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Tile constants.
constexpr int kKeyBlock = 64;      // tokens per K quantization block (one INT8 scale each)
constexpr int kChunk = 256;        // tokens per partial sum of the fp64 key mean
constexpr int kBQ = 128;           // query rows per workgroup of the FP8 variant (4 waves x 32);
                                   // the 16-bit-PV variant uses 256 (8 waves)
constexpr int kBK = 128;           // keys per online-softmax step
constexpr int kQPad = 256;         // Lq is padded to a multiple of this in the workspace
constexpr int kKPad = kBK;         // Lk is padded to a multiple of this in the workspace

struct StatsArgs {
    const void* k;
    const void* v;
    int64_t ks0, ks1, ks2;         // element strides of k (batch, head, token)
    int64_t vs0, vs1, vs2;
    int Hkv, Lk, D, Dp, nchunk, smooth;
    double* kpart;                 // [B][Hkv][nchunk][Dp]
    float* vpart;                  // [B][Hkv][nchunk][Dp]
};

struct QuantQArgs {
    const void* q;
    int64_t qs0, qs1, qs2;
    int B, Hq, Lq, Lq_pad, D;
    int8_t* qhat;                  // [B][Hq][Lq_pad][Dp]
    float* sq;                     // [B][Hq][Lq_pad]
};

struct QuantKVArgs {
    const void* k;
    const void* v;
    int64_t ks0, ks1, ks2;
    int64_t vs0, vs1, vs2;
    int Hkv, Lk, Lk_pad, D, nkb, nchunk, smooth;
    const double* kpart;           // [B][Hkv][nchunk][Dp] chunk partial key sums
    const float* vpart;            // [B][Hkv][nchunk][Dp] chunk partial max |v|
    float* kbar;                   // [B][Hkv][Dp] written by the block-0 workgroups
    float* vmax;                   // [B][Hkv][Dp] written by the block-0 workgroups
    int8_t* khat;                  // [B][Hkv][Lk_pad][Dp]
    float* sk;                     // [B][Hkv][nkb]
    uint8_t* vhat;                 // [B][Hkv][nkb][Dp][64] elements, permuted inside each block
    int pv16;                      // 0: FP8 E4M3 codes; 1: the 16-bit input values
};

struct AttnArgs {
    const int8_t* qhat;
    const float* sq;
    const int8_t* khat;
    const float* sk;
    const uint8_t* vhat;
    const float* vmax;
    void* o;
    int64_t os0, os1, os2;
    int B, Hq, Hkv, G, Lq, Lk, Lq_pad, Lk_pad, nkb, D;
    int nqt;                       // query tiles per head
    float scale_log2;              // sm_scale * log2(e)
    // debug dump of int32 logits (one head)
    int32_t* dump;
    int dump_b, dump_hq;
};

// Launchers; return the hipError_t of the launch.
hipError_t launch_stats_q(const StatsArgs& sa, const QuantQArgs& qa, int B, int Dp, int dtype, bool vec_q,
                          hipStream_t s);
hipError_t launch_quant_kv(const QuantKVArgs& a, int B, int Dp, int dtype, bool vec,
                           hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out, bool pv16,
                       hipStream_t s);
hipError_t launch_attn_dump(const AttnArgs& a, int Dp, hipStream_t s);

}  // namespace sage
