// Main attention kernel for gfx950: INT8 QK^T on the matrix cores, online
// softmax, FP8 (E4M3) P.V into FP32 accumulators.
//
// Method sources (page, section):
//   topgit.dev "SageAttention: Quantized Attention Library", core features and
//   "SageAttention vs FlashAttention": INT8 QK^T after smoothing, FP8 PV, the
//   blockwise (FlashAttention-style) softmax over key blocks;
//   gittoolsai.com README translation, performance section: "8+8" = INT8 QK^T
//   and FP8 PV; usage section: is_causal, HND/NHD, GQA, Lq != Lk;
//   stable-diffusion.cpp "SageAttention" doc: original softmax scale kept,
//   output cropped to the original head dim.
//
// Orientation. Each wave owns 32 query rows. The logits are computed
// transposed, S^T = Khat . Qhat^T, with v_mfma_i32_32x32x32_i8 (A = 32 keys x
// 32 channels, B = 32 channels x 32 queries). In the 32x32 accumulator, lane l
// holds query column l%32 and keys 8*(r/4) + 4*(l/32) + r%4 (r = 0..15), so a
// query's row max and normaliser only need one exchange between the two
// lane halves (v_permlane32_swap) and every per-query constant is a lane
// scalar. The FP32 probabilities of a 64-key sub-block are converted to E4M3
// in place and form directly the B operand (64 keys x 32 queries) of
// v_mfma_f32_32x32x64_f8f6f4; the A operand is V^T (32 channels x 64 keys),
// which the prologue stored with the matching token permutation. The output
// accumulates transposed as well, O^T (Dp x 32 queries) in FP32.
//
// The normaliser l is the sum of the same FP8 probabilities that multiply V;
// it comes from one extra matrix-core product with an all-ones A operand.
//
// Workgroup: 4 waves = 128 queries. Key blocks of 128 tokens (2 quantization
// blocks of 64) are staged global -> registers -> LDS, double buffered with
// one barrier per step; LDS rows are XOR-swizzled in 16-byte chunks so the
// operand reads are free of bank conflicts.
#include "sage_kernels.h"

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));


__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
    // format selectors 0/0: both operands FP8 E4M3; no block scales.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS swizzle: 16-byte chunk k of row i (row length rb bytes) is stored at
// chunk k ^ ((i / (128 / rb)) % (rb / 16)).
template <int RB>
__device__ __forceinline__ int swz(int i, int k) {
    constexpr int RPL = (RB >= 128) ? 1 : 128 / RB;
    constexpr int CPR = RB / 16;
    return k ^ ((i / RPL) % (CPR < 8 ? CPR : 8));
}

template <typename T>
__device__ __forceinline__ uint16_t from_f32(float x);
template <>
__device__ __forceinline__ uint16_t from_f32<__half>(float x) {
    return __half_as_ushort(__float2half_rn(x));
}
template <>
__device__ __forceinline__ uint16_t from_f32<__hip_bfloat16>(float x) {
    // round to nearest even (finite values)
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}


template <int DP, typename T, bool CAUSAL, bool DUMP, bool VEC_OUT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    constexpr int NC = DP / 32;                 // 32-channel chunks of the QK contraction
    constexpr int NU = DP / 32;                 // 32-channel tiles of the output
    constexpr int KBYTES = kBK * DP;            // bytes of one K block (= one V block)
    constexpr int NLD = KBYTES / 16 / 256;      // 16-byte chunks per thread per tensor
    __shared__ __align__(16) uint8_t ks[2][KBYTES];
    __shared__ __align__(16) uint8_t vs[2][KBYTES];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int lq = l & 31;
    const int hh = l >> 5;

    // ---- block -> (b, hq, query tile), XCD-aware ----
    int b, hq, qt;
    if (DUMP) {
        b = a.dump_b;
        hq = a.dump_hq;
        qt = blockIdx.x;
    } else {
        const int n = blockIdx.x;
        const int N = gridDim.x;
        const int full = N / 8;
        // consecutive logical tiles (same kv head) land on the same XCD
        const int L = (n < full * 8) ? (n % 8) * full + n / 8 : n;
        qt = L % a.nqt;
        int rest = L / a.nqt;
        const int g = rest % a.G;
        rest /= a.G;
        const int hkv_ = rest % a.Hkv;
        b = rest / a.Hkv;
        hq = hkv_ * a.G + g;
    }
    const int hkv = hq / a.G;
    const int q0 = qt * kBQ + w * 32;           // first query of this wave
    const int qi = q0 + lq;                     // this lane's query

    const int64_t qrow = (static_cast<int64_t>(b) * a.Hq + hq) * a.Lq_pad + qi;
    v4i qb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        qb[c] = *reinterpret_cast<const v4i*>(a.qhat + qrow * DP + 32 * c + 16 * hh);
    const float scq = a.sq[qrow] * a.scale_log2;

    const int64_t kvh = static_cast<int64_t>(b) * a.Hkv + hkv;
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.khat) + kvh * a.Lk_pad * DP;
    const uint8_t* vg = a.vhat + kvh * a.nkb * (DP * 64);
    const float* skp = a.sk + kvh * a.nkb;

    int nkblk = a.Lk_pad / kBK;
    if (CAUSAL) {
        const int last = min(a.Lk, qt * kBQ + kBQ);      // keys 0..last-1 can be visible
        nkblk = (last + kBK - 1) / kBK;
    }

    // ---- staging helpers ----
    uint4 kr[NLD], vr[NLD];
    auto gload = [&](int kb) {
        const uint4* ksrc = reinterpret_cast<const uint4*>(kg + static_cast<int64_t>(kb) * KBYTES);
        const uint4* vsrc = reinterpret_cast<const uint4*>(vg + static_cast<int64_t>(kb) * KBYTES);
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            kr[n] = ksrc[tid + 256 * n];
            vr[n] = vsrc[tid + 256 * n];
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const int g = tid + 256 * n;
            // K: row i of DP bytes, chunk k
            const int ki = g / (DP / 16), kk = g % (DP / 16);
            *reinterpret_cast<uint4*>(&ks[buf][ki * DP + 16 * swz<DP>(ki, kk)]) = kr[n];
            // V: sub-block sb, row d of 64 bytes, chunk k
            const int sb = g / (DP * 4), rem = g % (DP * 4);
            const int vd = rem / 4, vk = rem % 4;
            *reinterpret_cast<uint4*>(&vs[buf][sb * DP * 64 + vd * 64 + 16 * swz<64>(vd, vk)]) = vr[n];
        }
    };

    v16f oacc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[u][r] = 0.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;
    const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kb = 0; kb < nkblk; ++kb) {
        const int buf = kb & 1;
        const bool more = kb + 1 < nkblk;
        if (more) gload(kb + 1);

        const int k0 = kb * kBK;
        const bool wave_active = !CAUSAL || DUMP || k0 <= q0 + 31;
        if (wave_active) {
            // ---- S^T = Khat . Qhat^T : 4 tiles of 32 keys ----
            v16i s[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[t][r] = 0;
                const int row = 32 * t + lq;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const v4i ka = *reinterpret_cast<const v4i*>(&ks[buf][row * DP + 16 * swz<DP>(row, 2 * c + hh)]);
                    s[t] = mfma_i8(ka, qb[c], s[t]);
                }
            }

            if (DUMP) {
                int32_t* out = a.dump + static_cast<int64_t>(qi) * a.Lk_pad + k0;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        out[32 * t + 8 * (r / 4) + 4 * hh + (r % 4)] = s[t][r];
            } else {
                // ---- masking (tail keys, causal diagonal) ----
                const bool need_mask = (k0 + kBK > a.Lk) || (CAUSAL && k0 + kBK - 1 > q0);
                if (need_mask) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * t + 8 * (r / 4) + 4 * hh + (r % 4);
                            const bool masked = key >= a.Lk || (CAUSAL && key > qi);
                            if (masked) s[t][r] = INT32_MIN;
                        }
                }
                // ---- row max per 64-key sub-block (int domain), then logits ----
                float sc[2], mlog[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    int mx = INT32_MIN;
#pragma unroll
                    for (int t = 2 * sb; t < 2 * sb + 2; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = max(mx, s[t][r]);
                    // lanes l and l^32 hold the two key halves of the same query
                    const auto pr = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
                    mx = max(static_cast<int>(pr[0]), static_cast<int>(pr[1]));
                    sc[sb] = scq * skp[(k0 >> 6) + sb];
                    mlog[sb] = (mx == INT32_MIN) ? -INFINITY : static_cast<float>(mx) * sc[sb];
                }
                const float m_new = fmaxf(m_run, fmaxf(mlog[0], mlog[1]));
                const float mref = (m_new == -INFINITY) ? 0.0f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
                const float bias = 8.0f - mref;          // P is scaled by 2^8 before FP8

                // ---- P = exp2(logit - m) * 2^8 -> E4M3, packed as the B operand ----
                v8i pb[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int wd = 0; wd < 8; ++wd) {
                        const int t = 2 * sb + wd / 4;
                        const int r0 = 4 * (wd % 4);
                        float p[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int sv = s[t][r0 + e];
                            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(sv), sc[sb], bias));
                            if (need_mask && sv == INT32_MIN) p[e] = 0.0f;
                        }
                        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                        word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
                        pb[sb][wd] = word;
                    }
                }

                // ---- normaliser: sum of the FP8 probabilities via an all-ones A ----
                v16f lacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;
                lacc = mfma_f8(ones, pb[0], lacc);
                lacc = mfma_f8(ones, pb[1], lacc);
                l_run = alpha * l_run + lacc[0];

                // ---- O^T = alpha * O^T + V^T . P^T ----
                if (__any(alpha != 1.0f)) {
#pragma unroll
                    for (int u = 0; u < NU; ++u)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;
                }
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const uint8_t* vsb = &vs[buf][sb * DP * 64];
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        const int d = 32 * u + lq;
                        const v4i lo = *reinterpret_cast<const v4i*>(&vsb[d * 64 + 16 * swz<64>(d, 2 * hh)]);
                        const v4i hi = *reinterpret_cast<const v4i*>(&vsb[d * 64 + 16 * swz<64>(d, 2 * hh + 1)]);
                        const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        oacc[u] = mfma_f8(va, pb[sb], oacc[u]);
                    }
                }
                m_run = m_new;
            }
        }

        if (more) lstore(buf ^ 1);
        __syncthreads();
    }

    if (DUMP) return;

    // ---- epilogue: O = O^T * s_v[d] / l, crop to (Lq, D), cast ----
    if (qi >= a.Lq) return;
    const float inv_l = 1.0f / l_run;
    const float* vmax = a.vmax + kvh * DP;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.os0 + hq * a.os1 + static_cast<int64_t>(qi) * a.os2;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * u + 8 * r4 + 4 * hh;
            if (d0 >= a.D) continue;
            uint16_t h4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sv = vmax[d0 + e] / 448.0f;
                h4[e] = from_f32<T>(oacc[u][4 * r4 + e] * sv * inv_l);
            }
            if (VEC_OUT) {
                uint2 pk;
                pk.x = static_cast<uint32_t>(h4[0]) | (static_cast<uint32_t>(h4[1]) << 16);
                pk.y = static_cast<uint32_t>(h4[2]) | (static_cast<uint32_t>(h4[3]) << 16);
                *reinterpret_cast<uint2*>(orow + d0) = pk;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (d0 + e < a.D) orow[d0 + e] = h4[e];
            }
        }
    }
}

template <int DP, typename T>
hipError_t attn_dispatch(const AttnArgs& a, bool causal, bool vec_out, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.nqt) * a.Hq * a.B;
    if (causal) {
        if (vec_out) attn_kernel<DP, T, true, false, true><<<grid, 256, 0, s>>>(a);
        else attn_kernel<DP, T, true, false, false><<<grid, 256, 0, s>>>(a);
    } else {
        if (vec_out) attn_kernel<DP, T, false, false, true><<<grid, 256, 0, s>>>(a);
        else attn_kernel<DP, T, false, false, false><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out,
                       hipStream_t s) {
    if (dtype == 0)
        return Dp == 64 ? attn_dispatch<64, __half>(a, causal, vec_out, s)
                        : attn_dispatch<128, __half>(a, causal, vec_out, s);
    return Dp == 64 ? attn_dispatch<64, __hip_bfloat16>(a, causal, vec_out, s)
                    : attn_dispatch<128, __hip_bfloat16>(a, causal, vec_out, s);
}

hipError_t launch_attn_dump(const AttnArgs& a, int Dp, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.nqt);
    if (Dp == 64)
        attn_kernel<64, __half, false, true, false><<<grid, 256, 0, s>>>(a);
    else
        attn_kernel<128, __half, false, true, false><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sage
