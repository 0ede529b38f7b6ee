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
// query's row max only needs one exchange between the two lane halves
// (v_permlane32_swap) and every per-query constant is a lane scalar. The FP32
// probabilities of a 64-key sub-block are converted to E4M3 in place and form
// directly the B operand (64 keys x 32 queries) of v_mfma_f32_32x32x64_f8f6f4;
// the A operand is V^T (32 channels x 64 keys), which the prologue stored with
// the matching token permutation. The output accumulates transposed as well,
// O^T (Dp x 32 queries) in FP32.
//
// The normaliser l is the sum of the same FP8 probabilities that multiply V;
// it comes from one extra matrix-core product with an all-ones A operand.
//
// Workgroup: 4 waves = 128 queries. Key blocks of 128 tokens (2 quantization
// blocks of 64) are copied global -> LDS directly (no register staging),
// double buffered with one barrier per step; LDS rows are XOR-swizzled in
// 16-byte chunks so the operand reads are free of bank conflicts. Blocks that
// need no mask (all but the causal diagonal and the ragged tail) run a
// separate loop without any masking code.
#include "sage_kernels.h"

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int KBYTES128 = kBK * 128;

__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
    // format selectors 0/0: both operands FP8 E4M3; no block scales.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// int32 accumulators start at this bias so that the bits of (bias + A) read as
// the float 1.5 * 2^23 + A exactly for |A| < 2^22 (|A| <= 128 * 127^2 here):
// the logits need no int -> float conversion, one FMA dequantizes them.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

// LDS swizzle: 16-byte chunk k of row i (rows of RB bytes) is stored at chunk
// k ^ swz_row<RB>(i). Rows sharing a 128-byte bank line get different masks,
// so the 8 lanes served together by one ds_read_b128 phase hit 8 distinct
// 16-byte bank groups.
template <int RB>
__device__ __forceinline__ int swz_row(int i) {
    constexpr int RPL = (RB >= 128) ? 1 : 128 / RB;     // rows per 128-byte line
    constexpr int CPR = RB / 16;                         // chunks per row
    return (i / RPL) % (CPR < 8 ? CPR : 8);
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

// Direct global -> LDS copy of one 128-key block of Khat (128 x DP bytes,
// swizzled rows) and of V^T (two 64-key sub-blocks of DP x 64 bytes). Each
// instruction moves 64 lanes x 16 bytes into 1 KB of LDS at a wave-uniform
// base, lane i landing at base + 16 i, so each lane fetches the global chunk
// that the swizzle places at its slot.
template <int DP>
__device__ __forceinline__ void stage_block(const uint8_t* kg, const uint8_t* vg,
                                            uint8_t* kl, uint8_t* vl, int w, int l) {
    constexpr int KCH = kBK * DP / 16;          // 16-byte chunks per tensor block
    constexpr int PER_WAVE = KCH / 4;
#pragma unroll
    for (int n = 0; n < PER_WAVE / 64; ++n) {
        const int c = w * PER_WAVE + n * 64 + l;     // LDS chunk slot of this lane
        const int ki = c / (DP / 16), kp = c % (DP / 16);
        const int kc = ki * (DP / 16) + (kp ^ swz_row<DP>(ki));
        __builtin_amdgcn_global_load_lds(kg + 16 * kc, (lds_void*)(kl + 16 * (w * PER_WAVE + n * 64)), 16, 0, 0);
        const int sb = c / (DP * 4), rem = c % (DP * 4);
        const int vd = rem / 4, vp = rem % 4;
        const int vc = sb * (DP * 4) + vd * 4 + (vp ^ swz_row<64>(vd));
        __builtin_amdgcn_global_load_lds(vg + 16 * vc, (lds_void*)(vl + 16 * (w * PER_WAVE + n * 64)), 16, 0, 0);
    }
}

// S^T for one 128-key block: 4 tiles of 32 keys, accumulators biased by kMagicBits.
template <int DP>
__device__ __forceinline__ void qk_block(v16i (&s)[4], const uint8_t* ksm, const v4i (&qb)[DP / 32],
                                         int lq, int hh) {
    const v16i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                        kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                        kMagicBits, kMagicBits, kMagicBits, kMagicBits};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int row = 32 * t + lq;
#pragma unroll
        for (int c = 0; c < DP / 32; ++c) {
            const v4i ka = *reinterpret_cast<const v4i*>(&ksm[row * DP + 16 * (swz_row<DP>(row) ^ (2 * c + hh))]);
            s[t] = mfma_i8(ka, qb[c], c == 0 ? magic : s[t]);
        }
    }
}

template <int NU>
struct SoftmaxState {
    v16f o[NU];
    float m;
    float l;
};

// One 128-key step of the online softmax for the wave's 32 queries.
// EXACT: take (bits - bias) back to the integer exactly (Sterbenz) before the
// dequantizing FMA. Otherwise the bias is folded into the FMA's addend, which
// costs one rounding of kMagic * scale in that addend: an error below 0.75
// steps of the integer logit grid, used only while kMagic * scale <= 2048
// (error <= 2^-13 in the exponent of P).
template <int DP, bool MASK, bool CAUSAL, bool EXACT>
__device__ __forceinline__ void softmax_step(SoftmaxState<DP / 32>& st, v16i (&s)[4],
                                             const uint8_t* vsm, const float* skp, int k0,
                                             int Lk, int qi, int hh, int lq, float scq) {
    constexpr int NU = DP / 32;
    if (MASK) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 32 * t + 8 * (r / 4) + 4 * hh + (r % 4);
                const bool masked = key >= Lk || (CAUSAL && key > qi);
                if (masked) s[t][r] = 0;             // below every biased logit
            }
    }
    // row max per 64-key sub-block on the biased integers, then in the log2 domain
    float sc[2], cb[2], mlog[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        int mx = 0;
#pragma unroll
        for (int t = 2 * sb; t < 2 * sb + 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = max(mx, s[t][r]);
        // lanes l and l^32 hold the two key halves of the same query
        const auto pr = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
        mx = max(static_cast<int>(pr[0]), static_cast<int>(pr[1]));
        sc[sb] = scq * skp[(k0 >> 6) + sb];
        cb[sb] = kMagic * sc[sb];
        mlog[sb] = (mx == 0) ? -INFINITY : (__int_as_float(mx) - kMagic) * sc[sb];
    }
    const float m_new = fmaxf(st.m, fmaxf(mlog[0], mlog[1]));
    const float mref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mref);

    // P = 2^(logit - m) * 2^8 -> E4M3, packed as the B operand of the PV product
    v8i pb[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const float bias = EXACT ? 8.0f - mref : 8.0f - mref - cb[sb];
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) {
            const int t = 2 * sb + wd / 4;
            const int r0 = 4 * (wd % 4);
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sv = s[t][r0 + e];
                const float f = EXACT ? __int_as_float(sv) - kMagic : __int_as_float(sv);
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f, sc[sb], bias));
                if (MASK && sv == 0) p[e] = 0.0f;
            }
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
            pb[sb][wd] = word;
        }
    }

    // normaliser: the sum of the FP8 probabilities, from an all-ones A operand
    const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
    v16f lacc = {};
    lacc = mfma_f8(ones, pb[0], lacc);
    lacc = mfma_f8(ones, pb[1], lacc);
    st.l = alpha * st.l + lacc[0];

    // O^T = alpha * O^T + V^T . P^T
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.o[u][r] *= alpha;
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const uint8_t* vsb = vsm + sb * DP * 64;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int d = 32 * u + lq;
            const v4i lo = *reinterpret_cast<const v4i*>(&vsb[d * 64 + 16 * (swz_row<64>(d) ^ (2 * hh))]);
            const v4i hi = *reinterpret_cast<const v4i*>(&vsb[d * 64 + 16 * (swz_row<64>(d) ^ (2 * hh + 1))]);
            const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            st.o[u] = mfma_f8(va, pb[sb], st.o[u]);
        }
    }
    st.m = m_new;
}

struct TileCoords {
    int b, hq, hkv, qt, q0, qi, w, l, lq, hh;
    int64_t kvh, qrow;
};

// Everything after the block -> tile mapping; EXACT is uniform over the workgroup.
template <int DP, typename T, bool CAUSAL, bool VEC_OUT, bool EXACT>
__device__ __forceinline__ void attn_tile(const AttnArgs& a, const TileCoords& tc,
                                          uint8_t (*ks)[KBYTES128], uint8_t (*vs)[KBYTES128]) {
    constexpr int NC = DP / 32;
    constexpr int NU = DP / 32;
    constexpr int KBYTES = kBK * DP;
    const int w = tc.w, l = tc.l, lq = tc.lq, hh = tc.hh, qi = tc.qi, q0 = tc.q0;

    v4i qb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        qb[c] = *reinterpret_cast<const v4i*>(a.qhat + tc.qrow * DP + 32 * c + 16 * hh);
    const float scq = a.sq[tc.qrow] * a.scale_log2;

    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.khat) + tc.kvh * a.Lk_pad * DP;
    const uint8_t* vg = a.vhat + tc.kvh * a.nkb * (DP * 64);
    const float* skp = a.sk + tc.kvh * a.nkb;

    // blocks [0, nfull) need no mask; [nfull, nkblk) do
    int nkblk = a.Lk_pad / kBK;
    int nfull = a.Lk / kBK;
    if (CAUSAL) {
        const int last = min(a.Lk, tc.qt * kBQ + kBQ);     // keys 0..last-1 can be visible
        nkblk = (last + kBK - 1) / kBK;
        nfull = min(nfull, (tc.qt * kBQ) / kBK);
    }

    SoftmaxState<NU> st;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[u][r] = 0.0f;
    st.m = -INFINITY;
    st.l = 0.0f;

    stage_block<DP>(kg, vg, ks[0], vs[0], w, l);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    int kb = 0;
    for (; kb < nfull; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nkblk)
            stage_block<DP>(kg + static_cast<int64_t>(kb + 1) * KBYTES,
                            vg + static_cast<int64_t>(kb + 1) * KBYTES, ks[buf ^ 1], vs[buf ^ 1], w, l);
        v16i s[4];
        qk_block<DP>(s, ks[buf], qb, lq, hh);
        softmax_step<DP, false, CAUSAL, EXACT>(st, s, vs[buf], skp, kb * kBK, a.Lk, qi, hh, lq, scq);
        // the next block's copies must have landed before anyone reads them,
        // and nobody may overwrite this block's buffers before all waves are done
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (; kb < nkblk; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nkblk)
            stage_block<DP>(kg + static_cast<int64_t>(kb + 1) * KBYTES,
                            vg + static_cast<int64_t>(kb + 1) * KBYTES, ks[buf ^ 1], vs[buf ^ 1], w, l);
        const int k0 = kb * kBK;
        if (!CAUSAL || k0 <= q0 + 31) {            // some key of the block is visible to this wave
            v16i s[4];
            qk_block<DP>(s, ks[buf], qb, lq, hh);
            softmax_step<DP, true, CAUSAL, true>(st, s, vs[buf], skp, k0, a.Lk, qi, hh, lq, scq);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: O = O^T * s_v[d] / l, crop to (Lq, D), cast ----
    if (qi >= a.Lq) return;
    const float inv_l = 1.0f / st.l;
    const float* vmax = a.vmax + tc.kvh * DP;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + tc.b * a.os0 + tc.hq * a.os1 + static_cast<int64_t>(qi) * a.os2;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * u + 8 * r4 + 4 * hh;
            if (d0 >= a.D) continue;
            const float4 vm = *reinterpret_cast<const float4*>(vmax + d0);
            const float vmv[4] = {vm.x, vm.y, vm.z, vm.w};
            uint16_t h4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                h4[e] = from_f32<T>(st.o[u][4 * r4 + e] * (vmv[e] * (1.0f / 448.0f)) * inv_l);
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

template <int DP, typename T, bool CAUSAL, bool VEC_OUT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    __shared__ __align__(16) uint8_t ks[2][KBYTES128];
    __shared__ __align__(16) uint8_t vs[2][KBYTES128];
    __shared__ float red[4];

    TileCoords tc;
    const int tid = threadIdx.x;
    tc.w = tid >> 6;
    tc.l = tid & 63;
    tc.lq = tc.l & 31;
    tc.hh = tc.l >> 5;

    // ---- block -> (b, hq, query tile), XCD-aware ----
    {
        const int n = blockIdx.x;
        const int N = gridDim.x;
        const int full = N / 8;
        // workgroups are dealt to the 8 XCDs round robin; this makes
        // consecutive logical tiles (same kv head) land on the same XCD
        const int L = (n < full * 8) ? (n % 8) * full + n / 8 : n;
        tc.qt = L % a.nqt;
        int rest = L / a.nqt;
        const int g = rest % a.G;
        rest /= a.G;
        tc.hkv = rest % a.Hkv;
        tc.b = rest / a.Hkv;
        tc.hq = tc.hkv * a.G + g;
    }
    tc.q0 = tc.qt * kBQ + tc.w * 32;
    tc.qi = tc.q0 + tc.lq;
    tc.kvh = static_cast<int64_t>(tc.b) * a.Hkv + tc.hkv;
    tc.qrow = (static_cast<int64_t>(tc.b) * a.Hq + tc.hq) * a.Lq_pad + tc.qi;

    // The largest dequantization scale this workgroup can meet decides whether
    // the one-FMA form is accurate enough (see softmax_step).
    float mq = a.sq[tc.qrow];
    for (int off = 32; off >= 1; off >>= 1) mq = fmaxf(mq, __shfl_xor(mq, off, 64));
    float mk = 0.0f;
    const float* skp = a.sk + tc.kvh * a.nkb;
    for (int i = tid; i < a.nkb; i += 256) mk = fmaxf(mk, skp[i]);
    for (int off = 32; off >= 1; off >>= 1) mk = fmaxf(mk, __shfl_xor(mk, off, 64));
    if (tc.l == 0) {
        red[tc.w] = mq;
        red[tc.w] = fmaxf(red[tc.w], 0.0f);
    }
    __syncthreads();
    mq = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    if (tc.l == 0) red[tc.w] = mk;
    __syncthreads();
    mk = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const bool exact = kMagic * (mq * a.scale_log2) * mk > 2048.0f;

    if (exact)
        attn_tile<DP, T, CAUSAL, VEC_OUT, true>(a, tc, ks, vs);
    else
        attn_tile<DP, T, CAUSAL, VEC_OUT, false>(a, tc, ks, vs);
}

// int32 logits of one head through the same staging and tile routine.
template <int DP>
__global__ __launch_bounds__(256) void qk_dump_kernel(AttnArgs a) {
    __shared__ __align__(16) uint8_t ks[2][KBYTES128];
    __shared__ __align__(16) uint8_t vs[2][KBYTES128];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, hh = l >> 5;
    const int b = a.dump_b, hq = a.dump_hq, hkv = hq / a.G;
    const int qi = blockIdx.x * kBQ + w * 32 + lq;
    const int64_t qrow = (static_cast<int64_t>(b) * a.Hq + hq) * a.Lq_pad + qi;
    const int64_t kvh = static_cast<int64_t>(b) * a.Hkv + hkv;
    v4i qb[DP / 32];
#pragma unroll
    for (int c = 0; c < DP / 32; ++c)
        qb[c] = *reinterpret_cast<const v4i*>(a.qhat + qrow * DP + 32 * c + 16 * hh);
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.khat) + kvh * a.Lk_pad * DP;
    const uint8_t* vg = a.vhat + kvh * a.nkb * (DP * 64);
    const int nkblk = a.Lk_pad / kBK;
    for (int kb = 0; kb < nkblk; ++kb) {
        stage_block<DP>(kg + static_cast<int64_t>(kb) * kBK * DP, vg + static_cast<int64_t>(kb) * kBK * DP,
                        ks[0], vs[0], w, l);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        v16i s[4];
        qk_block<DP>(s, ks[0], qb, lq, hh);
        int32_t* out = a.dump + static_cast<int64_t>(qi) * a.Lk_pad + kb * kBK;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                out[32 * t + 8 * (r / 4) + 4 * hh + (r % 4)] = s[t][r] - kMagicBits;
        __syncthreads();
    }
}

template <int DP, typename T>
hipError_t attn_dispatch(const AttnArgs& a, bool causal, bool vec_out, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.nqt) * a.Hq * a.B;
    if (causal) {
        if (vec_out) attn_kernel<DP, T, true, true><<<grid, 256, 0, s>>>(a);
        else attn_kernel<DP, T, true, false><<<grid, 256, 0, s>>>(a);
    } else {
        if (vec_out) attn_kernel<DP, T, false, true><<<grid, 256, 0, s>>>(a);
        else attn_kernel<DP, T, false, false><<<grid, 256, 0, s>>>(a);
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
        qk_dump_kernel<64><<<grid, 256, 0, s>>>(a);
    else
        qk_dump_kernel<128><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sage
