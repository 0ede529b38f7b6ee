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

#include <type_traits>

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
// k ^ swz_row<RB>(i). gfx950 LDS has 64 four-byte banks (a 256-byte period) and
// serves a ds_read_b128 sixteen lanes at a time; the operand reads have 16
// consecutive lanes on 16 consecutive rows at the same logical chunk, so the
// rows that share a bank period (256 / RB of them) are told apart by the row
// offset and the rest by the XOR mask: the 16 lanes hit 16 distinct slots.
template <int RB>
__device__ __forceinline__ int swz_row(int i) {
    constexpr int RPP = 256 / RB;                        // rows per 256-byte bank period
    constexpr int CPR = RB / 16;                         // chunks per row
    return (i / RPP) % CPR;
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

// One 16-byte-per-lane global -> LDS copy; the LDS address must be wave-uniform
// (lane i lands at l + 16 i).
__device__ __forceinline__ void copy16_to_lds(const uint8_t* g, uint8_t* l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0);
}

// Direct global -> LDS copy of one 128-key block of Khat (128 x DP bytes,
// swizzled rows) and of V^T (two 64-key sub-blocks of DP x 64 bytes). Each
// instruction moves 64 lanes x 16 bytes into 1 KB of LDS at a wave-uniform
// base, lane i landing at base + 16 i, so each lane fetches the global chunk
// that the swizzle places at its slot. The per-lane source offsets do not
// depend on the block and are computed once (StageOffsets).
template <int DP>
struct StageOffsets {
    static constexpr int KCH = kBK * DP / 16;   // 16-byte chunks per tensor block
    static constexpr int PER_WAVE = KCH / 4;
    static constexpr int N = PER_WAVE / 64;     // instructions per tensor per wave
    uint32_t k[N], v[N];
    __device__ __forceinline__ void init(int w, int l) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int c = w * PER_WAVE + n * 64 + l;     // LDS chunk slot of this lane
            const int ki = c / (DP / 16), kp = c % (DP / 16);
            k[n] = 16u * static_cast<uint32_t>(ki * (DP / 16) + (kp ^ swz_row<DP>(ki)));
            const int sb = c / (DP * 4), rem = c % (DP * 4);
            const int vd = rem / 4, vp = rem % 4;
            v[n] = 16u * static_cast<uint32_t>(sb * (DP * 4) + vd * 4 + (vp ^ swz_row<64>(vd)));
        }
    }
    // copy the block at kg / vg into the LDS buffers kl / vl
    __device__ __forceinline__ void stage(const uint8_t* kg, const uint8_t* vg, uint8_t* kl,
                                          uint8_t* vl, int w) const {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            copy16_to_lds(kg + k[n], kl + 16 * (w * PER_WAVE + n * 64));
            copy16_to_lds(vg + v[n], vl + 16 * (w * PER_WAVE + n * 64));
        }
    }
};

// Per-lane byte offsets of the matrix-core operands inside an LDS block; the
// tile / sub-block indices only add constants.
template <int DP>
struct LdsOffsets {
    int k[DP / 32];     // K chunk c of row lq (tile t adds 32 * t * DP)
    int v[2];           // V^T halves of row lq (tile u adds 32 * u * 64, sub-block sb adds sb * DP * 64)
    __device__ __forceinline__ void init(int lq, int hh) {
#pragma unroll
        for (int c = 0; c < DP / 32; ++c) k[c] = lq * DP + 16 * (swz_row<DP>(lq) ^ (2 * c + hh));
        v[0] = lq * 64 + 16 * (swz_row<64>(lq) ^ (2 * hh));
        v[1] = lq * 64 + 16 * (swz_row<64>(lq) ^ (2 * hh + 1));
    }
};

// The wave's Q operands (B of the QK^T product): DP / 32 chunks of 16 bytes.
template <int DP>
struct QOps {
    v4i c[DP / 32];
};

// S^T for one 128-key block: 4 tiles of 32 keys, accumulators biased by
// kMagicBits. Chunks are the outer loop so that four independent accumulation
// chains are in flight on the matrix core.
template <int DP>
__device__ __forceinline__ void qk_block(v16i (&s)[4], const uint8_t* ksm, const LdsOffsets<DP>& lo,
                                         const QOps<DP>& qb) {
    const v16i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                        kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                        kMagicBits, kMagicBits, kMagicBits, kMagicBits};
#pragma unroll
    for (int c = 0; c < DP / 32; ++c) {
        v4i ka[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            ka[t] = *reinterpret_cast<const v4i*>(ksm + lo.k[c] + 32 * t * DP);
#pragma unroll
        for (int t = 0; t < 4; ++t) s[t] = mfma_i8(ka[t], qb.c[c], c == 0 ? magic : s[t]);
    }
}

// max over the 32 biased logits of one 64-key sub-block (tiles t0, t0 + 1), as
// a shallow tree of three-input maxima.
__device__ __forceinline__ int subblock_max(const v16i& a, const v16i& b) {
    int m[11];
#pragma unroll
    for (int i = 0; i < 5; ++i) m[i] = max(max(a[3 * i], a[3 * i + 1]), a[3 * i + 2]);
    m[5] = max(a[15], b[15]);
#pragma unroll
    for (int i = 0; i < 5; ++i) m[6 + i] = max(max(b[3 * i], b[3 * i + 1]), b[3 * i + 2]);
    const int x = max(max(m[0], m[1]), m[2]);
    const int y = max(max(m[3], m[4]), m[5]);
    const int z = max(max(m[6], m[7]), m[8]);
    const int u = max(m[9], m[10]);
    return max(max(x, y), max(z, u));
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
                                             const uint8_t* vsm, const LdsOffsets<DP>& lo,
                                             const float* skp, int k0, int Lk, int qi, int hh,
                                             float scq) {
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
        int mx = subblock_max(s[2 * sb], s[2 * sb + 1]);
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
            const v4i x0 = *reinterpret_cast<const v4i*>(vsb + lo.v[0] + 32 * u * 64);
            const v4i x1 = *reinterpret_cast<const v4i*>(vsb + lo.v[1] + 32 * u * 64);
            const v8i va = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            st.o[u] = mfma_f8(va, pb[sb], st.o[u]);
        }
    }
    st.m = m_new;
}

// One step on block kb held in LDS buffer BUF, prefetching block kb + 1 into
// the other buffer.
template <int DP, bool CAUSAL, bool EXACT, int BUF, bool MASK>
__device__ __forceinline__ void tile_step(SoftmaxState<DP / 32>& st, const StageOffsets<DP>& so,
                                          const LdsOffsets<DP>& lo, const QOps<DP>& qb,
                                          uint8_t (*ks)[KBYTES128], uint8_t (*vs)[KBYTES128],
                                          const uint8_t* kg, const uint8_t* vg, const float* skp,
                                          int kb, int nkblk, int Lk, int q0, int qi, int w, int hh,
                                          float scq) {
    constexpr int KBYTES = kBK * DP;
    if (kb + 1 < nkblk)
        so.stage(kg + static_cast<int64_t>(kb + 1) * KBYTES, vg + static_cast<int64_t>(kb + 1) * KBYTES,
                 ks[BUF ^ 1], vs[BUF ^ 1], w);
    const int k0 = kb * kBK;
    if (!MASK || !CAUSAL || k0 <= q0 + 31) {     // some key of the block is visible to this wave
        v16i s[4];
        qk_block<DP>(s, ks[BUF], lo, qb);
        softmax_step<DP, MASK, CAUSAL, MASK || EXACT>(st, s, vs[BUF], lo, skp, k0, Lk, qi, hh, scq);
    }
    // the next block's copies must have landed before anyone reads them, and
    // nobody may overwrite this block's buffers before all waves are done
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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

    QOps<DP> qb;
#pragma unroll
    for (int c = 0; c < NC; ++c)
        qb.c[c] = *reinterpret_cast<const v4i*>(a.qhat + tc.qrow * DP + 32 * c + 16 * hh);
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

    StageOffsets<DP> so;
    so.init(w, l);
    LdsOffsets<DP> lo;
    lo.init(lq, hh);

    so.stage(kg, vg, ks[0], vs[0], w);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

#define SAGE_STEP(BUF, MASK, KB)                                                                   \
    tile_step<DP, CAUSAL, EXACT, BUF, MASK>(st, so, lo, qb, ks, vs, kg, vg, skp, KB, nkblk, a.Lk, \
                                            q0, qi, w, hh, scq)
    int kb = 0;
    for (; kb + 1 < nfull; kb += 2) {
        SAGE_STEP(0, false, kb);
        SAGE_STEP(1, false, kb + 1);
    }
    if (kb < nfull) {
        SAGE_STEP(0, false, kb);
        ++kb;
    }
    for (; kb < nkblk; ++kb) {
        if (kb & 1)
            SAGE_STEP(1, true, kb);
        else
            SAGE_STEP(0, true, kb);
    }
#undef SAGE_STEP

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
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
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
    tc.w = __builtin_amdgcn_readfirstlane(tc.w);     // wave-uniform (lets branches on it stay scalar)
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
    QOps<DP> qb;
#pragma unroll
    for (int c = 0; c < DP / 32; ++c)
        qb.c[c] = *reinterpret_cast<const v4i*>(a.qhat + qrow * DP + 32 * c + 16 * hh);
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.khat) + kvh * a.Lk_pad * DP;
    const uint8_t* vg = a.vhat + kvh * a.nkb * (DP * 64);
    const int nkblk = a.Lk_pad / kBK;
    StageOffsets<DP> so;
    so.init(w, l);
    LdsOffsets<DP> lo;
    lo.init(lq, hh);
    for (int kb = 0; kb < nkblk; ++kb) {
        so.stage(kg + static_cast<int64_t>(kb) * kBK * DP, vg + static_cast<int64_t>(kb) * kBK * DP,
                 ks[0], vs[0], w);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        v16i s[4];
        qk_block<DP>(s, ks[0], lo, qb);
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
