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
// it comes from a 16 x 16 x 128 matrix-core product per 64 keys whose A
// operand selects each query's row (accumulated over the whole tile), or,
// when the head dim is padded, from a channel of ones that the prologue puts
// into V^T.
//
// Workgroup: 4 waves = 128 queries. Key blocks of 128 tokens (2 quantization
// blocks of 64) are copied global -> LDS directly (no register staging),
// double buffered with one barrier per step; LDS rows are XOR-swizzled in
// 16-byte chunks so the operand reads are free of bank conflicts. Blocks that
// need no mask (all but the causal diagonal and the ragged tail) run a
// separate loop without any masking code. The Q codes come either from the
// workspace or, on the one-call paths, from the input q, quantized by each
// tile for its own rows with the prologue's per-token rule.
#pragma once

#include "sage_kernels.h"

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include <type_traits>

namespace sage {
namespace {

#include "quant_rules.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;


__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// 16-bit P.V product (32 x 32 x 16, FP32 accumulation) in the input format T.
template <typename T>
__device__ __forceinline__ v16f mfma_16(v4i a, v4i b, v16f c);
template <>
__device__ __forceinline__ v16f mfma_16<__half>(v4i a, v4i b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ v16f mfma_16<__hip_bfloat16>(v4i a, v4i b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// 16 x 16 x 32 product (FP32 accumulation) in the 16-bit format T; the same
// lane grouping as mfma_f8_16 with 8 keys per lane and group.
template <typename T>
__device__ __forceinline__ v4f mfma16_16(v4i a, v4i b, v4f c);
template <>
__device__ __forceinline__ v4f mfma16_16<__half>(v4i a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ v4f mfma16_16<__hip_bfloat16>(v4i a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// Two fp32 values rounded to nearest even in the format T, packed (x0 low).
template <typename T>
__device__ __forceinline__ int pack2_16(float x0, float x1);
template <>
__device__ __forceinline__ int pack2_16<__half>(float x0, float x1) {
    const v2f f = {x0, x1};
    return __builtin_bit_cast(int, __builtin_convertvector(f, v2h));
}
template <>
__device__ __forceinline__ int pack2_16<__hip_bfloat16>(float x0, float x1) {
    const v2f f = {x0, x1};
    return __builtin_bit_cast(int, __builtin_convertvector(f, v2bf));
}

__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
    // format selectors 0/0: both operands FP8 E4M3; no block scales.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16 x 16 x 128 FP8 product (E4M3 operands, no block scales). Lane l holds A
// row l % 16 and B column l % 16 for the keys of group l / 16; D element i of
// lane l is row 4 (l / 16) + i of column l % 16.
__device__ __forceinline__ v4f mfma_f8_16(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The A operand that turns the 16 x 16 x 128 product of an FP8 P operand of
// the 32 x 32 x 64 product (query l % 32, key half l / 32 on lane l) into its
// row sums: the 64 lanes fall into key groups g = l / 16 that hold queries
// 16 (g % 2) .. + 15, so row 0 takes ones on the groups of queries 0..15 and
// row 1 on those of queries 16..31. Lane n < 16 then holds the sum of query n
// in D element 0 and of query n + 16 in element 1.
// one: the word of ones of the P format (four E4M3 or two 16-bit 1.0s).
__device__ __forceinline__ int rowsum_sel_word(int l, int one) {
    const int m = l % 16, g = l / 16;
    return ((m == 0 && g % 2 == 0) || (m == 1 && g % 2 == 1)) ? one : 0;
}

// The A operand from its word (N registers), built where it is used: the
// empty statement keeps the compiler from hoisting the copies out of the
// loop and holding them in registers for the whole tile.
template <int N>
__device__ __forceinline__ int __attribute__((ext_vector_type(N))) rowsum_sel(int word) {
    asm volatile("" : "+v"(word));
    int __attribute__((ext_vector_type(N))) sel;
#pragma unroll
    for (int i = 0; i < N; ++i) sel[i] = word;
    return sel;
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

// One 16-byte-per-lane copy from a buffer into LDS: lane i reads bytes
// off .. off + 15 of the buffer r and lands at l + 16 i (l wave-uniform).
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t* l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 16, static_cast<int>(off), 0, 0, 0);
}

// x, known to be the same on every lane, as a scalar value
__device__ __forceinline__ int64_t wave_uniform(int64_t x) {
    const uint64_t u = static_cast<uint64_t>(x);
    const uint64_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((hi << 32) | __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u)));
}

// The two K scales of 128-key block kb (skp wave-uniform), through the scalar
// cache into scalar registers. The workspace is written only by earlier
// launches, whose writes a new launch sees through the scalar cache as well.
__device__ __forceinline__ void load_kscales(const float* skp, int kb, float (&skb)[2]) {
    typedef __attribute__((address_space(4))) const v2f cv2f;
    const cv2f* p = (const cv2f*)(reinterpret_cast<uintptr_t>(skp + 2 * kb));
    const v2f v = *p;
    skb[0] = v[0];
    skb[1] = v[1];
}

// Buffer descriptor of the bytes [base, base + bytes) (base wave-uniform):
// the block base stays in scalar registers and every lane holds only its
// 32-bit offset; an offset outside the range would read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0), bytes,
                                             0x00020000);   // raw byte buffer, 32-bit data format
}

// Direct global -> LDS copy of one 128-key block of Khat (128 x DP bytes,
// swizzled rows) and of V^T (two 64-key sub-blocks of DP x 64 elements of VB
// bytes), shared by the NW waves of the workgroup. Each instruction moves 64
// lanes x 16 bytes into 1 KB of LDS at a wave-uniform base, lane i landing at
// base + 16 i, so each lane fetches the global chunk that the swizzle places
// at its slot. The per-lane source offsets do not depend on the block and are
// computed once.
template <int DP, int NW, int VB>
struct StageOffsets {
    static constexpr int KCH = kBK * DP / 16;        // 16-byte chunks per K block
    static constexpr int VCH = kBK * DP * VB / 16;   // 16-byte chunks per V^T block
    static constexpr int KPW = KCH / NW, VPW = VCH / NW;
    static constexpr int NK = KPW / 64, NV = VPW / 64;   // instructions per wave
    static constexpr int VROW = 64 * VB;                 // bytes per V^T row (64 keys)
    static_assert(NK >= 1 && NV >= 1 && KPW % 64 == 0 && VPW % 64 == 0, "whole wave copies");
    uint32_t k[NK], v[NV];
    __device__ __forceinline__ void init(int w, int l) {
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            const int c = w * KPW + n * 64 + l;          // LDS chunk slot of this lane
            const int ki = c / (DP / 16), kp = c % (DP / 16);
            k[n] = 16u * static_cast<uint32_t>(ki * (DP / 16) + (kp ^ swz_row<DP>(ki)));
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            constexpr int CPR = VROW / 16;               // chunks per V^T row
            const int c = w * VPW + n * 64 + l;
            const int sb = c / (DP * CPR), rem = c % (DP * CPR);
            const int vd = rem / CPR, vp = rem % CPR;
            v[n] = 16u * static_cast<uint32_t>(sb * (DP * CPR) + vd * CPR + (vp ^ swz_row<VROW>(vd)));
        }
    }
    // copy the block at kg / vg (wave-uniform) into the LDS buffers kl / vl
    __device__ __forceinline__ void stage(const uint8_t* kg, const uint8_t* vg, uint8_t* kl,
                                          uint8_t* vl, int w) const {
        const __amdgpu_buffer_rsrc_t rk = block_rsrc(kg, 16 * KCH);
        const __amdgpu_buffer_rsrc_t rv = block_rsrc(vg, 16 * VCH);
#pragma unroll
        for (int n = 0; n < NK; ++n) copy16_to_lds(rk, k[n], kl + 16 * (w * KPW + n * 64));
#pragma unroll
        for (int n = 0; n < NV; ++n) copy16_to_lds(rv, v[n], vl + 16 * (w * VPW + n * 64));
    }
};

// Per-lane byte offsets of the matrix-core operands inside an LDS block; the
// tile / sub-block indices only add constants.
template <int DP, bool PV16>
struct LdsOffsets {
    int k[DP / 32];     // K chunk c of row lq (tile t adds 32 * t * DP)
    // FP8: V^T halves 0/1 of row lq (tile u adds 32 * u * 64, sub-block sb adds sb * DP * 64).
    // 16-bit: the 16 bytes of 16-key group g of row lq (tile u adds 32 * u * 128,
    // sub-block sb adds sb * DP * 128).
    int v[PV16 ? 4 : 2];
    __device__ __forceinline__ void init(int lq, int hh) {
#pragma unroll
        for (int c = 0; c < DP / 32; ++c) k[c] = lq * DP + 16 * (swz_row<DP>(lq) ^ (2 * c + hh));
        if (PV16) {
#pragma unroll
            for (int g = 0; g < 4; ++g) v[g] = lq * 128 + 16 * (swz_row<128>(lq) ^ (2 * g + hh));
        } else {
            v[0] = lq * 64 + 16 * (swz_row<64>(lq) ^ (2 * hh));
            v[1] = lq * 64 + 16 * (swz_row<64>(lq) ^ (2 * hh + 1));
        }
    }
};

// The wave's Q operands (B of the QK^T product): DP / 32 chunks of 16 bytes.
template <int DP>
struct QOps {
    v4i c[DP / 32];
};

// S^T for one 128-key block: 4 tiles of 32 keys, accumulators biased by
// kMagicBits. Tiles are the outer loop: the first tiles' logits are complete
// after a quarter and a half of the products, so the softmax's maxima over
// them can run under the remaining products (a dependent chain of 32 x 32
// products costs the matrix core no extra cycles).
template <int DP, bool PV16>
__device__ __forceinline__ void qk_block(v16i (&s)[4], const uint8_t* ksm, const LdsOffsets<DP, PV16>& lo,
                                         const QOps<DP>& qb) {
    const v16i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                        kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                        kMagicBits, kMagicBits, kMagicBits, kMagicBits};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        v4i ka[DP / 32];
#pragma unroll
        for (int c = 0; c < DP / 32; ++c)
            ka[c] = *reinterpret_cast<const v4i*>(ksm + lo.k[c] + 32 * t * DP);
#pragma unroll
        for (int c = 0; c < DP / 32; ++c) s[t] = mfma_i8(ka[c], qb.c[c], c == 0 ? magic : s[t]);
    }
    // operand reads ahead of the products, as many as the registers allow
    // (the logits' registers are still free here), so that few products
    // wait for LDS
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * (DP / 32), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * (DP / 32), 0);
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

// The FP8 path's lazy reference (log2 units; see softmax_step).
constexpr float kLazyOver = 2.0f;
constexpr float kLazySlack = 0.75f;

template <int NU>
struct SoftmaxState {
    v16f o[NU];
    float m;
    float l;
    v4f ls;        // without a channel of ones: the row sums of P (rowsum_sel layout)
};

// One 128-key step of the online softmax for the wave's 32 queries, and the
// P.V product. Causal: keys after qlim (this lane's last visible key) are
// masked. PV16: P is rounded to the 16-bit input format T and multiplies
// the 16-bit V^T (the INT8-QK / 16-bit-PV variant); otherwise P * 2^8 is
// converted to E4M3 and multiplies the FP8 V^T.
// EXACT: take (bits - bias) back to the integer exactly (Sterbenz) before the
// dequantizing FMA. Otherwise the bias is folded into the FMA's addend, which
// costs one rounding of kMagic * scale in that addend: an error below 0.75
// steps of the integer logit grid, used only while kMagic * scale <= 2048
// (error <= 2^-14 in the exponent of P while the addend stays below 2048;
// the exact form costs 64 more vector instructions per step). The limit is
// set by rows where one key dominates: there a rounding of P to E4M3 that
// lands on the other side of a midpoint than the exact value's moves the
// output by several hundredths, and with the next binade's bound (2^-13 up
// to 4096) such rows broke the max-abs bar.
//
// AFTER: a step after the tile's first one on unmasked blocks, where every
// row already has a finite reference (unmasked blocks come before masked
// ones, so the first step was unmasked too and gave each row a visible
// key): the first-block cases are left out.
template <int DP, typename T, bool MASK, bool CAUSAL, bool EXACT, bool PV16, bool LCH, bool AFTER = false>
__device__ __forceinline__ void softmax_step(SoftmaxState<DP / 32>& st, v16i (&s)[4],
                                             const uint8_t* vsm, const LdsOffsets<DP, PV16>& lo,
                                             float sc0, float sc1, int k0, int Lk, int qlim, int hh) {
    constexpr int NU = DP / 32;
    if (MASK) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 32 * t + 8 * (r / 4) + 4 * hh + (r % 4);
                const bool masked = key >= Lk || (CAUSAL && key > qlim);
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
        sc[sb] = sb ? sc1 : sc0;
        cb[sb] = kMagic * sc[sb];
        // (a biased logit is 0 only where a mask cleared it)
        mlog[sb] = (MASK && mx == 0) ? -INFINITY : (__int_as_float(mx) - kMagic) * sc[sb];
    }
    // FP8: a lazy reference above the maximum (log2 units). The first block
    // with a visible key sets a row's reference to its maximum plus
    // kLazyOver; later blocks leave it unless their maximum passes it by more
    // than kLazySlack, and then set it to their maximum plus kLazyOver. So P
    // stays at most 2^kLazySlack (P * 2^8 <= 430.5, below 448, the E4M3
    // maximum), and the wave rescales O^T and l only when some row's
    // reference moved after its first block, which for most blocks after the
    // first it does not. 16-bit P: lazy maxima. The wave keeps its rows'
    // running maxima while no row's block maximum passes its own by more
    // than 2^8, so P < 2^8 and most blocks after the first few skip the
    // rescale of O^T and l.
    const float m_blk = fmaxf(mlog[0], mlog[1]);
    bool grow;
    float m_new;
    if constexpr (PV16) {
        grow = __any(m_blk > st.m + 8.0f);
        m_new = grow ? fmaxf(st.m, m_blk) : st.m;
    } else if constexpr (AFTER) {
        const bool move = m_blk > st.m + kLazySlack;
        grow = __any(move);
        m_new = move ? m_blk + kLazyOver : st.m;
    } else {
        const bool first = st.m == -INFINITY;
        const bool move = first ? m_blk != -INFINITY : m_blk > st.m + kLazySlack;
        grow = __any(move && !first);
        m_new = move ? m_blk + kLazyOver : st.m;
    }
    const float mref = (AFTER || m_new != -INFINITY) ? m_new : 0.0f;
    // 1 where the reference stayed, 0 on a row's first visible block (O^T and
    // l are still 0 there)
    const float alpha = grow || !PV16 ? __builtin_amdgcn_exp2f(st.m - mref) : 1.0f;
    // P = 2^(logit - m) (times 2^8 for FP8)
    constexpr float kPScaleLog2 = PV16 ? 0.0f : 8.0f;

    if constexpr (!PV16) {
        // P * 2^8 -> E4M3, packed as the B operand of the FP8 P.V product
        v8i pb[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const float bias = EXACT ? kPScaleLog2 - mref : kPScaleLog2 - mref - cb[sb];
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
                // the first conversion writes the low half of the word and the
                // second the high half, so the word's initial bits are never
                // read: start from a register already holding a value
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
                pb[sb][wd] = word;
            }
        }

        // O^T = alpha * O^T + V^T . P^T, and l = alpha * l + the sum of the
        // FP8 probabilities: a 16 x 16 x 128 product accumulated over the
        // whole tile, unless V^T carries a channel of ones (then the P.V
        // product below accumulates l in O^T channel D)
        if (grow) {
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[u][r] *= alpha;
            if constexpr (!LCH) {
                // lane n < 16 holds the sums of queries n and n + 16
                const float alpha_hi = __shfl(alpha, (static_cast<int>(threadIdx.x) & 15) + 16, 64);
                st.ls[0] *= alpha;
                st.ls[1] *= alpha_hi;
            }
        }
        if constexpr (!LCH) {
            const v8i sel = rowsum_sel<8>(rowsum_sel_word(static_cast<int>(threadIdx.x) & 63, 0x38383838));
            st.ls = mfma_f8_16(sel, pb[0], st.ls);
            st.ls = mfma_f8_16(sel, pb[1], st.ls);
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
        // the V^T operand reads ahead of the products
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * NU, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NU, 0);
    } else {
        // P rounded to T in pairs: per 16-key group g of a sub-block (tile
        // t = 2 sb + g / 2, accumulator rows 8 (g % 2) .. + 7) one B operand
        // of the 32 x 32 x 16 product; operand slot i (of 8) of lane half hh
        // holds key 32 t + 16 (g % 2) + 8 (i / 4) + 4 hh + i % 4, the key the
        // prologue stored at the matching V^T position.
        v4i ph[8];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const float bias = EXACT ? -mref : -mref - cb[sb];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int t = 2 * sb + g / 2;
                const int r0 = 8 * (g % 2);
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sv = s[t][r0 + e];
                    const float f = EXACT ? __int_as_float(sv) - kMagic : __int_as_float(sv);
                    p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f, sc[sb], bias));
                    if (MASK && sv == 0) p[e] = 0.0f;
                }
#pragma unroll
                for (int w = 0; w < 4; ++w) ph[4 * sb + g][w] = pack2_16<T>(p[2 * w], p[2 * w + 1]);
            }
        }
        // O^T = alpha * O^T + V^T . P^T, and l = alpha * l + the sum of the
        // rounded probabilities (16 x 16 x 32 products accumulated over the
        // tile), unless V^T carries a channel of ones
        if (grow) {
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[u][r] *= alpha;
            if constexpr (!LCH) {
                const float alpha_hi = __shfl(alpha, (static_cast<int>(threadIdx.x) & 15) + 16, 64);
                st.ls[0] *= alpha;
                st.ls[1] *= alpha_hi;
            }
        }
        if constexpr (!LCH) {
            const v4i sel = rowsum_sel<4>(rowsum_sel_word(static_cast<int>(threadIdx.x) & 63,
                                                          std::is_same<T, __half>::value ? 0x3C003C00 : 0x3F803F80));
#pragma unroll
            for (int i = 0; i < 8; ++i) st.ls = mfma16_16<T>(sel, ph[i], st.ls);
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const uint8_t* vsb = vsm + sb * DP * 128;
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const v4i va = *reinterpret_cast<const v4i*>(vsb + lo.v[g] + 32 * u * 128);
                    st.o[u] = mfma_16<T>(va, ph[4 * sb + g], st.o[u]);
                }
        }
    }
    st.m = m_new;
}

// Workgroup shape of each variant: NW waves of 32 query rows. The 16-bit
// variant's V^T blocks take twice the LDS, so it runs one workgroup of 8
// waves per compute unit where the FP8 variant runs two of 4; both keep two
// waves on every SIMD.
template <bool PV16>
struct Shape {
    static constexpr int NW = PV16 ? 8 : 4;      // waves per workgroup
    static constexpr int BQ = NW * 32;           // query rows per workgroup
    static constexpr int VB = PV16 ? 2 : 1;      // bytes per V^T element
    static constexpr int WG_PER_CU = PV16 ? 1 : 2;
};

// One step on block kb held in LDS buffer BUF, prefetching block kn into the
// other buffer when it is still in the range (kb_end is its end). Causal:
// query i sees keys j <= i + coff. on = false: the wave skips the block (its
// rows' block-mask flag is 0) but still takes part in the copies and barrier.
template <int DP, typename T, bool CAUSAL, bool EXACT, bool PV16, bool LCH, int BUF, bool MASK, bool AFTER = false>
__device__ __forceinline__ void tile_step(SoftmaxState<DP / 32>& st, const StageOffsets<DP, Shape<PV16>::NW, Shape<PV16>::VB>& so,
                                          const LdsOffsets<DP, PV16>& lo, const QOps<DP>& qb,
                                          uint8_t* const (&ks)[2], uint8_t* const (&vs)[2],
                                          const uint8_t* kg, const uint8_t* vg, const float* skp,
                                          float (&skb)[2], int kb, int kn, int kb_end, int Lk, int q0, int qi,
                                          int coff, int w, int hh, float scq, bool on) {
    constexpr int KBYTES = kBK * DP;
    constexpr int VBYTES = kBK * DP * Shape<PV16>::VB;
    const int k0 = kb * kBK;
    // skb holds this block's two K scales, loaded one step earlier through
    // the scalar cache, so that no wait for them involves the block copies
    // (vector-memory counter); the next block's are loaded at the end of the
    // step, after this block's LDS reads, whose waits would otherwise include
    // the scalar load as well.
    const float sc0 = scq * skb[0], sc1 = scq * skb[1];
    if (kn < kb_end)
        so.stage(kg + static_cast<int64_t>(kn) * KBYTES, vg + static_cast<int64_t>(kn) * VBYTES,
                 ks[BUF ^ 1], vs[BUF ^ 1], w);
    if (on && (!MASK || !CAUSAL || k0 <= q0 + 31 + coff)) {     // some key of the block is visible to this wave
        v16i s[4];
        qk_block<DP, PV16>(s, ks[BUF], lo, qb);
        softmax_step<DP, T, MASK, CAUSAL, MASK || EXACT, PV16, LCH, AFTER>(st, s, vs[BUF], lo, sc0, sc1, k0, Lk,
                                                                    qi + coff, hh);
    }
    if (kn < kb_end) load_kscales(skp, kn, skb);
    // the next block's copies must have landed before anyone reads them, and
    // nobody may overwrite this block's buffers before all waves are done
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

struct TileCoords {
    int b, hq, hkv, qt, sp, q0, qi, w, l, lq, hh;
    int Lq, Lk;             // lengths of this batch entry
    int64_t kvh, qrow;      // (b, kv head) index; workspace Q row of this lane's query
    int64_t kblk, qtok0;    // first workspace K block of (b, kv head); first input token of the entry
};

// The wave's Q operands (lane half hh holds bytes 32 c + 16 hh .. + 15 of its
// query's code row, c = 0 .. DP/32 - 1) and the lane's query scale s_q. From
// the workspace, or, when a.q is set, computed here from the input row by the
// prologue's per-token rule (s_q = amax / 127, codes rne(q * 127 / amax)
// clamped to +-127; rows past Lq give zero codes and scale), with the same
// arithmetic, so the codes and scale are the prologue's bit for bit. The two
// lane halves hold complementary halves of the row and exchange their maxima.
template <int DP, typename T>
__device__ __forceinline__ float load_q(const AttnArgs& a, const TileCoords& tc, QOps<DP>& qb) {
    constexpr int NC = DP / 32;
    if (a.q == nullptr) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qb.c[c] = *reinterpret_cast<const v4i*>(a.qhat + tc.qrow * DP + 32 * c + 16 * tc.hh);
        return a.sq[tc.qrow];
    }
    float x[NC][2][8];
    if (tc.qi < tc.Lq) {
        const uint16_t* row = static_cast<const uint16_t*>(a.q) + tc.b * a.qs0 + tc.hq * a.qs1 +
                              (tc.qtok0 + tc.qi) * a.qs2;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int d0 = 32 * c + 16 * tc.hh + 8 * g;
                if (a.q_vec) load8<T, true>(row, d0, a.D, x[c][g]);
                else load8<T, false>(row, d0, a.D, x[c][g]);
            }
    } else {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int u = 0; u < 8; ++u) x[c][g][u] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(x[c][g][u]));
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
    m = fmaxf(__int_as_float(static_cast<int>(pr[0])), __int_as_float(static_cast<int>(pr[1])));
    const float s = m / 127.0f;
    const float rc = m > 0.0f ? 127.0f / m : 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t word = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                word |= static_cast<uint32_t>(static_cast<uint8_t>(int8_code(x[c][k / 2][4 * (k % 2) + u], rc)))
                        << (8 * u);
            qb.c[c][k] = static_cast<int>(word);
        }
    return s;
}

// floor(x / m) for m > 0 and any sign of x
__device__ __forceinline__ int floor_div(int x, int m) { return x >= 0 ? x / m : -((m - 1 - x) / m); }

// The tile's split range of 128-key blocks [kb0, kb1) of its entry (trimmed at
// the causal diagonal); blocks [kb0, nfull) need no mask and [nfull, kb1) do.
// Causal: query i sees keys j <= i + coff.
struct KeyRange {
    int kb0, kb1, nfull, coff;
};

template <bool CAUSAL, int BQ>
__device__ __forceinline__ KeyRange key_range(const AttnArgs& a, const TileCoords& tc) {
    KeyRange r;
    const int Lk = tc.Lk;
    const int nb = (Lk + kBK - 1) / kBK;
    r.kb0 = static_cast<int>(static_cast<int64_t>(tc.sp) * nb / a.nsplit);
    r.kb1 = static_cast<int>(static_cast<int64_t>(tc.sp + 1) * nb / a.nsplit);
    r.nfull = Lk / kBK;
    r.coff = (CAUSAL && a.causal_br) ? Lk - tc.Lq : 0;
    if (CAUSAL) {
        const int last = min(Lk, tc.qt * BQ + BQ + r.coff);     // keys 0..last-1 can be visible
        r.kb1 = min(r.kb1, last > 0 ? (last + kBK - 1) / kBK : 0);
        r.nfull = min(r.nfull, max(0, floor_div(tc.qt * BQ + r.coff + 1, kBK)));
    }
    r.nfull = max(r.kb0, min(r.nfull, r.kb1));
    return r;
}

// After the last key block: the normaliser from O^T channel D (LCH), then
// either the split partial (unnormalised O^T in output units, with the running
// max and normaliser) or the normalised, cropped and cast output row and the
// log-sum-exp.
template <int DP, typename T, bool VEC_OUT, bool PV16, bool LCH>
__device__ __forceinline__ void tile_epilogue(const AttnArgs& a, const TileCoords& tc, SoftmaxState<DP / 32>& st) {
    constexpr int NU = DP / 32;
    const int hh = tc.hh, qi = tc.qi;
    if constexpr (LCH) {
        // the normaliser accumulated in O^T channel D: lane half hc of tile
        // u_l holds it in element r_l; the other half takes it across
        const int c = a.D % 32, u_l = a.D / 32, hc = (c / 4) & 1, r_l = 4 * (c / 8) + c % 4;
        float mine = 0.0f;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (u == u_l && r == r_l && hh == hc) mine = st.o[u][r];
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(mine), __float_as_int(mine), false, false);
        st.l = __int_as_float(static_cast<int>(pr[0])) + __int_as_float(static_cast<int>(pr[1]));
    } else {
        // the row sums of P: query q on lane q % 16, element q / 16 (rowsum_sel)
        const int src = tc.lq & 15;
        const float l0 = __shfl(st.ls[0], src, 64), l1 = __shfl(st.ls[1], src, 64);
        st.l = tc.lq < 16 ? l0 : l1;
    }
    if (qi >= tc.Lq) return;
    const float* vmax = a.vmax + tc.kvh * DP;
    // P carries a factor 2^8 in the FP8 product, none in the 16-bit one
    constexpr float kPScaleLog2 = PV16 ? 0.0f : 8.0f;

    if (a.nsplit > 1) {
        // ---- partial: the range's own normalised output row O^T * s_v[d] / l
        // (FP8 V) or O^T / l (16-bit V) in the output format, with (m, l):
        // bounded by max |v|, so the format holds it, and half the bytes of
        // fp32 for the merge to read ----
        const int64_t prow = static_cast<int64_t>(tc.sp) * a.part_rows + tc.qrow;
        if (hh == 0) a.part_ml[prow] = make_float2(st.m, st.l);
        if (st.m == -INFINITY) return;          // nothing visible: the merge skips this split
        const float inv_l = st.l > 0.0f ? 1.0f / st.l : 0.0f;
        uint16_t* prow_o = a.part_o + prow * DP;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * u + 8 * r4 + 4 * hh;
                if (d0 >= a.D) continue;
                float vs4[4] = {inv_l, inv_l, inv_l, inv_l};
                if constexpr (!PV16) {
                    const float4 vm = *reinterpret_cast<const float4*>(vmax + d0);
                    vs4[0] = (vm.x * (1.0f / 448.0f)) * inv_l;
                    vs4[1] = (vm.y * (1.0f / 448.0f)) * inv_l;
                    vs4[2] = (vm.z * (1.0f / 448.0f)) * inv_l;
                    vs4[3] = (vm.w * (1.0f / 448.0f)) * inv_l;
                }
                uint16_t h4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = from_f32<T>(st.o[u][4 * r4 + e] * vs4[e]);
                uint2 pk;
                pk.x = static_cast<uint32_t>(h4[0]) | (static_cast<uint32_t>(h4[1]) << 16);
                pk.y = static_cast<uint32_t>(h4[2]) | (static_cast<uint32_t>(h4[3]) << 16);
                *reinterpret_cast<uint2*>(prow_o + d0) = pk;
            }
        }
        return;
    }

    // ---- epilogue: O = O^T * s_v[d] / l (FP8 V) or O^T / l (16-bit V), crop to (Lq, D), cast ----
    // l = 0 only when no key is visible to the query: its output row is 0
    const float inv_l = st.l > 0.0f ? 1.0f / st.l : 0.0f;
    if (a.lse != nullptr && hh == 0)
        a.lse[tc.b * a.ls0 + tc.hq * a.ls1 + (tc.qtok0 + qi) * a.ls2] =
            st.l > 0.0f ? (st.m + log2f(st.l) - kPScaleLog2) * 0.6931471805599453f : -INFINITY;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + tc.b * a.os0 + tc.hq * a.os1 + (tc.qtok0 + qi) * a.os2;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * u + 8 * r4 + 4 * hh;
            if (d0 >= a.D) continue;
            float vs4[4] = {inv_l, inv_l, inv_l, inv_l};
            // (an entry without keys has no V scales written: leave them unread)
            if (!PV16 && inv_l != 0.0f) {
                const float4 vm = *reinterpret_cast<const float4*>(vmax + d0);
                vs4[0] = (vm.x * (1.0f / 448.0f)) * inv_l;
                vs4[1] = (vm.y * (1.0f / 448.0f)) * inv_l;
                vs4[2] = (vm.z * (1.0f / 448.0f)) * inv_l;
                vs4[3] = (vm.w * (1.0f / 448.0f)) * inv_l;
            }
            uint16_t h4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h4[e] = from_f32<T>(st.o[u][4 * r4 + e] * vs4[e]);
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

// Everything after the block -> tile mapping; EXACT is uniform over the workgroup.
// The tile runs the online softmax over its split's range of 128-key blocks
// (all of them when nsplit = 1) and then writes either the normalised output
// (and the log-sum-exp when asked) or, under a split, the unnormalised partial
// with its running max and normaliser. SPARSE: only the blocks whose mask flag
// is set for one of the workgroup's query blocks are loaded; a wave computes
// a loaded block only if its own query block's flag is set. LCH: V^T carries
// the channel of ones (D < Dp) and O^T channel D is the normaliser.
template <int DP, typename T, bool CAUSAL, bool VEC_OUT, bool EXACT, bool PV16, bool SPARSE, bool LCH>
__device__ __forceinline__ void attn_tile(const AttnArgs& a, const TileCoords& tc,
                                          uint8_t* const (&ks)[2], uint8_t* const (&vs)[2],
                                          const QOps<DP>& qb, float sq_row, const KeyRange& kr) {
    constexpr int NU = DP / 32;
    constexpr int BQ = Shape<PV16>::BQ;
    constexpr int VB = Shape<PV16>::VB;
    const int w = tc.w, l = tc.l, lq = tc.lq, hh = tc.hh, qi = tc.qi, q0 = tc.q0;

    const float scq = sq_row * a.scale_log2;

    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.khat) + tc.kblk * kKeyBlock * DP;
    const uint8_t* vg = a.vhat + tc.kblk * (DP * 64 * VB);
    const float* skp = a.sk + tc.kblk;
    const int Lk = tc.Lk;

    const int kb0 = kr.kb0, kb1 = kr.kb1, nfull = kr.nfull, coff = kr.coff;

    SoftmaxState<NU> st;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[u][r] = 0.0f;
    st.m = -INFINITY;
    st.l = 0.0f;
    st.ls = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    StageOffsets<DP, Shape<PV16>::NW, VB> so;
    so.init(w, l);
    LdsOffsets<DP, PV16> lo;
    lo.init(lq, hh);

#define SAGE_STEP_A(BUF, MASK, AFTER, KB, KN, ON)                                                             \
    tile_step<DP, T, CAUSAL, EXACT, PV16, LCH, BUF, MASK, AFTER>(st, so, lo, qb, ks, vs, kg, vg, skp, skb, KB, KN, \
                                                            kb1, Lk, q0, qi, coff, w, hh, scq, ON)
#define SAGE_STEP(BUF, MASK, KB, KN, ON) SAGE_STEP_A(BUF, MASK, false, KB, KN, ON)
    float skb[2] = {0.0f, 0.0f};     // K scales of the next block to run
    if constexpr (!SPARSE) {
        if (kb0 < kb1) {       // the kernel started the first block's copies before the Q loads
            load_kscales(skp, kb0, skb);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        int kb = kb0;
        if (kb < nfull) {
            // the first unmasked step, then the others (every row then has
            // a finite reference)
            SAGE_STEP(0, false, kb, kb + 1, true);
            ++kb;
            for (; kb + 1 < nfull; kb += 2) {
                SAGE_STEP_A(1, false, true, kb, kb + 1, true);
                SAGE_STEP_A(0, false, true, kb + 1, kb + 2, true);
            }
            if (kb < nfull) {
                SAGE_STEP_A(1, false, true, kb, kb + 1, true);
                ++kb;
            }
        }
        for (; kb < kb1; ++kb) {
            if ((kb - kb0) & 1)
                SAGE_STEP(1, true, kb, kb + 1, true);
            else
                SAGE_STEP(0, true, kb, kb + 1, true);
        }
    } else {
        // flags of the workgroup's query blocks (BQ / 128 of them) and of this wave's
        const int64_t qb0 = static_cast<int64_t>(tc.qt) * (BQ / kMaskBlockQ);
        const uint8_t* m0 = a.bmask + ((static_cast<int64_t>(tc.b) * a.Hq + tc.hq) * a.bm_nq + qb0) * a.bm_nk;
        const uint8_t* m1 = (BQ > kMaskBlockQ && qb0 + 1 < a.bm_nq) ? m0 + a.bm_nk : m0;
        const uint8_t* mw = (w * 32 >= kMaskBlockQ) ? m1 : m0;
        // The flags of 64 blocks at a time, as wave-uniform bit words (lane i
        // reads block 64 c + i): any query block of the workgroup, and this
        // wave's. One load per 64 blocks instead of one per step.
        uint64_t any_bits = 0, own_bits = 0;
        int cur = -1;
        auto load_flags = [&](int c) {
            const int k = 64 * c + l;
            int f_any = 0, f_own = 0;
            if (k < kb1) {
                f_any = (m0[k] | m1[k]) != 0;
                f_own = mw[k] != 0;
            }
            any_bits = __ballot(f_any);
            own_bits = __ballot(f_own);
            cur = c;
        };
        // next block at or after k that some wave of the workgroup computes
        auto next_on = [&](int k) {
            while (k < kb1) {
                const int c = k >> 6;
                if (c != cur) load_flags(c);
                const uint64_t rest = any_bits >> (k & 63);
                if (rest != 0) return k + static_cast<int>(__builtin_ctzll(rest));
                k = (c + 1) << 6;
            }
            return kb1;
        };
        int kb = next_on(kb0);
        if (kb < kb1) {
            load_kscales(skp, kb, skb);
            so.stage(kg + static_cast<int64_t>(kb) * (kBK * DP), vg + static_cast<int64_t>(kb) * (kBK * DP * VB),
                     ks[0], vs[0], w);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        int par = 0;
        while (kb < kb1) {
            const bool on = ((own_bits >> (kb & 63)) & 1) != 0;    // kb's word is loaded
            const int kn = next_on(kb + 1);
            if (par == 0) {
                if (kb >= nfull) SAGE_STEP(0, true, kb, kn, on);
                else SAGE_STEP(0, false, kb, kn, on);
            } else {
                if (kb >= nfull) SAGE_STEP(1, true, kb, kn, on);
                else SAGE_STEP(1, false, kb, kn, on);
            }
            kb = kn;
            par ^= 1;
        }
    }
#undef SAGE_STEP
#undef SAGE_STEP_A

    tile_epilogue<DP, T, VEC_OUT, PV16, LCH>(a, tc, st);
}

// Block -> tile mapping shared by the attention kernels: fills tc for this
// lane; false when the workgroup's tile lies past its entry's last query.
template <bool CAUSAL, int BQ>
__device__ __forceinline__ bool map_tile(const AttnArgs& a, TileCoords& tc) {
    const int tid = threadIdx.x;
    tc.w = tid >> 6;
    tc.l = tid & 63;
    tc.lq = tc.l & 31;
    tc.hh = tc.l >> 5;
    // ---- block -> (b, kv head, split, q head of the group, query tile), XCD-aware ----
    const int nqt = (a.m.Lq + BQ - 1) / BQ;           // tiles of the longest entry
    {
        const int n = blockIdx.x;
        const int N = gridDim.x;
        const int full = N / 8;
        // workgroups are dealt to the 8 XCDs round robin; for dense problems
        // this makes consecutive logical tiles (same kv head and key range)
        // land on the same XCD, whose L2 then holds that head's K and V.
        // Packed sequences keep the dispatch order: their entries differ in
        // work, and a contiguous share per XCD would leave the XCD that holds
        // the longest sequence running long after the others are idle.
        const bool remap = a.m.cu_q == nullptr && n < full * 8;
        int L = remap ? (n % 8) * full + n / 8 : n;
        // block-sparse without a causal mask: the XCD's tiles heaviest first
        if (!CAUSAL && remap && a.tord != nullptr) L = a.tord[L];
        tc.qt = L % nqt;
        int rest = L / nqt;
        if (CAUSAL) {
            // a tile's work grows with its index, so the heaviest tiles are
            // dealt out first and the light ones fill the tail: across all the
            // heads an XCD holds when its share is whole heads, else per head
            const int hx = full / nqt;
            if (remap && hx > 0 && full % nqt == 0) {
                const int i = n / 8;              // place in this XCD's dispatch order
                tc.qt = nqt - 1 - i / hx;
                rest = (n % 8) * hx + i % hx;
            } else {
                tc.qt = nqt - 1 - tc.qt;
            }
        }
        const int g = rest % a.G;
        rest /= a.G;
        tc.sp = rest % a.nsplit;
        rest /= a.nsplit;
        tc.hkv = rest % a.Hkv;
        tc.b = rest / a.Hkv;
        tc.hq = tc.hkv * a.G + g;
    }
    tc.w = __builtin_amdgcn_readfirstlane(tc.w);     // wave-uniform (lets branches on it stay scalar)
    const Seq sq = seq_at(a.m, tc.b);
    if (tc.qt * BQ >= sq.Lq) return false;            // past the entry's last query (whole workgroup)
    tc.Lq = sq.Lq;
    tc.Lk = sq.Lk;
    tc.qtok0 = sq.qtok0;
    tc.q0 = tc.qt * BQ + tc.w * 32;
    tc.qi = tc.q0 + tc.lq;
    tc.kvh = static_cast<int64_t>(tc.b) * a.Hkv + tc.hkv;
    tc.qrow = sq.qrow0 + tc.hq * a.m.q_hstride + tc.qi;
    // wave-uniform, so that the K/V block addresses (and the copies' buffer
    // descriptors) are scalar
    tc.kblk = wave_uniform(sq.kblk0 + tc.hkv * a.m.kb_hstride);
    return true;
}

// The largest dequantization scale the workgroup can meet decides whether the
// one-FMA form is accurate enough (see softmax_step); uniform over the
// workgroup. red: 2 NW floats of LDS.
template <int NW>
__device__ __forceinline__ bool exact_form(const AttnArgs& a, const TileCoords& tc, float sq_row, float* red) {
    float mq = sq_row;
    for (int off = 32; off >= 1; off >>= 1) mq = fmaxf(mq, __shfl_xor(mq, off, 64));
    float mk = 0.0f;
    const float* skp = a.sk + tc.kblk;
    const int nkb = (tc.Lk + kBK - 1) / kBK * (kBK / kKeyBlock);
    for (int i = threadIdx.x; i < nkb; i += NW * 64) mk = fmaxf(mk, skp[i]);
    for (int off = 32; off >= 1; off >>= 1) mk = fmaxf(mk, __shfl_xor(mk, off, 64));
    if (tc.l == 0) {
        red[tc.w] = fmaxf(mq, 0.0f);
        red[NW + tc.w] = mk;
    }
    __syncthreads();
    mq = red[0];
    mk = red[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        mq = fmaxf(mq, red[i]);
        mk = fmaxf(mk, red[NW + i]);
    }
    return kMagic * (mq * a.scale_log2) * mk > 2048.0f;
}

// Start the copies of the tile's first key block (dense launches), so that
// their latency overlaps the Q loads and the set-up after them.
template <int DP, int NW, int VB>
__device__ __forceinline__ void stage_first(const AttnArgs& a, const TileCoords& tc, const KeyRange& kr,
                                            uint8_t* kl, uint8_t* vl) {
    if (kr.kb0 >= kr.kb1) return;
    StageOffsets<DP, NW, VB> so;
    so.init(tc.w, tc.l);
    so.stage(reinterpret_cast<const uint8_t*>(a.khat) + (tc.kblk * kKeyBlock + static_cast<int64_t>(kr.kb0) * kBK) * DP,
             a.vhat + (tc.kblk * 64 + static_cast<int64_t>(kr.kb0) * kBK) * DP * VB, kl, vl, tc.w);
}

template <int DP, typename T, bool CAUSAL, bool VEC_OUT, bool PV16, bool SPARSE, bool LCH>
__global__ __launch_bounds__(Shape<PV16>::NW * 64, Shape<PV16>::WG_PER_CU) void attn_kernel(AttnArgs a) {
    constexpr int NW = Shape<PV16>::NW;
    constexpr int BQ = Shape<PV16>::BQ;
    constexpr int VBYTES = kBK * DP * Shape<PV16>::VB;
    __shared__ __align__(16) uint8_t k0s[kBK * DP];
    __shared__ __align__(16) uint8_t k1s[kBK * DP];
    __shared__ __align__(16) uint8_t v0s[VBYTES];
    __shared__ __align__(16) uint8_t v1s[VBYTES];
    __shared__ float red[2 * NW];
    uint8_t* const ks[2] = {k0s, k1s};
    uint8_t* const vs[2] = {v0s, v1s};

    TileCoords tc;
    if (!map_tile<CAUSAL, BQ>(a, tc)) return;
    const KeyRange kr = key_range<CAUSAL, BQ>(a, tc);
    if (!SPARSE) stage_first<DP, NW, Shape<PV16>::VB>(a, tc, kr, ks[0], vs[0]);
    QOps<DP> qb;
    const float sq_row = load_q<DP, T>(a, tc, qb);
    // an entry without keys runs no block, and its rows come out as 0 (the
    // empty softmax sum)
    if (exact_form<NW>(a, tc, sq_row, red))
        attn_tile<DP, T, CAUSAL, VEC_OUT, true, PV16, SPARSE, LCH>(a, tc, ks, vs, qb, sq_row, kr);
    else
        attn_tile<DP, T, CAUSAL, VEC_OUT, false, PV16, SPARSE, LCH>(a, tc, ks, vs, qb, sq_row, kr);
}


// Merge of the key-range splits of one query row (the log-sum-exp combination
// of partial softmaxes: with m = max_s m_s and w_s = 2^(m_s - m), the output
// is sum_s w_s l_s Ô_s / sum_s w_s l_s, Ô_s the range's normalised row, and
// the log-sum-exp is ln 2 (m + log2 of the denominator), less the 2^8 of FP8
// P). A split in which no key was visible
// has m_s = -inf and adds nothing; a row without any visible key is 0 with
// log-sum-exp -inf. DP / 4 threads per row, four channels each.
template <int DP, typename T, bool VEC_OUT>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, float pscale_log2) {
    constexpr int TPR = DP / 4;
    constexpr int ROWS = 256 / TPR;
    const int t = threadIdx.x;
    const int r = t / TPR;
    const int d0 = 4 * (t % TPR);
    const int b = blockIdx.z, hq = blockIdx.y;
    const Seq sq = seq_at(a.m, b);
    const int qi = blockIdx.x * ROWS + r;
    if (qi >= sq.Lq) return;
    const int64_t prow = sq.qrow0 + hq * a.m.q_hstride + qi;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[s * a.part_rows + prow].x);
    float L = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (M != -INFINITY) {
        for (int s = 0; s < a.nsplit; ++s) {
            const int64_t ps = s * a.part_rows + prow;
            const float2 ml = a.part_ml[ps];
            if (ml.x == -INFINITY) continue;
            const float wl = exp2f(ml.x - M) * ml.y;
            L += wl;
            if (d0 < a.D) {
                const uint2 pk = *reinterpret_cast<const uint2*>(a.part_o + ps * DP + d0);
                acc.x += wl * to_f32<T>(static_cast<uint16_t>(pk.x & 0xFFFFu));
                acc.y += wl * to_f32<T>(static_cast<uint16_t>(pk.x >> 16));
                acc.z += wl * to_f32<T>(static_cast<uint16_t>(pk.y & 0xFFFFu));
                acc.w += wl * to_f32<T>(static_cast<uint16_t>(pk.y >> 16));
            }
        }
    }
    if (a.lse != nullptr && d0 == 0)
        a.lse[b * a.ls0 + hq * a.ls1 + (sq.qtok0 + qi) * a.ls2] =
            L > 0.0f ? (M + log2f(L) - pscale_log2) * 0.6931471805599453f : -INFINITY;
    if (d0 >= a.D) return;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t h4[4] = {from_f32<T>(acc.x * inv), from_f32<T>(acc.y * inv), from_f32<T>(acc.z * inv),
                      from_f32<T>(acc.w * inv)};
    uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.os0 + hq * a.os1 + (sq.qtok0 + qi) * a.os2;
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

// int32 logits of one head through the same staging and tile routine (the
// FP8 variant's workgroup shape; the logits do not depend on the variant).
// Block-sparse launches without a causal mask: the logical tiles of XCD
// blockIdx.x's share [x full, (x + 1) full) in decreasing order of the key
// blocks they load (a counting sort), so that the heavy tiles start first and
// the light ones fill the tail; ties in any order (each tile's result does not
// depend on when it runs). A tile's logical index decodes as in map_tile; it
// loads the blocks of its key range whose flag is set for one of its query
// blocks.
template <int BQ>
__global__ __launch_bounds__(256) void deal_tiles_kernel(AttnArgs a, int nqt, int full) {
    constexpr int NBIN = 1024;                 // counts clamp here (only the order's quality suffers)
    __shared__ int hist[NBIN];
    __shared__ int part[256];
    const int x = blockIdx.x, t = threadIdx.x;
    const int nb = (a.m.Lk + kBK - 1) / kBK;
    const int nbin = min(nb, NBIN - 1) + 1;
    for (int i = t; i < NBIN; i += 256) hist[i] = 0;
    __syncthreads();
    auto count_of = [&](int L) {
        const int qt = L % nqt;
        int rest = L / nqt;
        const int g = rest % a.G;
        rest /= a.G;
        const int sp = rest % a.nsplit;
        rest /= a.nsplit;
        const int hkv = rest % a.Hkv;
        const int b = rest / a.Hkv;
        const int hq = hkv * a.G + g;
        const int kb0 = static_cast<int>(static_cast<int64_t>(sp) * nb / a.nsplit);
        const int kb1 = static_cast<int>(static_cast<int64_t>(sp + 1) * nb / a.nsplit);
        const int64_t qb0 = static_cast<int64_t>(qt) * (BQ / kMaskBlockQ);
        const uint8_t* m0 = a.bmask + ((static_cast<int64_t>(b) * a.Hq + hq) * a.bm_nq + qb0) * a.bm_nk;
        const uint8_t* m1 = (BQ > kMaskBlockQ && qb0 + 1 < a.bm_nq) ? m0 + a.bm_nk : m0;
        int c = 0;
        for (int kb = kb0; kb < kb1; ++kb) c += (m0[kb] | m1[kb]) != 0;
        return min(c, nbin - 1);
    };
    for (int i = t; i < full; i += 256) atomicAdd(&hist[count_of(x * full + i)], 1);
    __syncthreads();
    // hist[c] <- number of tiles with a count above c: thread t holds bins
    // 4t .. 4t + 3; a suffix scan over the threads' sums
    int own[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 4 * t + j;
        own[j] = c < nbin ? hist[c] : 0;
        sum += own[j];
    }
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int v = t + off < 256 ? part[t + off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int above = t + 1 < 256 ? part[t + 1] : 0;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
        const int c = 4 * t + j;
        if (c < nbin) hist[c] = above;
        above += own[j];
    }
    __syncthreads();
    for (int i = t; i < full; i += 256) {
        const int L = x * full + i;
        a.tord[x * full + atomicAdd(&hist[count_of(L)], 1)] = L;
    }
}

template <int DP>
__global__ __launch_bounds__(256) void qk_dump_kernel(AttnArgs a) {
    constexpr int BQ = Shape<false>::BQ;
    __shared__ __align__(16) uint8_t k0s[kBK * DP];
    __shared__ __align__(16) uint8_t v0s[kBK * DP];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, hh = l >> 5;
    const int b = a.dump_b, hq = a.dump_hq, hkv = hq / a.G;
    const int qi = blockIdx.x * BQ + w * 32 + lq;
    const Seq sq = seq_at(a.m, b);
    const int64_t qrow = sq.qrow0 + hq * a.m.q_hstride + qi;
    const int64_t kblk = wave_uniform(sq.kblk0 + hkv * a.m.kb_hstride);
    QOps<DP> qb;
#pragma unroll
    for (int c = 0; c < DP / 32; ++c)
        qb.c[c] = *reinterpret_cast<const v4i*>(a.qhat + qrow * DP + 32 * c + 16 * hh);
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.khat) + kblk * kKeyBlock * DP;
    const uint8_t* vg = a.vhat + kblk * (DP * 64);
    const int nkblk = (sq.Lk + kBK - 1) / kBK;
    StageOffsets<DP, 4, 1> so;
    so.init(w, l);
    LdsOffsets<DP, false> lo;
    lo.init(lq, hh);
    for (int kb = 0; kb < nkblk; ++kb) {
        so.stage(kg + static_cast<int64_t>(kb) * kBK * DP, vg + static_cast<int64_t>(kb) * kBK * DP,
                 k0s, v0s, w);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        v16i s[4];
        qk_block<DP, false>(s, k0s, lo, qb);
        int32_t* out = a.dump + static_cast<int64_t>(qi) * a.dump_ld + kb * kBK;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                out[32 * t + 8 * (r / 4) + 4 * hh + (r % 4)] = s[t][r] - kMagicBits;
        __syncthreads();
    }
}

template <int DP, typename T, bool PV16>
hipError_t attn_dispatch(const AttnArgs& a, bool causal, bool vec_out, hipStream_t s) {
    constexpr int BQ = Shape<PV16>::BQ;
    constexpr unsigned threads = Shape<PV16>::NW * 64;
    const unsigned nqt = static_cast<unsigned>((a.m.Lq + BQ - 1) / BQ);
    const unsigned grid = nqt * a.Hq * a.B * a.nsplit;
    // block-sparse launches keep the all-ones normaliser product, which
    // saves a second set of block-sparse instantiations
#define SAGE_LAUNCH(C, V)                                                                             \
    do {                                                                                              \
        if (a.bmask != nullptr) attn_kernel<DP, T, C, V, PV16, true, false><<<grid, threads, 0, s>>>(a); \
        else if (a.lch) attn_kernel<DP, T, C, V, PV16, false, true><<<grid, threads, 0, s>>>(a);        \
        else attn_kernel<DP, T, C, V, PV16, false, false><<<grid, threads, 0, s>>>(a);                  \
    } while (0)
    if (causal) {
        if (vec_out) SAGE_LAUNCH(true, true);
        else SAGE_LAUNCH(true, false);
    } else {
        if (vec_out) SAGE_LAUNCH(false, true);
        else SAGE_LAUNCH(false, false);
    }
#undef SAGE_LAUNCH
    return hipGetLastError();
}

template <typename T, bool PV16>
hipError_t attn_dispatch_dp(const AttnArgs& a, int Dp, bool causal, bool vec_out, hipStream_t s) {
    return Dp == 64 ? attn_dispatch<64, T, PV16>(a, causal, vec_out, s)
                    : attn_dispatch<128, T, PV16>(a, causal, vec_out, s);
}

template <int DP, typename T>
hipError_t combine_dispatch(const AttnArgs& a, bool vec_out, float pscale_log2, hipStream_t s) {
    constexpr int ROWS = 256 / (DP / 4);
    const dim3 grid(static_cast<unsigned>((a.m.Lq + ROWS - 1) / ROWS), static_cast<unsigned>(a.Hq),
                    static_cast<unsigned>(a.B));
    if (vec_out) combine_kernel<DP, T, true><<<grid, 256, 0, s>>>(a, pscale_log2);
    else combine_kernel<DP, T, false><<<grid, 256, 0, s>>>(a, pscale_log2);
    return hipGetLastError();
}

}  // namespace
}  // namespace sage
