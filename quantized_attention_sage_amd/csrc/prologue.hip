// Quantization prologue for gfx950: K/V statistics, Q and K INT8 codes,
// V FP8 E4M3 codes (transposed and permuted for the matrix-core operand).
//
// Method sources (page, section):
//   stable-diffusion.cpp "SageAttention" doc, kernel table and the paragraph
//   after it: K is smoothed, V is quantized per channel to FP8 and padded and
//   permuted for the matrix unit; head dims pad to 64 or 128.
//   topgit.dev "SageAttention: Quantized Attention Library", core features:
//   per-token INT8 Q/K granularity and smoothing of K.
//   "SageAttention-RDNA4" releases, v0.4.0: a hand-written prologue with 64-bit
//   offsets and the key mean summed in fp64; v0.2.0: one Q scale per token.
//
// Every fp32 step here (products, divisions, rounding to integers) is the
// value contract of the workspace and is written to round once per
// operation: the file is compiled with -ffp-contract=off and no fast-math,
// division is correctly rounded and denormals are kept.
#include "sage_kernels.h"

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <type_traits>

namespace sage {
namespace {

#include "quant_rules.h"

// The 16-bit pattern of an fp32 value that holds a T value exactly.
template <typename T>
__device__ __forceinline__ uint16_t bits16(float x);

template <>
__device__ __forceinline__ uint16_t bits16<__half>(float x) {
    return __half_as_ushort(__float2half_rn(x));
}

template <>
__device__ __forceinline__ uint16_t bits16<__hip_bfloat16>(float x) {
    return static_cast<uint16_t>(__float_as_uint(x) >> 16);
}

// Eight channels of one token row kept as loaded (16 bytes when VEC, else
// already converted), so that many rows can be in flight in few registers.
template <typename T, bool VEC>
struct Row8 {
    uint4 u;
    float f[VEC ? 1 : 8];
    __device__ __forceinline__ void load(const uint16_t* row, int d0, int D) {
        if (VEC) {
            u = d0 < D ? *reinterpret_cast<const uint4*>(row + d0) : make_uint4(0, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < (VEC ? 1 : 8); ++i) f[i] = (d0 + i < D) ? to_f32<T>(row[d0 + i]) : 0.0f;
        }
    }
    __device__ __forceinline__ void zero() {
        u = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < (VEC ? 1 : 8); ++i) f[i] = 0.0f;
    }
    __device__ __forceinline__ void get(float (&x)[8]) const {
        if (VEC) {
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = to_f32<T>(static_cast<uint16_t>(w[i] & 0xFFFFu));
                x[2 * i + 1] = to_f32<T>(static_cast<uint16_t>(w[i] >> 16));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = f[VEC ? 0 : i];
        }
    }
};

// ---------------------------------------------------------------------------
// K/V statistics of one 256-token chunk of one (batch, kv-head).
// Threads 0..127 own one K channel each and sum the chunk's tokens in order in
// fp64; threads 128..255 own one V channel each and take the max |v|. Loads
// are one element per thread per token (a wave reads 64 consecutive channels,
// 128 contiguous bytes); 32 tokens are loaded before any of them is added, so
// that enough bytes are in flight to cover the HBM latency.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void stats_body(const StatsArgs& a, int c, int h, int b) {
    constexpr int U = 32;
    const int t = threadIdx.x;
    const Seq sq = seq_at(a.m, b);
    const int j0 = c * kChunk;
    if (j0 >= sq.Lk) return;                       // past this entry's last chunk
    const int j1 = min(j0 + kChunk, sq.Lk);
    const int64_t slot = (sq.chunk0 + h * a.m.c_hstride + c) * a.Dp;
    const bool is_k = t < 128;
    const int d = is_k ? t : t - 128;
    if (d >= a.Dp) return;
    const bool live = d < a.D && (!is_k || a.smooth);
    const uint16_t* base = is_k ? static_cast<const uint16_t*>(a.k) + b * a.ks0 + h * a.ks1 + sq.ktok0 * a.ks2 + d
                                : static_cast<const uint16_t*>(a.v) + b * a.vs0 + h * a.vs1 + sq.ktok0 * a.vs2 + d;
    const int64_t ts = is_k ? a.ks2 : a.vs2;
    double s = 0.0;
    float m = 0.0f;
    if (live) {
        int j = j0;
        for (; j + U <= j1; j += U) {
            float x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = to_f32<T>(base[(j + u) * ts]);
            if (is_k) {
#pragma unroll
                for (int u = 0; u < U; ++u) s += static_cast<double>(x[u]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) m = fmaxf(m, fabsf(x[u]));
            }
        }
        for (; j < j1; ++j) {
            const float x = to_f32<T>(base[j * ts]);
            if (is_k)
                s += static_cast<double>(x);
            else
                m = fmaxf(m, fabsf(x));
        }
    }
    if (is_k)
        a.kpart[slot + d] = s;
    else
        a.vpart[slot + d] = m;
}

// ---------------------------------------------------------------------------
// Q: one INT8 scale per token. Each row of Dp channels is handled by Dp/8
// lanes holding 8 channels each; the row max is a butterfly over those lanes.
// A thread handles QR rows (their loads are issued together). Rows
// Lq..Lq_pad-1 get zero codes and a zero scale.
// ---------------------------------------------------------------------------
constexpr int QR = 4;


template <typename T, int DP, bool VEC>
__device__ __forceinline__ void quant_q_body(const QuantQArgs& a, int tile, int h, int b) {
    constexpr int LPR = DP / 8;                 // lanes per row
    constexpr int RPP = 256 / LPR;              // rows per pass
    const Seq sq = seq_at(a.m, b);
    const int nrow = (sq.Lq + kQPad - 1) / kQPad * kQPad;   // rows written: Lq rounded up to 256
    const int i0 = tile * (RPP * QR);
    if (i0 >= nrow) return;
    const int t = threadIdx.x;
    const int sub = t % LPR;
    const int d0 = sub * 8;
    const int64_t rbase = sq.qrow0 + h * a.m.q_hstride;
    float x[QR][8];
#pragma unroll
    for (int r = 0; r < QR; ++r) {
        const int i = i0 + r * RPP + t / LPR;
        if (i < sq.Lq) {
            const uint16_t* rp = static_cast<const uint16_t*>(a.q) + b * a.qs0 + h * a.qs1 + (sq.qtok0 + i) * a.qs2;
            load8<T, VEC>(rp, d0, a.D, x[r]);
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) x[r][u] = 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < QR; ++r) {
        const int i = i0 + r * RPP + t / LPR;
        float m = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(x[r][u]));
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        const float s = m / 127.0f;
        const float rc = m > 0.0f ? 127.0f / m : 0.0f;
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            w0 |= (static_cast<uint32_t>(static_cast<uint8_t>(int8_code(x[r][u], rc)))) << (8 * u);
            w1 |= (static_cast<uint32_t>(static_cast<uint8_t>(int8_code(x[r][u + 4], rc)))) << (8 * u);
        }
        if (i < nrow) {
            *reinterpret_cast<uint2*>(a.qhat + (rbase + i) * DP + d0) = make_uint2(w0, w1);
            if (sub == 0) a.sq[rbase + i] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// First launch of the prologue: the K/V chunk statistics (blocks
// [0, nstats), block n = chunk + nchunk * (head + Hkv * batch)) and the Q
// codes (the blocks after them, one tile of rows of one head of one
// entry). Both only read the inputs, so one launch
// lets their HBM traffic overlap.
// ---------------------------------------------------------------------------
template <typename T, int DP, bool VEC_Q>
__global__ __launch_bounds__(256) void stats_q_kernel(StatsArgs sa, QuantQArgs qa, int nstats) {
    const int n = blockIdx.x;
    if (n < nstats) {
        const int c = n % sa.nchunk;
        const int rest = n / sa.nchunk;
        stats_body<T>(sa, c, rest % sa.Hkv, rest / sa.Hkv);
    } else {
        const int r = n - nstats;                 // Q block r = tile + ntile * (head + Hq * batch)
        const int tile = r % qa.ntile;
        const int rest = r / qa.ntile;
        quant_q_body<T, DP, VEC_Q>(qa, tile, rest % qa.Hq, rest / qa.Hq);
    }
}

// Position of token j (0..63) inside a permuted 64-token V block. It matches
// the order in which the attention kernel packs P into the FP8 matrix-core
// operand: byte p of lane-half h holds key 32*(p/16) + 8*((p%16)/4) + 4*h + p%4,
// and V-row bytes are stored at position 32*h + p.
__device__ __forceinline__ int vpos(int j) {
    return 32 * ((j >> 2) & 1) + 16 * (j >> 5) + 4 * ((j >> 3) & 3) + (j & 3);
}

// The same for the 16-bit V^T of the INT8-QK / 16-bit-PV variant: the 16-bit
// matrix-core product takes 16 keys, 8 consecutive elements per lane half,
// and the attention kernel puts key 16 g + 8 a + 4 h + e (a, h in {0, 1},
// e < 4) of lane half h at element 8 h + 4 a + e of group g: bits 2 and 3 of
// the key index swap.
__device__ __forceinline__ int vpos16(int j) {
    return (j & ~12) | ((j >> 1) & 4) | ((j << 1) & 8);
}

// ---------------------------------------------------------------------------
// The statistics of one (batch, kv-head) from its chunk partials, for long
// sequences (more than kStatsInline chunks), where every K/V block workgroup
// adding them itself would re-read them many times over: thread d < Dp adds
// the key sums of channel d in chunk order in fp64 and writes
// kbar = fp32(sum / Lk) (0 for padded channels or without smoothing); thread
// Dp + d takes the max of the V chunk maxima. The partials are loaded
// kStatsFinal at a time, then added in order (the zero fill past the last
// chunk adds nothing: the sum starts at +0).
// ---------------------------------------------------------------------------
constexpr int kStatsInline = 32;
constexpr int kStatsFinal = 64;

// How the K/V codes kernel gets each head's statistics: from the chunk
// partials (long entries, or bf16), or summed by every workgroup itself
// (short fp16 entries), with the block's own rows loaded after the sums or
// ahead of them.
constexpr int kStatsPartials = 0;
constexpr int kStatsFull = 1;
constexpr int kStatsFullEarly = 2;
constexpr int64_t kEarlyRowsMaxWgs = 256;

template <int DP>
__global__ __launch_bounds__(2 * DP) void stats_final_kernel(QuantKVArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const Seq sq = seq_at(a.m, b);
    const int Lk = sq.Lk;
    if (Lk == 0) return;                       // an entry without keys has no blocks to code
    const int nchunk = (Lk + kChunk - 1) / kChunk;
    const int64_t head = static_cast<int64_t>(b) * a.Hkv + h;
    const int64_t cslot = sq.chunk0 + h * a.m.c_hstride;
    const bool is_k = t < DP;
    const int d = is_k ? t : t - DP;
    const bool real = d < a.D;
    if (is_k) {
        const double* kp = a.kpart + cslot * DP + d;
        double sum = 0.0;
        for (int c0 = 0; c0 < nchunk; c0 += kStatsFinal) {
            double ks[kStatsFinal];
#pragma unroll
            for (int u = 0; u < kStatsFinal; ++u) ks[u] = c0 + u < nchunk ? kp[(c0 + u) * DP] : 0.0;
#pragma unroll
            for (int u = 0; u < kStatsFinal; ++u) sum += ks[u];
        }
        a.kbar[head * DP + d] = (real && a.smooth) ? static_cast<float>(sum / static_cast<double>(Lk)) : 0.0f;
    } else {
        const float* vp = a.vpart + cslot * DP + d;
        float mx = 0.0f;
        for (int c0 = 0; c0 < nchunk; c0 += kStatsFinal) {
            float vs[kStatsFinal];
#pragma unroll
            for (int u = 0; u < kStatsFinal; ++u) vs[u] = c0 + u < nchunk ? vp[(c0 + u) * DP] : 0.0f;
#pragma unroll
            for (int u = 0; u < kStatsFinal; ++u) mx = fmaxf(mx, vs[u]);
        }
        a.vmax[head * DP + d] = real ? mx : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// K and V of one 64-token block of one (batch, kv-head).
// First the head's statistics (kbar and vmax, which stats_final_kernel wrote
// to the workspace), one channel per thread into LDS.
// K: k~ = k - kbar (fp32), block amax over real tokens and channels, one scale,
//    INT8 codes row-major [token][Dp].
// V: per-channel scale from vmax, E4M3 codes (hardware RNE conversion after a
//    clamp to +-448), transposed to [Dp][64] with the token permutation vpos;
//    PV16: the 16-bit input values themselves, transposed with vpos16. When
//    D < Dp, channel D holds 1.0 for every real token: the attention kernel's
//    P.V product then yields the softmax normaliser (the sum of P) in that
//    output channel.
// Grid (nkb, Hkv, B), 256 threads, one workgroup per block; each thread
// holds 8 channels of 64 / (256 / (Dp/8)) rows of K, and 8 channels of 4
// consecutive rows of V. Short heads (FULL, SPLIT) use (2 nkb, Hkv, B):
// workgroup 2 i codes K of block i and workgroup 2 i + 1 its V, each scanning
// the head for the one statistic it needs, so each scans and holds half
// (c2's K/V prologue 11.4 -> 9.3 us); with chunk partials the split measured
// slower (c3 50 -> 66 us: twice the workgroups, each as long in latency).
// ---------------------------------------------------------------------------
template <typename T, int DP, bool VEC, bool PV16, int MODE>
__global__ __launch_bounds__(256) void quant_kv_kernel(QuantKVArgs a) {
    constexpr bool FULL = MODE != kStatsPartials;   // the workgroup adds up its head's k or v itself
    constexpr bool EARLY = MODE == kStatsFullEarly;
    constexpr bool SPLIT = FULL;                // separate K and V workgroups
    constexpr int LPR = DP / 8;
    constexpr int RPP = 256 / LPR;              // rows per pass
    constexpr int NP = kKeyBlock / RPP;         // passes over the 64 rows
    __shared__ float red[4];
    __shared__ float kbar_s[DP], vmax_s[DP];
    constexpr int VB = PV16 ? 2 : 1;            // bytes per V^T element
    constexpr int VRS = PV16 ? 36 : 18;         // LDS words per V^T row (32 or 16, padded)
    __shared__ __align__(16) uint8_t vt[DP * VRS * 4];

    const int blk = SPLIT ? blockIdx.x >> 1 : blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    // what this workgroup codes (uniform over it)
    const bool do_k = !SPLIT || (blockIdx.x & 1) == 0;
    const bool do_v = !SPLIT || (blockIdx.x & 1) == 1;
    const Seq sq = seq_at(a.m, b);
    const int Lk = sq.Lk;
    // blocks of this entry: its tokens rounded up to 128 (the attention step)
    if (blk >= (Lk + kBK - 1) / kBK * (kBK / kKeyBlock)) return;
    const int nchunk = (Lk + kChunk - 1) / kChunk;
    const int t = threadIdx.x;
    const int sub = t % LPR;
    const int d0 = sub * 8;
    const int64_t head = static_cast<int64_t>(b) * a.Hkv + h;
    const int64_t kblock = sq.kblk0 + h * a.m.kb_hstride + blk;     // workspace K block
    const int jb = blk * kKeyBlock;
    const uint16_t* kin = static_cast<const uint16_t*>(a.k) + b * a.ks0 + h * a.ks1 + sq.ktok0 * a.ks2;
    const uint16_t* vin = static_cast<const uint16_t*>(a.v) + b * a.vs0 + h * a.vs1 + sq.ktok0 * a.vs2;

    // The head's key mean and V channel maxima, one channel per thread into
    // LDS: for up to kStatsInline chunks added here from the chunk partials
    // (the first PU loaded before the K rows, so they arrive first, any
    // further ones PU at a time; the first workgroup of each head also
    // stores the results), otherwise read from the workspace, where
    // stats_final_kernel put them.
    constexpr int PU = 16;                      // chunk partials loaded together
    const bool stat_thread = t < DP;

    // This thread's K rows and V rows of the block (the V codes take tokens
    // 4 tq .. 4 tq + 3 and channels 8 cg .. 8 cg + 7, see below). EARLY: they
    // are loaded first and arrive with the statistics loads, which saves
    // dependent round trips; otherwise the K rows (or a split V workgroup's
    // V rows) are loaded after the statistics, and a combined workgroup's V
    // rows once its K codes are out.
    Row8<T, VEC> kr[NP];
    Row8<T, VEC> vr[4];
    const int tq = t & 15, cg = t >> 4;
    const bool vlive = cg < LPR;                // DP = 64: threads 128.. hold no channels
    auto load_k_rows = [&]() {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int j = jb + p * RPP + t / LPR;
            if (j < Lk)
                kr[p].load(kin + j * a.ks2, d0, a.D);
            else
                kr[p].zero();
        }
    };
    auto load_v_rows = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = jb + 4 * tq + r;
            if (vlive && j < Lk)
                vr[r].load(vin + j * a.vs2, 8 * cg, a.D);
            else
                vr[r].zero();
        }
    };
    if constexpr (EARLY) {
        if (do_k)
            load_k_rows();
        else
            load_v_rows();
    }
    if constexpr (FULL) {
        // Short fp16 heads (one launch for the whole K/V prologue): every
        // workgroup adds up its head's keys (K workgroups) or takes its V
        // channel maxima (V workgroups) itself, thread (t % LPR) taking
        // eight channels of rows t / LPR, t / LPR + RPP, ..., then a tree over
        // the threads of each channel group. fp64 adds of at most 2^13 fp16
        // values (multiples of 2^-24 below 2^16) are exact, so every order
        // gives the chunk-ordered sum bit for bit.
        __shared__ double ksum_s[4][DP];
        __shared__ float vmx_s[4][DP];
        double s8[8];
        float m8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            s8[u] = 0.0;
            m8[u] = 0.0f;
        }
        const uint16_t* src = do_k ? kin : vin;
        const int64_t rs = do_k ? a.ks2 : a.vs2;
        constexpr int RB = 8;                   // rows in flight per thread
        for (int j0 = t / LPR; j0 < Lk; j0 += RB * RPP) {
            Row8<T, VEC> rw[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int j = j0 + i * RPP;
                if (j < Lk)
                    rw[i].load(src + j * rs, d0, a.D);
                else
                    rw[i].zero();
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                float x[8];
                rw[i].get(x);
                if (do_k) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) s8[u] += static_cast<double>(x[u]);
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) m8[u] = fmaxf(m8[u], fabsf(x[u]));
                }
            }
        }
        if (do_k) {
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
                for (int u = 0; u < 8; ++u) s8[u] += __shfl_xor(s8[u], off, 64);
            if ((t & 63) < LPR) {
#pragma unroll
                for (int u = 0; u < 8; ++u) ksum_s[t >> 6][d0 + u] = s8[u];
            }
        } else {
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
                for (int u = 0; u < 8; ++u) m8[u] = fmaxf(m8[u], __shfl_xor(m8[u], off, 64));
            if ((t & 63) < LPR) {
#pragma unroll
                for (int u = 0; u < 8; ++u) vmx_s[t >> 6][d0 + u] = m8[u];
            }
        }
        __syncthreads();
        if (stat_thread) {
            const bool real = t < a.D;
            if (do_k) {
                const double sum = (ksum_s[0][t] + ksum_s[1][t]) + (ksum_s[2][t] + ksum_s[3][t]);
                const float kbar = (real && a.smooth) ? static_cast<float>(sum / static_cast<double>(Lk)) : 0.0f;
                kbar_s[t] = kbar;
                if (blk == 0) a.kbar[head * DP + t] = kbar;
            } else {
                const float mx = fmaxf(fmaxf(vmx_s[0][t], vmx_s[1][t]), fmaxf(vmx_s[2][t], vmx_s[3][t]));
                const float vmax = real ? mx : 0.0f;
                vmax_s[t] = vmax;
                if (blk == 0) a.vmax[head * DP + t] = vmax;
            }
        }
    }
    const bool inline_stats = !FULL && nchunk <= kStatsInline;
    const int64_t cslot = sq.chunk0 + h * a.m.c_hstride;
    const double* kp = a.kpart + cslot * DP + t;
    const float* vp = a.vpart + cslot * DP + t;
    double ks[PU];
    float vs[PU];
    if (stat_thread && !FULL) {
        if (inline_stats) {
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                if (do_k) ks[u] = u < nchunk ? kp[u * DP] : 0.0;
                if (do_v) vs[u] = u < nchunk ? vp[u * DP] : 0.0f;
            }
        } else {
            if (do_k) ks[0] = a.kbar[head * DP + t];
            if (do_v) vs[0] = a.vmax[head * DP + t];
        }
    }

    // without EARLY: the K rows now (the V rows of a combined workgroup once
    // its K codes are out, which keeps its registers low)
    if constexpr (!EARLY) {
        if (do_k)
            load_k_rows();
        else
            load_v_rows();
    }

    if (stat_thread && !FULL) {
        const bool real = t < a.D;
        if (inline_stats && do_k) {
            // chunk partials added in chunk order in fp64 (the zero fill past
            // nchunk adds nothing: the sum starts at +0)
            double sum = 0.0;
#pragma unroll
            for (int u = 0; u < PU; ++u) sum += ks[u];
            for (int c0 = PU; c0 < nchunk; c0 += PU) {
                // the next PU partials, loaded together, then added in chunk order
#pragma unroll
                for (int u = 0; u < PU; ++u) ks[u] = c0 + u < nchunk ? kp[(c0 + u) * DP] : 0.0;
#pragma unroll
                for (int u = 0; u < PU; ++u) sum += ks[u];
            }
            const float kbar = (real && a.smooth) ? static_cast<float>(sum / static_cast<double>(Lk)) : 0.0f;
            kbar_s[t] = kbar;
            if (blk == 0) a.kbar[head * DP + t] = kbar;
        }
        if (inline_stats && do_v) {
            float mx = 0.0f;
#pragma unroll
            for (int u = 0; u < PU; ++u) mx = fmaxf(mx, vs[u]);
            for (int c0 = PU; c0 < nchunk; c0 += PU) {
#pragma unroll
                for (int u = 0; u < PU; ++u) vs[u] = c0 + u < nchunk ? vp[(c0 + u) * DP] : 0.0f;
#pragma unroll
                for (int u = 0; u < PU; ++u) mx = fmaxf(mx, vs[u]);
            }
            const float vmax = real ? mx : 0.0f;
            vmax_s[t] = vmax;
            if (blk == 0) a.vmax[head * DP + t] = vmax;
        }
        if (!inline_stats) {
            if (do_k) kbar_s[t] = static_cast<float>(ks[0]);
            if (do_v) vmax_s[t] = vs[0];
        }
    }
    __syncthreads();
    if (do_k) {
        float kb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kb[u] = kbar_s[d0 + u];

        // ---- K ----
        float kx[NP][8];
        float m = 0.0f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int j = jb + p * RPP + t / LPR;
            kr[p].get(kx[p]);
            if (j < Lk) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    kx[p][u] = kx[p][u] - kb[u];
                    if (d0 + u < a.D) m = fmaxf(m, fabsf(kx[p][u]));
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        if ((t & 63) == 0) red[t >> 6] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float s = m / 127.0f;
        const float r = m > 0.0f ? 127.0f / m : 0.0f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int j = jb + p * RPP + t / LPR;
            uint32_t w0 = 0, w1 = 0;
            if (j < Lk) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int8_t c0 = (d0 + u < a.D) ? int8_code(kx[p][u], r) : 0;
                    const int8_t c1 = (d0 + u + 4 < a.D) ? int8_code(kx[p][u + 4], r) : 0;
                    w0 |= static_cast<uint32_t>(static_cast<uint8_t>(c0)) << (8 * u);
                    w1 |= static_cast<uint32_t>(static_cast<uint8_t>(c1)) << (8 * u);
                }
            }
            *reinterpret_cast<uint2*>(a.khat + (kblock * kKeyBlock + (j - jb)) * DP + d0) = make_uint2(w0, w1);
        }
        if (t == 0) a.sk[kblock] = s;
        if constexpr (SPLIT) return;        // a V workgroup follows
    }

    // ---- V ----
    // Thread (tq, cg) takes tokens 4 tq .. 4 tq + 3 of the block and channels
    // 8 cg .. 8 cg + 7. The four tokens are consecutive in V^T's permuted
    // order (both permutations keep the two low bits of the token index), so
    // each channel's four codes form one aligned 32-bit word (FP8) or 64-bit
    // pair (16-bit) of its V^T row. Rows are padded in LDS (VRS words) so
    // that the stores of a wave fall in distinct banks.
    if constexpr (!SPLIT) load_v_rows();
    if (vlive) {
        float vx[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[r].get(vx[r]);
        const int nreal = Lk - (jb + 4 * tq);    // tokens 0 .. nreal-1 of the four are real
        if constexpr (PV16) {
            uint32_t* vtw = reinterpret_cast<uint32_t*>(vt);
            const int e0 = vpos16(4 * tq);       // first of the four elements, a multiple of 4
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int d = 8 * cg + u;
                uint16_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) h[r] = bits16<T>((d == a.D && r < nreal) ? 1.0f : vx[r][u]);
                *reinterpret_cast<uint2*>(vtw + d * VRS + e0 / 2) =
                    make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16));
            }
        } else {
            float rv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float c = vmax_s[8 * cg + u];
                rv[u] = c > 0.0f ? 448.0f / c : 0.0f;
            }
            uint32_t* vtw = reinterpret_cast<uint32_t*>(vt);
            const int w0 = vpos(4 * tq) / 4;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int d = 8 * cg + u;
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    y[r] = fminf(fmaxf(vx[r][u] * rv[u], -448.0f), 448.0f);
                    if (d == a.D && r < nreal) y[r] = 1.0f;          // the normaliser channel
                }
                // the first conversion writes the low half of the word and the
                // second the high half
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
                vtw[d * VRS + w0] = static_cast<uint32_t>(word);
            }
        }
    }
    __syncthreads();
    // copy out: word g of the [DP][64 tokens] block, rows unpadded
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.vhat + kblock * (DP * kKeyBlock * VB));
    const uint32_t* vtr = reinterpret_cast<const uint32_t*>(vt);
    constexpr int RW = kKeyBlock * VB / 4;      // words per V^T row
    for (int g = t; g < DP * RW; g += 256) dst[g] = vtr[(g / RW) * VRS + g % RW];
}

}  // namespace

template <typename T, int DP>
static void stats_q_dispatch(const StatsArgs& sa, const QuantQArgs& qa, int B, bool vec_q, hipStream_t s) {
    const int nstats = sa.nchunk * sa.Hkv * B;
    const unsigned grid = static_cast<unsigned>(nstats + static_cast<int64_t>(qa.ntile) * qa.Hq * B);
    if (grid == 0) return;                // no keys and no Q tiles (Q quantized by the attention kernel)
    if (vec_q)
        stats_q_kernel<T, DP, true><<<grid, 256, 0, s>>>(sa, qa, nstats);
    else
        stats_q_kernel<T, DP, false><<<grid, 256, 0, s>>>(sa, qa, nstats);
}

hipError_t launch_stats_q(const StatsArgs& sa, const QuantQArgs& qa, int B, int Dp, int dtype, bool vec_q,
                          hipStream_t s) {
    if (dtype == 0) {
        if (Dp == 64) stats_q_dispatch<__half, 64>(sa, qa, B, vec_q, s);
        else stats_q_dispatch<__half, 128>(sa, qa, B, vec_q, s);
    } else {
        if (Dp == 64) stats_q_dispatch<__hip_bfloat16, 64>(sa, qa, B, vec_q, s);
        else stats_q_dispatch<__hip_bfloat16, 128>(sa, qa, B, vec_q, s);
    }
    return hipGetLastError();
}

template <typename T, int DP, int MODE>
static void quant_kv_launch(const QuantKVArgs& a, dim3 grid, bool vec, hipStream_t s) {
    if (a.pv16) {
        if (vec)
            quant_kv_kernel<T, DP, true, true, MODE><<<grid, 256, 0, s>>>(a);
        else
            quant_kv_kernel<T, DP, false, true, MODE><<<grid, 256, 0, s>>>(a);
    } else {
        if (vec)
            quant_kv_kernel<T, DP, true, false, MODE><<<grid, 256, 0, s>>>(a);
        else
            quant_kv_kernel<T, DP, false, false, MODE><<<grid, 256, 0, s>>>(a);
    }
}

template <typename T, int DP>
static void quant_kv_dispatch(const QuantKVArgs& a, int nkb, int B, bool vec, hipStream_t s) {
    if (a.nchunk > kStatsInline) stats_final_kernel<DP><<<dim3(a.Hkv, B), 2 * DP, 0, s>>>(a);
    dim3 grid(nkb, a.Hkv, B);
    if constexpr (std::is_same<T, __half>::value) {
        if (a.full_stats) {
            dim3 g2(2 * nkb, a.Hkv, B);         // a K and a V workgroup per block
            // Early row loads: always at 64 channels (measured faster from one
            // to four workgroups per CU); at 128 channels only while the grid
            // is at most one workgroup per CU, since there the 32 registers
            // they hold across the statistics loop cost throughput on fuller
            // grids (3 % slower at 1024 workgroups, 6 % faster at 128).
            const int64_t nblk = static_cast<int64_t>(nkb) * a.Hkv * B;
            if (DP == 64 || nblk <= kEarlyRowsMaxWgs)
                quant_kv_launch<T, DP, kStatsFullEarly>(a, g2, vec, s);
            else if constexpr (DP == 128)
                quant_kv_launch<T, DP, kStatsFull>(a, g2, vec, s);
            return;
        }
    }
    quant_kv_launch<T, DP, kStatsPartials>(a, grid, vec, s);
}

hipError_t launch_quant_kv(const QuantKVArgs& a, int nkb, int B, int Dp, int dtype, bool vec,
                           hipStream_t s) {
    if (a.full_stats && dtype != 0) return hipErrorInvalidValue;   // in-kernel sums are exact for fp16 only
    if (dtype == 0) {
        if (Dp == 64) quant_kv_dispatch<__half, 64>(a, nkb, B, vec, s);
        else quant_kv_dispatch<__half, 128>(a, nkb, B, vec, s);
    } else {
        if (Dp == 64) quant_kv_dispatch<__hip_bfloat16, 64>(a, nkb, B, vec, s);
        else quant_kv_dispatch<__hip_bfloat16, 128>(a, nkb, B, vec, s);
    }
    return hipGetLastError();
}

}  // namespace sage
