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
constexpr int kMaskBlockQ = 128;   // queries per block-mask flag (keys per flag: kBK)

// Where the tokens and workspace rows of batch entry b are. Dense problems:
// every entry has Lq / Lk tokens at batch stride. Packed variable-length
// problems (cu_q != nullptr): entry b holds tokens [cu_q[b], cu_q[b+1]) of the
// packed q and [cu_k[b], cu_k[b+1]) of k and v, and its workspace rows start
// at fixed functions of those offsets (see seq_at), so the layout is known on
// the host from the packed totals alone.
struct SeqMap {
    const int32_t* cu_q;           // device prefix sums [B+1], nullptr for dense problems
    const int32_t* cu_k;
    int Lq, Lk;                    // dense: the lengths; packed: upper bounds of every entry's lengths
    int total_q, total_k;          // packed: number of q and of k/v tokens
    int64_t q_bstride, q_hstride;  // workspace Q rows (qhat, sq): entry b, head h start at
                                   //   qrow0(b) + h * q_hstride (qrow0 includes b * q_bstride)
    int64_t kb_bstride, kb_hstride;// workspace 64-token K blocks (khat rows / 64, sk, vhat blocks)
    int64_t c_bstride, c_hstride;  // workspace 256-token chunks (kpart, vpart)
};

// One batch entry, resolved.
struct Seq {
    int Lq, Lk;                    // its lengths
    int64_t qtok0, ktok0;          // token index of its first q / k row in the inputs (0 when dense)
    int64_t qrow0, kblk0, chunk0;  // its first workspace Q row, K block and chunk, head 0
};

// Packed layout: entry b's Q rows start at cu_q[b] + 255 b, which leaves every
// entry room for its rows rounded up to 256; its K blocks start at
// floor((cu_k[b] + 127 b) / 64), room for its tokens rounded up to 128; its
// chunks at floor((cu_k[b] + 255 b) / 256). Offsets are clamped to the packed
// totals and lengths to the bounds, so malformed prefix sums cannot address
// outside the buffers.
__device__ __forceinline__ Seq seq_at(const SeqMap& m, int b) {
    Seq s;
    if (m.cu_q == nullptr) {
        s.Lq = m.Lq;
        s.Lk = m.Lk;
        s.qtok0 = 0;
        s.ktok0 = 0;
        s.qrow0 = b * m.q_bstride;
        s.kblk0 = b * m.kb_bstride;
        s.chunk0 = b * m.c_bstride;
    } else {
        const int q0 = min(max(m.cu_q[b], 0), m.total_q);
        const int q1 = min(max(m.cu_q[b + 1], q0), min(m.total_q, q0 + m.Lq));
        const int k0 = min(max(m.cu_k[b], 0), m.total_k);
        const int k1 = min(max(m.cu_k[b + 1], k0), min(m.total_k, k0 + m.Lk));
        s.Lq = q1 - q0;
        s.Lk = k1 - k0;
        s.qtok0 = q0;
        s.ktok0 = k0;
        s.qrow0 = q0 + 255LL * b;
        s.kblk0 = (k0 + 127LL * b) / 64;
        s.chunk0 = (k0 + 255LL * b) / 256;
    }
    return s;
}

struct StatsArgs {
    SeqMap m;
    const void* k;
    const void* v;
    int64_t ks0, ks1, ks2;         // element strides of k (batch, head, token)
    int64_t vs0, vs1, vs2;
    int Hkv, D, Dp, nchunk, smooth; // nchunk: chunks of the longest entry
    double* kpart;                 // [chunk slot][Dp], slot = chunk0(b) + h * c_hstride + chunk
    float* vpart;                  // same slots
};

struct QuantQArgs {
    SeqMap m;
    const void* q;
    int64_t qs0, qs1, qs2;
    int B, Hq, D;
    int ntile;                     // row tiles per (entry, head) of the longest entry
    int8_t* qhat;                  // [row][Dp], row = qrow0(b) + h * q_hstride + i
    float* sq;                     // [row]
};

struct QuantKVArgs {
    SeqMap m;
    const void* k;
    const void* v;
    int64_t ks0, ks1, ks2;
    int64_t vs0, vs1, vs2;
    int Hkv, D, smooth;
    const double* kpart;           // chunk partial key sums (StatsArgs slots)
    const float* vpart;            // chunk partial max |v|
    float* kbar;                   // [B][Hkv][Dp] written by the first block's workgroup of each
    float* vmax;                   //   head, or before the codes kernel for long entries
    int8_t* khat;                  // [64 * block + token][Dp], block = kblk0(b) + h * kb_hstride + i
    float* sk;                     // [block]
    uint8_t* vhat;                 // [block][Dp][64] elements, permuted inside each block
    int pv16;                      // 0: FP8 E4M3 codes; 1: the 16-bit input values
    int nchunk;                    // 256-token chunks of the longest entry (more than 32: the
                                   //   statistics are finished by a launch of their own)
    int full_stats;                // 1: fp16 inputs and at most kFullStatsKeys keys per entry; every
                                   //   workgroup adds up its head's k and v itself (no statistics
                                   //   launch, no chunk partials)
};

struct AttnArgs {
    SeqMap m;
    const int8_t* qhat;
    const float* sq;
    const int8_t* khat;
    const float* sk;
    const uint8_t* vhat;
    const float* vmax;
    void* o;
    int64_t os0, os1, os2;         // element strides of o (batch, head, token)
    const void* q;                 // non-null: the input q (element strides qs0..qs2); the kernel
                                   //   quantizes its own query rows with the prologue's rule, and
                                   //   qhat / sq are not read. Null: Q codes and scales come from
                                   //   the workspace
    int64_t qs0, qs1, qs2;
    int q_vec;                     // q rows may be read 16 bytes at a time (aligned, D % 8 == 0)
    int B, Hq, Hkv, G, D;
    float scale_log2;              // sm_scale * log2(e)
    int lch;                       // D < Dp: V^T channel D holds 1.0 (the prologue writes it), so
                                   //   O^T channel D accumulates the normaliser
    int causal_br;                 // causal launches: 1 = bottom-right alignment, key j visible to
                                   //   query i iff j <= i + Lk - Lq (per entry); 0 = j <= i
    int nsplit;                    // key ranges per query tile; 1 = one pass that writes o
    uint16_t* part_o;              // nsplit > 1: [split][Q row][Dp] each range's normalised output
                                   //   row, in the output format
    float2* part_ml;               // nsplit > 1: [split][Q row] (running max, log2 units; normaliser)
    int64_t part_rows;             // Q rows per split (the workspace's Q rows, all heads)
    float* lse;                    // optional: natural-log sum of the softmax weights per query
    int64_t ls0, ls1, ls2;         // element strides of lse (batch, head, token)
    const uint8_t* bmask;          // block-sparse launches: [B][Hq][bm_nq][bm_nk] flags, one per
                                   //   kMaskBlockQ queries x kBK keys; 0 = block skipped
    int bm_nq, bm_nk;
    int32_t* tord;                 // non-null (dense block-sparse launches without a causal mask):
                                   //   the logical tile each workgroup runs, per XCD share, heaviest
                                   //   first (written by the tile-dealing kernel)
    // debug dump of int32 logits (one head of a dense problem)
    int32_t* dump;
    int64_t dump_ld;               // row length of the dump (Lk_pad)
    int dump_b, dump_hq;
};

// Launchers; return the hipError_t of the launch.
hipError_t launch_stats_q(const StatsArgs& sa, const QuantQArgs& qa, int B, int Dp, int dtype, bool vec_q,
                          hipStream_t s);
// nkb: 64-token K blocks of the longest entry, rounded up to 128 tokens
hipError_t launch_quant_kv(const QuantKVArgs& a, int nkb, int B, int Dp, int dtype, bool vec,
                           hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out, bool pv16,
                       hipStream_t s);   // block-sparse when a.bmask != nullptr
// the two P.V formats of launch_attn (separate translation units)
hipError_t launch_attn_fp8(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out, hipStream_t s);
hipError_t launch_attn_pv16(const AttnArgs& a, int Dp, int dtype, bool causal, bool vec_out, hipStream_t s);
hipError_t launch_attn_dump(const AttnArgs& a, int Dp, hipStream_t s);
// block-sparse launches: orders each XCD's share of `full` logical tiles (of
// query tiles of bq rows, nqt per head) by their count of loaded key blocks
// into a.tord
hipError_t launch_deal_tiles(const AttnArgs& a, int bq, int nqt, int full, hipStream_t s);
// nsplit > 1: merges the partials of every split into o (and lse)
hipError_t launch_combine(const AttnArgs& a, int Dp, int dtype, bool vec_out, bool pv16, hipStream_t s);

constexpr int kMaxSplit = 16;      // largest number of key ranges per query tile
constexpr int kFullStatsKeys = 1024;  // keys per entry up to which short fp16 heads skip the
                                      // statistics launch

}  // namespace sage
