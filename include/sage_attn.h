/*
 * sage_attn.h -- C ABI of the MI355X (gfx950) quantized-attention library.
 *
 * The library computes SageAttention2-style quantized scaled-dot-product
 * attention: K is smoothed (its per-head mean over tokens is subtracted),
 * Q and K are quantized to INT8, QK^T runs in int32 on the matrix cores and
 * is dequantized, an online (FlashAttention-style) softmax produces P, V is
 * quantized per channel to FP8 E4M3, and P (also FP8) times V accumulates in
 * FP32. Sources for each step, by page and section:
 *   - "SageAttention: Quantized Attention Library" (topgit.dev), core
 *     features list: INT8 QK^T with smoothing, FP8 PV, GQA, HND/NHD;
 *   - "thu-ml/SageAttention" README translation (gittoolsai.com), usage
 *     section: sageattn(q, k, v, tensor_layout, is_causal), fp16/bf16 inputs,
 *     (B,H,S,D) "HND" and (B,S,H,D) "NHD", Lq != Lk and grouped-query heads;
 *   - stable-diffusion.cpp "SageAttention" doc, kernel table and shape
 *     paragraph: smooth K, per-channel FP8 V padded and permuted for the
 *     matrix unit, head dims 1..128 zero-padded to 64 or 128 with the original
 *     softmax scale, output cropped; an unavailable feature is an error;
 *   - "SageAttention-RDNA4" releases: v0.4.0 (hand-written prologue, 64-bit
 *     offsets, key mean summed in fp64), v0.3.0 (strided q/k/v views served
 *     without copies; a refusal carries its reason).
 *
 * Conventions shared by every entry point
 *   - All tensors live in device memory owned by the caller; the library
 *     allocates nothing and keeps no state except a thread-local error text.
 *   - Every call validates all of its arguments on the host before anything
 *     is enqueued. On failure it returns a non-zero sage_status, enqueues
 *     nothing, and sage_last_error() describes the reason. There is no
 *     fallback to another algorithm.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream) and
 *     the call returns without synchronizing. Inputs are read only. The
 *     workspace must stay alive until the enqueued work has finished, and two
 *     calls in flight must not share a workspace.
 *   - Offsets are 64-bit everywhere; element strides are int64.
 *   - A HIP error at launch is returned as SAGE_E_HIP with the HIP message.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SAGE_OK = 0,
    SAGE_E_INVALID = 1,      /* malformed argument (null pointer, bad size, bad stride) */
    SAGE_E_UNSUPPORTED = 2,  /* well formed but outside what the kernels implement (e.g. D > 128) */
    SAGE_E_WORKSPACE = 3,    /* workspace missing, misaligned or too small */
    SAGE_E_HIP = 4           /* the HIP runtime reported an error */
} sage_status;

typedef enum { SAGE_FP16 = 0, SAGE_BF16 = 1 } sage_dtype;

/* Memory order of q, k, v and o: HND = (batch, head, token, dim),
 * NHD = (batch, token, head, dim) (README usage section). */
typedef enum { SAGE_HND = 0, SAGE_NHD = 1 } sage_layout;

/*
 * Format of the P.V product (README translation, kernel list and performance
 * note: "8+8" = INT8 QK^T with FP8 PV, "8+16" = INT8 QK^T with FP16 PV;
 * sm_120a build page, accuracy table: sageattn_qk_int8_pv_fp8_cuda and
 * sageattn_qk_int8_pv_fp16_cuda).
 *   SAGE_PV_FP8:  V quantized per channel to FP8 E4M3, P scaled by 2^8 and
 *                 converted to E4M3 (the default, and the faster product);
 *   SAGE_PV_FP16: V not quantized; P rounded to nearest even in the 16-bit
 *                 input format (binary16 for SAGE_FP16 inputs, bfloat16 for
 *                 SAGE_BF16 inputs) and multiplied with V in that format, FP32
 *                 accumulation (the more accurate product).
 * Q/K quantization, smoothing and the online softmax are the same in both.
 */
typedef enum { SAGE_PV_FP8 = 0, SAGE_PV_FP16 = 1 } sage_pv;

/*
 * Problem description. Strides are in elements, for the (batch, head, token)
 * axes in that order; the dim axis always has stride 1. Any strides are
 * accepted, which covers views into a fused qkv projection (RDNA4 releases
 * v0.3.0); the fast vector loads are used when every base is 16-byte aligned
 * and D and all strides are multiples of 8, scalar loads otherwise.
 * Hq must be a multiple of Hkv (grouped-query attention: q head h reads kv
 * head h / (Hq/Hkv)).
 */
typedef struct {
    int32_t B, Hq, Hkv, Lq, Lk, D;
    int32_t dtype;              /* sage_dtype, shared by q, k, v and o */
    int32_t pv;                 /* sage_pv; sage_problem_init sets SAGE_PV_FP8 */
    int64_t q_stride[3];
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
} sage_problem;

/*
 * Byte offsets of the quantized tensors inside a workspace, and their padded
 * sizes. Dp is the padded head dim (64 or 128); Lq_pad, Lk_pad are the token
 * counts rounded up to the kernel tiles; nkb = Lk_pad / 64 key blocks.
 *   qhat  int8 [B][Hq][Lq_pad][Dp]        per-token INT8 Q codes
 *   sq    f32  [B][Hq][Lq_pad]            per-token Q scale (amax/127)
 *   khat  int8 [B][Hkv][Lk_pad][Dp]       smoothed INT8 K codes
 *   sk    f32  [B][Hkv][nkb]              per-64-token-block K scale
 *   kbar  f32  [B][Hkv][Dp]               key mean over tokens (0 if smooth_k = 0)
 *   vhat  u8   [B][Hkv][nkb][Dp][64]      SAGE_PV_FP8: E4M3 V codes, transposed;
 *                                         inside each 64-token block, token j
 *                                         sits at position 32*((j>>2)&1)
 *                                         + 16*(j>>5) + 4*((j>>3)&3) + (j&3)
 *         u16  [B][Hkv][nkb][Dp][64]      SAGE_PV_FP16: the 16-bit V values,
 *                                         transposed; token j at position j
 *                                         with bits 2 and 3 swapped
 *   vmax  f32  [B][Hkv][Dp]               per-channel max |v| (FP8 V scale = vmax/448)
 *   kpart f64  [B][Hkv][nchunk][Dp]       per-256-token partial key sums (scratch of the
 *                                         prologue; a block-sparse attention call reuses
 *                                         it for the order of its query tiles)
 *   vpart f32  [B][Hkv][nchunk][Dp]       per-256-token partial max |v|
 * Padding rows/channels hold zero codes and zero scales, with one exception:
 * when D < Dp, V^T channel D holds 1.0 (E4M3 0x38, or 1.0 in the 16-bit
 * format) for every real token, so that the attention kernel's P.V product
 * also yields the sum of P (the softmax normaliser) in that channel.
 */
typedef struct {
    int32_t Dp, Lq_pad, Lk_pad, nkb, nchunk, reserved;
    int64_t qhat, sq, khat, sk, kbar, vhat, vmax, kpart, vpart;
    int64_t total_bytes;
} sage_ws_layout;

/* Human-readable text of a status code. Never NULL. */
const char *sage_status_str(int status);

/* Reason for the last non-OK status returned on the calling thread
 * ("" if none). Valid until the next library call on that thread. */
const char *sage_last_error(void);

/* Fill *p for contiguous tensors in `layout` (HND or NHD), all of shape
 * (B, H, L, D) with H = Hq for q and o, Hkv for k and v. Returns SAGE_OK or
 * SAGE_E_INVALID / SAGE_E_UNSUPPORTED for a bad shape or dtype. */
int sage_problem_init(sage_problem *p, int layout, int B, int Hq, int Hkv, int Lq, int Lk,
                      int D, int dtype);

/* Check *p (shape, dtype, strides) without touching any memory. */
int sage_problem_check(const sage_problem *p);

/* Workspace size in bytes for *p, 0 if *p is invalid. */
size_t sage_workspace_bytes(const sage_problem *p);

/* Offsets and padded sizes of the workspace tensors for *p. */
int sage_workspace_layout(const sage_problem *p, sage_ws_layout *out);

/* Number of keys per step of the online softmax (the reference P is
 * quantized against is updated once per block of this many keys). */
int sage_softmax_block_keys(void);

/* What P is quantized against (sage_softmax_spec). */
#define SAGE_REF_MAX 0   /* the running maximum of the row's logits */
#define SAGE_REF_LAZY 2  /* the row's maximum plus 2 factors of two, set by the
                          * first block with a visible key and moved (to the
                          * block's maximum plus 2 factors of two) only when a
                          * block's maximum passes it by more than 0.75 of a
                          * factor of two: P <= 2^0.75, 2^8 P inside E4M3 */

/*
 * The online-softmax rule of a P.V format (topgit.dev, "SageAttention vs
 * FlashAttention": blockwise softmax with a running maximum; the pages do not
 * say against which value P is rounded, and any reference at or above the
 * logits gives the same softmax after normalisation). *block_keys: keys per
 * softmax step (128); *reference: SAGE_REF_LAZY for SAGE_PV_FP8, SAGE_REF_MAX
 * for SAGE_PV_FP16 (whose kernel lets the maximum lag by up to a factor 2^8
 * and rescales only then, which moves the rounding point of P but not the
 * softmax). Either pointer may be NULL. SAGE_E_INVALID for an unknown pv.
 */
int sage_softmax_spec(int pv, int *block_keys, int *reference);

/*
 * The quantization prologue (stable-diffusion.cpp doc: smooth K, per-channel
 * FP8 V, pad and permute; RDNA4 releases v0.4.0: hand-written prologue, fp64
 * key mean). Reads q, k, v (device, layout and strides of *p) and writes every
 * tensor of the workspace. smooth_k = 0 skips the key mean (kbar = 0).
 * ws must be 256-byte aligned and at least sage_workspace_bytes(p) long.
 */
int sage_quantize(const sage_problem *p, const void *q, const void *k, const void *v,
                  int smooth_k, void *ws, size_t ws_bytes, void *stream);

/*
 * The attention kernel on a workspace filled by sage_quantize with the same
 * *p (README usage section: is_causal; sd.cpp doc: original softmax scale).
 * Writes o (device, dtype of *p, strides o_stride) for all Lq x D outputs.
 * is_causal = 1 masks key j for query i when j > i (top-left alignment, as
 * torch scaled_dot_product_attention does for Lq != Lk); is_causal = 2 masks
 * it when j > i + Lk - Lq (bottom-right alignment: the last query sees every
 * key; queries that see no key get zero rows). One pass, no key splits (see
 * sage_attn_quantized_ex). sm_scale must be finite and
 * > 0; callers pass 1/sqrt(D) of the original D by default.
 * o must not overlap the workspace.
 */
int sage_attn_quantized(const sage_problem *p, const void *ws, size_t ws_bytes, void *o,
                        int is_causal, float sm_scale, void *stream);

/* ------------------------------------------------------------------------ */
/* Key-range splits, bottom-right causal alignment and the log-sum-exp.      */
/*                                                                          */
/* The pages serve q with another sequence length than k and v (README      */
/* translation, news 2024-11-11; stable-diffusion.cpp doc, shape paragraph:  */
/* different query/key lengths). When Lq is short against Lk the query tiles */
/* alone leave compute units idle, so the keys of every query tile can be    */
/* cut into nsplit contiguous ranges, each run by its own workgroup with its */
/* own online softmax; a second kernel merges the partials exactly by the    */
/* log-sum-exp rule (m = max_s m_s, O = sum_s e^(m_s - m) O_s / sum_s        */
/* e^(m_s - m) l_s). Range s of the nb = ceil(Lk / 128) softmax blocks is   */
/* [floor(s nb / nsplit), floor((s + 1) nb / nsplit)). P is quantized       */
/* against each range's own running max, so a split result differs from the */
/* one-pass result by the rounding of P only.                                */
/* ------------------------------------------------------------------------ */
#define SAGE_MAX_SPLIT 16

typedef struct {
    int32_t is_causal;   /* 0: no mask; 1: key j masked for query i when j > i (top-left);
                            2: masked when j > i + Lk - Lq (bottom-right, per batch entry);
                            a query that sees no key gets a zero output row */
    int32_t nsplit;      /* key ranges per query tile, 1..SAGE_MAX_SPLIT; 0 = sage_split_count(p) */
    float sm_scale;      /* finite and > 0 */
    int32_t reserved;    /* must be 0 */
    float *lse;          /* optional device f32 [B][Hq][Lq], contiguous: for each query the natural
                            log of the sum of its softmax weights before normalisation, as the
                            weights were used (exp(logit - max) after rounding of P, times
                            exp(max)); -inf where no key is visible. NULL = not written */
    void *part;          /* device scratch of sage_split_bytes(p, nsplit) bytes, 256-byte aligned,
                            for the partials of a split run; unused (may be NULL) when the
                            resolved split count is 1. Must not overlap o, lse or the workspace */
    size_t part_bytes;
    const uint8_t *block_mask;  /* optional block-sparse pattern (see below); NULL = dense */
} sage_attn_opts;

/*
 * Block-sparse attention (README translation, news 2025-06-19: the Sparse
 * SageAttention APIs compute attention under any block-sparse pattern;
 * topgit.dev feature list: a sparse variant extends the quantized kernel to
 * arbitrary block-sparse patterns). block_mask is device u8
 * [B][Hq][ceil(Lq / SAGE_MASK_BLOCK_Q)][ceil(Lk / SAGE_MASK_BLOCK_K)],
 * contiguous: a zero flag skips the whole block of SAGE_MASK_BLOCK_Q queries
 * x SAGE_MASK_BLOCK_K keys (those logits are -inf, and the kernel neither
 * loads nor multiplies them). It combines with is_causal by "and"; a query
 * that sees no key gets a zero output row and LSE -inf. Dense problems only
 * (sage_varlen_attn_ex refuses a mask). It is read while o, lse and the
 * scratch are written, so it must not overlap them or the workspace.
 */
#define SAGE_MASK_BLOCK_Q 128
#define SAGE_MASK_BLOCK_K 128

/* The split count the library picks for *p when nsplit = 0: 1 when the query
 * tiles alone fill every workgroup slot of the 256 compute units, else as many
 * ranges as keep all tiles resident at once, at most SAGE_MAX_SPLIT and with
 * at least four 128-key blocks per range. 0 if *p is invalid. */
int sage_split_count(const sage_problem *p);

/* Bytes of scratch a run with nsplit ranges needs (0 = sage_split_count(p));
 * 0 when that count is 1 or *p is invalid. */
size_t sage_split_bytes(const sage_problem *p, int nsplit);

/* sage_attn_quantized with the options above. With a resolved split count
 * of 1 it is one kernel; otherwise the split kernel and the merge, both on
 * `stream`. */
int sage_attn_quantized_ex(const sage_problem *p, const void *ws, size_t ws_bytes, void *o,
                           const sage_attn_opts *opts, void *stream);

/* The whole path in one call (README usage section: sageattn(q, k, v,
 * tensor_layout, is_causal)): the result is that of sage_quantize followed by
 * sage_attn_quantized on the same stream, bit for bit. When the attention
 * launch holds more workgroups than the GPU runs at once, Q is quantized
 * inside the attention kernel, which reads q directly (each query's codes and
 * scale are computed where they are used, by the same per-token rule) and the
 * prologue skips its pass over q; otherwise the prologue codes Q as
 * sage_quantize does. The workspace's K and V sections are written as by
 * sage_quantize; its qhat and s_q sections are unspecified afterwards.
 * One pass, no key splits. o must not overlap q, k, v or the workspace; the
 * workspace must not overlap q, k or v. */
int sage_attn(const sage_problem *p, const void *q, const void *k, const void *v, void *o,
              int is_causal, float sm_scale, int smooth_k, void *ws, size_t ws_bytes,
              void *stream);

/* sage_attn with the options of sage_attn_quantized_ex (key ranges, LSE,
 * block mask): the same result as sage_quantize followed by
 * sage_attn_quantized_ex, bit for bit, with Q quantized where sage_attn
 * would (counting the workgroups of all key ranges). Besides the rules of
 * both, lse and the split scratch must not overlap q, k or v. */
int sage_attn_ex(const sage_problem *p, const void *q, const void *k, const void *v, void *o,
                 int smooth_k, void *ws, size_t ws_bytes, const sage_attn_opts *opts, void *stream);

/*
 * sage_attn_ex without any allocation by the caller or the library, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it).
 * The workspace and the split partials live in one library-owned static
 * device array of SAGE_NOALLOC_SCRATCH_BYTES, one per GPU, which the library
 * looks up on a device's first call and holds until the process ends. The
 * caller passes the inputs and the outputs (o, opts->lse) only; opts->part
 * must be NULL and opts->part_bytes 0. A problem whose workspace plus split
 * partials (sage_noalloc_bytes) exceed the array is refused with
 * SAGE_E_WORKSPACE before anything is enqueued (B=2 H=24 L=4096 D=128 fits;
 * B=1 H=40 L=14040 D=80 does not). The stream must belong to the current
 * device. Results are those of sage_attn_ex with the same options, bit for
 * bit. The prologue rewrites every scratch byte the attention kernel reads,
 * so nothing needs clearing between calls; but every call on one GPU uses
 * the same array, so calls that overlap in time on one GPU (on two streams,
 * or from two threads without ordering) race and give undefined results.
 */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* Scratch bytes sage_attn_noalloc needs for *p with nsplit key ranges
 * (0 = sage_split_count(p)); 0 if *p is invalid. */
size_t sage_noalloc_bytes(const sage_problem *p, int nsplit);
int sage_attn_noalloc(const sage_problem *p, const void *q, const void *k, const void *v, void *o,
                      int smooth_k, const sage_attn_opts *opts, void *stream);

/* The two launches of sage_attn_ex as separate calls, for callers that keep
 * one K/V workspace for several query sets, or time the two parts.
 * sage_quantize_kv: the K/V part of sage_quantize (key statistics, smoothed
 * INT8 K codes and scales, V codes and scales); the Q sections are left
 * unwritten. The workspace must not overlap k or v.
 * sage_attn_q_ex: sage_attn_quantized_ex on a workspace whose K/V sections
 * were written (by sage_quantize or sage_quantize_kv with the same *p), with
 * Q quantized inside the attention kernel from q; the workspace's Q sections
 * are not read. o, lse and the split scratch must not overlap q. */
int sage_quantize_kv(const sage_problem *p, const void *k, const void *v, int smooth_k, void *ws,
                     size_t ws_bytes, void *stream);
int sage_attn_q_ex(const sage_problem *p, const void *q, const void *ws, size_t ws_bytes, void *o,
                   const sage_attn_opts *opts, void *stream);

/*
 * Exact int32 logits qhat . khat^T of one (batch b, q-head hq), computed by the
 * same matrix-core tile routine as sage_attn_quantized, for bit-exact tests.
 * out: device int32 [Lq_pad][Lk_pad] (sizes from sage_workspace_layout).
 */
int sage_debug_qk_int32(const sage_problem *p, const void *ws, size_t ws_bytes, int b, int hq,
                        int32_t *out, void *stream);

/* ------------------------------------------------------------------------ */
/* Packed variable-length sequences (README translation, news 2024-11-12 and */
/* kernel list: sageattn_varlen, "different sequence lengths in one batch";  */
/* the topgit.dev feature list: variable-length sequences via              */
/* sageattn_varlen).                                                        */
/*                                                                          */
/* q is [total_q, Hq, D] and k, v are [total_k, Hkv, D] (token-major, as    */
/* the packed layout of the reference API); sequence b holds q rows         */
/* [cu_seqlens_q[b], cu_seqlens_q[b+1]) and k/v rows                        */
/* [cu_seqlens_k[b], cu_seqlens_k[b+1]). Each sequence is one attention     */
/* problem of its own: its own key mean (smoothing), K block scales, V      */
/* channel scales, causal mask (top-left within the sequence) and online    */
/* softmax; results are those of the dense call on that sequence alone.     */
/* The P.V format is chosen by pv as for dense problems (the reference's    */
/* varlen kernel uses FP16 PV; the Python binding defaults to it).          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t B, Hq, Hkv, D;      /* B = number of sequences */
    int32_t dtype;              /* sage_dtype */
    int32_t pv;                 /* sage_pv */
    int32_t total_q, total_k;   /* rows of the packed q and of the packed k / v */
    int32_t max_seqlen_q;       /* no sequence is longer (grid size; longer ones are cut) */
    int32_t max_seqlen_k;
    int64_t q_stride[2];        /* elements: (token, head); the dim stride is 1 */
    int64_t k_stride[2];
    int64_t v_stride[2];
    int64_t o_stride[2];
} sage_varlen_problem;

/* Fill *p for contiguous packed tensors [total, H, D] and check it. */
int sage_varlen_problem_init(sage_varlen_problem *p, int B, int Hq, int Hkv, int total_q,
                             int total_k, int max_seqlen_q, int max_seqlen_k, int D, int dtype,
                             int pv);

/* Check *p without touching any memory. */
int sage_varlen_problem_check(const sage_varlen_problem *p);

/*
 * Workspace of a packed problem: the same sections as sage_ws_layout, per
 * head over all sequences. Fields: Lq_pad = Q rows per head
 * (total_q + 256 B); Lk_pad = K rows per head (64 nkb); nkb = 64-token K
 * blocks per head ((total_k + 127 B) / 64 + 2); nchunk = key-sum chunks per
 * head ((total_k + 255 B) / 256 + 1). Sequence b's rows of head h start at
 * Q row h Lq_pad + cu_q[b] + 255 b, K block h nkb + (cu_k[b] + 127 b) / 64
 * and chunk h nchunk + (cu_k[b] + 255 b) / 256 (integer division), which
 * leaves each sequence its tokens rounded up to 256 Q rows, 128 K rows and
 * 256-token chunks. kbar and vmax are [B][Hkv][Dp].
 */
size_t sage_varlen_workspace_bytes(const sage_varlen_problem *p);
int sage_varlen_workspace_layout(const sage_varlen_problem *p, sage_ws_layout *out);

/*
 * Quantization prologue and attention for all sequences, on one stream, with
 * Q quantized where sage_attn would (the workspace's qhat and s_q sections
 * are unspecified afterwards).
 * cu_seqlens_q / cu_seqlens_k: device int32 arrays of B + 1 non-decreasing
 * offsets from 0 to total_q / total_k. They are read only by the kernels; the
 * host does not check their contents: an offset outside [0, total] is
 * clamped and a sequence longer than max_seqlen is cut to it, so malformed
 * offsets give unspecified results but never an access outside q, k, v, o or
 * the workspace. A sequence without keys gets zero output rows. is_causal as
 * for sage_attn_quantized, within each sequence.
 * o is [total_q, Hq, D] (strides o_stride) and must not overlap the inputs or
 * the workspace.
 */
int sage_varlen_attn(const sage_varlen_problem *p, const void *q, const void *k, const void *v,
                     void *o, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                     int is_causal, float sm_scale, int smooth_k, void *ws, size_t ws_bytes,
                     void *stream);

/* Packed-sequence forms of the split entry points. The split count applies to
 * every sequence (a sequence with fewer 128-key blocks than ranges leaves
 * some empty); nsplit = 0 picks it from the packed totals as
 * sage_split_count does from a dense shape. opts->lse, when set, is device
 * f32 [Hq][total_q] (head-major, the packed query order inside each head).
 * is_causal = 2 aligns each sequence's mask bottom-right. */
int sage_varlen_split_count(const sage_varlen_problem *p);
size_t sage_varlen_split_bytes(const sage_varlen_problem *p, int nsplit);
int sage_varlen_attn_ex(const sage_varlen_problem *p, const void *q, const void *k, const void *v,
                        void *o, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                        int smooth_k, void *ws, size_t ws_bytes, const sage_attn_opts *opts,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
