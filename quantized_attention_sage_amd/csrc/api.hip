// Host side of the C ABI declared in include/sage_attn.h: argument checks,
// workspace layout, kernel launches and error reporting.
//
// Every entry point checks all of its arguments before it enqueues anything;
// a refusal returns a status and leaves its reason in a thread-local string
// ("SageAttention-RDNA4" releases, v0.3.0: one acceptance rule whose refusal
// carries its reason; stable-diffusion.cpp doc: an unavailable feature is
// reported as an error rather than silently replaced).
#include "sage_attn.h"
#include "sage_kernels.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int ok() {
    g_err.clear();
    return SAGE_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int padded_dim(int D) { return D <= 64 ? 64 : 128; }

// Largest element offset reached by a (n0, n1, n2, D) view with strides s.
int64_t max_offset(const int64_t s[3], int64_t n0, int64_t n1, int64_t n2, int64_t D) {
    return s[0] * (n0 - 1) + s[1] * (n1 - 1) + s[2] * (n2 - 1) + (D - 1);
}

// True when distinct (i0, i1, i2) rows of D contiguous elements never overlap.
bool rows_disjoint(const int64_t s[3], const int64_t n[3], int64_t D) {
    int idx[3] = {0, 1, 2};
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (s[idx[b]] < s[idx[a]]) std::swap(idx[a], idx[b]);
    int64_t span = D;
    for (int a = 0; a < 3; ++a) {
        const int i = idx[a];
        if (n[i] <= 1) continue;
        if (s[i] < span) return false;
        span = s[i] * (n[i] - 1) + span;
    }
    return true;
}

bool vec_ok(const void* base, const int64_t s[3], int D, int align_elems) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(base);
    if (p % (2 * align_elems) != 0) return false;
    if (D % align_elems != 0) return false;
    for (int i = 0; i < 3; ++i)
        if (s[i] % align_elems != 0) return false;
    return true;
}

struct Extent {
    uintptr_t lo, hi;
};

Extent extent_of(const void* base, const int64_t s[3], int64_t n0, int64_t n1, int64_t n2,
                 int64_t D) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(base);
    return {p, p + 2 * static_cast<uintptr_t>(max_offset(s, n0, n1, n2, D) + 1)};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

int check_strides(const char* name, const int64_t s[3]) {
    for (int i = 0; i < 3; ++i)
        if (s[i] < 0)
            return fail(SAGE_E_UNSUPPORTED, "%s stride[%d] = %lld is negative", name, i,
                        static_cast<long long>(s[i]));
    return SAGE_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int hip_fail(hipError_t e, const char* what) {
    return fail(SAGE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int layout_of(const sage_problem* p, sage_ws_layout* L) {
    const int64_t B = p->B, Hq = p->Hq, Hkv = p->Hkv;
    std::memset(L, 0, sizeof(*L));
    L->Dp = padded_dim(p->D);
    L->Lq_pad = static_cast<int32_t>(round_up(p->Lq, sage::kQPad));
    L->Lk_pad = static_cast<int32_t>(round_up(p->Lk, sage::kKPad));
    L->nkb = L->Lk_pad / sage::kKeyBlock;
    L->nchunk = static_cast<int32_t>((p->Lk + sage::kChunk - 1) / sage::kChunk);
    const int64_t Dp = L->Dp;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    L->qhat = take(B * Hq * L->Lq_pad * Dp);
    L->sq = take(B * Hq * L->Lq_pad * 4);
    L->khat = take(B * Hkv * L->Lk_pad * Dp);
    L->sk = take(B * Hkv * L->nkb * 4);
    L->kbar = take(B * Hkv * Dp * 4);
    L->vhat = take(B * Hkv * static_cast<int64_t>(L->nkb) * Dp * 64 * (p->pv == SAGE_PV_FP16 ? 2 : 1));
    L->vmax = take(B * Hkv * Dp * 4);
    L->kpart = take(B * Hkv * static_cast<int64_t>(L->nchunk) * Dp * 8);
    L->vpart = take(B * Hkv * static_cast<int64_t>(L->nchunk) * Dp * 4);
    L->total_bytes = off;
    return SAGE_OK;
}

int check_ws(const sage_problem* p, const void* ws, size_t ws_bytes, sage_ws_layout* L) {
    layout_of(p, L);
    if (ws == nullptr) return fail(SAGE_E_WORKSPACE, "workspace pointer is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return fail(SAGE_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < static_cast<size_t>(L->total_bytes))
        return fail(SAGE_E_WORKSPACE, "workspace has %zu bytes, needs %lld", ws_bytes,
                    static_cast<long long>(L->total_bytes));
    return SAGE_OK;
}

// The batch-entry map of a dense problem: entry b at batch stride, uniform lengths.
sage::SeqMap dense_map(const sage_problem* p, const sage_ws_layout& L) {
    sage::SeqMap m{};
    m.Lq = p->Lq;
    m.Lk = p->Lk;
    m.q_bstride = static_cast<int64_t>(p->Hq) * L.Lq_pad;
    m.q_hstride = L.Lq_pad;
    m.kb_bstride = static_cast<int64_t>(p->Hkv) * L.nkb;
    m.kb_hstride = L.nkb;
    m.c_bstride = static_cast<int64_t>(p->Hkv) * L.nchunk;
    m.c_hstride = L.nchunk;
    return m;
}

// Everything the launches need, for dense and packed problems alike. Strides
// are (batch, head, token) element strides; packed problems have batch stride
// 0 and address entries through the map.
struct Plan {
    int B, Hq, Hkv, D, dtype, pv;
    int64_t qs[3], ks[3], vs[3], os[3];
    sage::SeqMap m;
    sage_ws_layout L;
    int nkb_max;           // 64-token blocks of the longest entry, rounded up to 128 tokens
    int nchunk_max;        // 256-token chunks of the longest entry
    int64_t qrows;         // workspace Q rows over all entries and heads
    int64_t qtiles;        // query tiles of the attention kernel at BQ = 128 (at most; an upper
                           //   bound for packed problems), for the split choice
    int nb_max;            // 128-key softmax blocks of the longest entry
};

// ---- key-range splits ----

constexpr int kComputeUnits = 256;     // MI355X

int query_rows_per_wg(int pv) { return pv == SAGE_PV_FP16 ? 2 * sage::kBQ : sage::kBQ; }

constexpr int kMinSplitBlocks = 4;     // 128-key blocks per range at least (a range's fixed
                                       // costs and the merge outweigh shorter ones)

// The split count for a launch of nwg query tiles over entries of at most nb
// softmax blocks: 1 when the tiles fill every workgroup slot, else as many
// ranges as keep all tiles resident in one round, each of at least
// kMinSplitBlocks blocks.
int64_t wg_slots(const Plan& P) { return static_cast<int64_t>(kComputeUnits) * (P.pv == SAGE_PV_FP16 ? 1 : 2); }
int64_t query_wgs(const Plan& P) {
    return (P.qtiles * sage::kBQ + query_rows_per_wg(P.pv) - 1) / query_rows_per_wg(P.pv);
}

int auto_split(const Plan& P) {
    const int64_t slots = wg_slots(P);
    const int64_t nwg = query_wgs(P);
    if (nwg >= slots) return 1;
    int64_t S = slots / (nwg > 0 ? nwg : 1);
    if (S > sage::kMaxSplit) S = sage::kMaxSplit;
    if (S > P.nb_max / kMinSplitBlocks) S = P.nb_max / kMinSplitBlocks;
    return S < 1 ? 1 : static_cast<int>(S);
}

// Short fp16 heads: the K/V codes kernel adds up each head's keys itself
// (exact in any order, see quant_kv_kernel), so the K/V prologue has no
// statistics launch.
bool kv_stats_inline(const Plan& P) { return P.dtype == 0 && P.m.Lk <= sage::kFullStatsKeys; }

// Whether the one-call paths quantize Q inside the attention kernel. That
// saves the prologue's pass over q, and costs each tile a 16-bit read of its
// rows and the code arithmetic before its first block, which other tiles'
// work hides when the launch runs in more than one round of workgroups. In
// one round every tile pays it at the same moment, so the prologue codes Q,
// unless the K/V statistics need no launch of their own: then the Q codes
// would be all that launch does, and fusing them saves the launch.
bool fuse_q(const Plan& P, int nsplit) { return query_wgs(P) * nsplit > wg_slots(P) || kv_stats_inline(P); }

// Scratch of a split run: each range's normalised rows [S][qrows][Dp] in the output format
// (16-bit), then (m, l) [S][qrows] f32.
int64_t part_ml_offset(const Plan& P, int S) { return round_up(static_cast<int64_t>(S) * P.qrows * P.L.Dp * 2, 256); }
int64_t split_bytes(const Plan& P, int S) {
    return S <= 1 ? 0 : part_ml_offset(P, S) + round_up(static_cast<int64_t>(S) * P.qrows * 8, 256);
}

// What one attention launch is asked to do.
struct AttnCall {
    int is_causal = 0;     // 0, 1 top-left, 2 bottom-right
    float sm_scale = 1.0f;
    int nsplit = 1;
    float* lse = nullptr;
    int64_t ls[3] = {0, 0, 0};
    void* part = nullptr;
    const uint8_t* bmask = nullptr;    // [B][Hq][ceil(Lq/128)][ceil(Lk/128)]
};

static_assert(SAGE_MASK_BLOCK_Q == sage::kMaskBlockQ && SAGE_MASK_BLOCK_K == sage::kBK,
              "block-mask granularity is the kernel's query tile and softmax block");

// The prologue. with_q = false leaves the Q codes to the attention kernel
// (fused Q): only the K/V statistics and codes are written.
int launch_quantize(const Plan& P, const void* q, const void* k, const void* v, int smooth_k, void* ws,
                    hipStream_t s, bool with_q = true) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    const sage_ws_layout& L = P.L;
    const bool vec_q = vec_ok(q, P.qs, P.D, 8);
    const bool vec_kv = vec_ok(k, P.ks, P.D, 8) && vec_ok(v, P.vs, P.D, 8);

    sage::StatsArgs sa{};
    sa.m = P.m;
    sa.k = k;
    sa.v = v;
    sa.ks0 = P.ks[0]; sa.ks1 = P.ks[1]; sa.ks2 = P.ks[2];
    sa.vs0 = P.vs[0]; sa.vs1 = P.vs[1]; sa.vs2 = P.vs[2];
    // short fp16 heads: the codes kernel adds up each head's k and v itself
    // (exact in any order, see quant_kv_kernel), so the statistics part of
    // the first launch is left out
    const bool full_stats = kv_stats_inline(P);
    sa.Hkv = P.Hkv; sa.D = P.D; sa.Dp = L.Dp; sa.nchunk = full_stats ? 0 : P.nchunk_max;
    sa.smooth = smooth_k ? 1 : 0;
    sa.kpart = reinterpret_cast<double*>(base + L.kpart);
    sa.vpart = reinterpret_cast<float*>(base + L.vpart);
    sage::QuantQArgs qa{};
    qa.m = P.m;
    qa.q = q;
    qa.qs0 = P.qs[0]; qa.qs1 = P.qs[1]; qa.qs2 = P.qs[2];
    qa.B = P.B; qa.Hq = P.Hq; qa.D = P.D;
    // rows per Q workgroup: 4 rows per thread, Dp/8 threads per row
    const int rows_per_wg = 4 * (256 / (L.Dp / 8));
    qa.ntile = with_q ? static_cast<int>(round_up(P.m.Lq, sage::kQPad) / rows_per_wg) : 0;
    qa.qhat = reinterpret_cast<int8_t*>(base + L.qhat);
    qa.sq = reinterpret_cast<float*>(base + L.sq);
    hipError_t e = sage::launch_stats_q(sa, qa, P.B, L.Dp, P.dtype, vec_q, s);
    if (e != hipSuccess) return hip_fail(e, "stats/quant_q launch");

    sage::QuantKVArgs ka{};
    ka.m = P.m;
    ka.k = k;
    ka.v = v;
    ka.ks0 = sa.ks0; ka.ks1 = sa.ks1; ka.ks2 = sa.ks2;
    ka.vs0 = sa.vs0; ka.vs1 = sa.vs1; ka.vs2 = sa.vs2;
    ka.Hkv = P.Hkv; ka.D = P.D; ka.smooth = sa.smooth;
    ka.kpart = sa.kpart;
    ka.vpart = sa.vpart;
    ka.kbar = reinterpret_cast<float*>(base + L.kbar);
    ka.vmax = reinterpret_cast<float*>(base + L.vmax);
    ka.khat = reinterpret_cast<int8_t*>(base + L.khat);
    ka.sk = reinterpret_cast<float*>(base + L.sk);
    ka.vhat = base + L.vhat;
    ka.pv16 = P.pv == SAGE_PV_FP16 ? 1 : 0;
    ka.nchunk = P.nchunk_max;
    ka.full_stats = full_stats ? 1 : 0;
    e = sage::launch_quant_kv(ka, P.nkb_max, P.B, L.Dp, P.dtype, vec_kv, s);
    if (e != hipSuccess) return hip_fail(e, "quant_kv launch");
    return ok();
}

void fill_attn_args(const Plan& P, const void* ws, sage::AttnArgs* a) {
    const uint8_t* base = static_cast<const uint8_t*>(ws);
    const sage_ws_layout& L = P.L;
    std::memset(a, 0, sizeof(*a));
    a->m = P.m;
    a->qhat = reinterpret_cast<const int8_t*>(base + L.qhat);
    a->sq = reinterpret_cast<const float*>(base + L.sq);
    a->khat = reinterpret_cast<const int8_t*>(base + L.khat);
    a->sk = reinterpret_cast<const float*>(base + L.sk);
    a->vhat = base + L.vhat;
    a->vmax = reinterpret_cast<const float*>(base + L.vmax);
    a->B = P.B; a->Hq = P.Hq; a->Hkv = P.Hkv; a->G = P.Hq / P.Hkv;
    a->D = P.D;
    a->lch = P.D < L.Dp ? 1 : 0;
}

// q non-null: the attention kernel quantizes Q from it (fused Q).
int launch_attention(const Plan& P, const void* ws, void* o, const AttnCall& c, hipStream_t s,
                     const void* q = nullptr) {
    sage::AttnArgs a;
    fill_attn_args(P, ws, &a);
    if (q != nullptr) {
        a.q = q;
        a.qs0 = P.qs[0]; a.qs1 = P.qs[1]; a.qs2 = P.qs[2];
        a.q_vec = vec_ok(q, P.qs, P.D, 8) ? 1 : 0;
    }
    a.o = o;
    a.os0 = P.os[0]; a.os1 = P.os[1]; a.os2 = P.os[2];
    a.scale_log2 = c.sm_scale * 1.4426950408889634f;
    a.causal_br = c.is_causal == 2 ? 1 : 0;
    a.nsplit = c.nsplit;
    a.lse = c.lse;
    a.ls0 = c.ls[0]; a.ls1 = c.ls[1]; a.ls2 = c.ls[2];
    a.bmask = c.bmask;
    a.bm_nq = static_cast<int>((P.m.Lq + sage::kMaskBlockQ - 1) / sage::kMaskBlockQ);
    a.bm_nk = static_cast<int>((P.m.Lk + sage::kBK - 1) / sage::kBK);
    if (c.nsplit > 1) {
        a.part_o = static_cast<uint16_t*>(c.part);
        a.part_ml = reinterpret_cast<float2*>(static_cast<uint8_t*>(c.part) + part_ml_offset(P, c.nsplit));
        a.part_rows = P.qrows;
    }
    if (c.bmask != nullptr && c.is_causal == 0 && P.m.cu_q == nullptr) {
        // block-sparse: each XCD's tiles dealt out heaviest first; the order
        // lives in the workspace's chunk-partial section, which only the
        // prologue uses, when it fits there
        const int bq = query_rows_per_wg(P.pv);
        const int64_t nqt = (P.m.Lq + bq - 1) / bq;
        const int64_t ntile = nqt * P.Hq * P.B * c.nsplit;
        const int64_t full = ntile / 8;
        if (full >= 2 && ntile * 4 <= P.L.vpart - P.L.kpart) {
            a.tord = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(const_cast<void*>(ws)) + P.L.kpart);
            const hipError_t e = sage::launch_deal_tiles(a, bq, static_cast<int>(nqt), static_cast<int>(full), s);
            if (e != hipSuccess) return hip_fail(e, "tile order launch");
        }
    }
    const bool vec_out = vec_ok(o, P.os, P.D, 4);
    const bool pv16 = P.pv == SAGE_PV_FP16;
    hipError_t e = sage::launch_attn(a, P.L.Dp, P.dtype, c.is_causal != 0, vec_out, pv16, s);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if (c.nsplit > 1) {
        e = sage::launch_combine(a, P.L.Dp, P.dtype, vec_out, pv16, s);
        if (e != hipSuccess) return hip_fail(e, "split merge launch");
    }
    return ok();
}

AttnCall one_pass(int is_causal, float sm_scale) {
    AttnCall c;
    c.is_causal = is_causal;
    c.sm_scale = sm_scale;
    return c;
}

// Checks of the options shared by the dense and the packed split entry points.
int check_opts(const sage_attn_opts* opts) {
    if (opts == nullptr) return fail(SAGE_E_INVALID, "opts pointer is NULL");
    if (opts->is_causal < 0 || opts->is_causal > 2)
        return fail(SAGE_E_INVALID, "is_causal must be 0, 1 or 2 (got %d)", opts->is_causal);
    if (opts->nsplit < 0 || opts->nsplit > sage::kMaxSplit)
        return fail(SAGE_E_INVALID, "nsplit must be in 0..%d (got %d)", sage::kMaxSplit, opts->nsplit);
    if (opts->reserved != 0) return fail(SAGE_E_INVALID, "opts->reserved must be 0");
    if (!(std::isfinite(opts->sm_scale) && opts->sm_scale > 0.0f))
        return fail(SAGE_E_INVALID, "sm_scale must be finite and > 0 (got %g)", static_cast<double>(opts->sm_scale));
    if (reinterpret_cast<uintptr_t>(opts->lse) % 4 != 0) return fail(SAGE_E_INVALID, "lse must be 4-byte aligned");
    return SAGE_OK;
}

// Resolves the split count and checks the scratch against the other buffers;
// fills *c.
int plan_call(const Plan& P, const sage_attn_opts* opts, Extent wse, Extent oe, int64_t lse_elems, AttnCall* c) {
    c->is_causal = opts->is_causal;
    c->sm_scale = opts->sm_scale;
    c->nsplit = opts->nsplit == 0 ? auto_split(P) : opts->nsplit;
    c->lse = opts->lse;
    const Extent le{reinterpret_cast<uintptr_t>(opts->lse),
                    reinterpret_cast<uintptr_t>(opts->lse) + static_cast<uintptr_t>(opts->lse ? 4 * lse_elems : 0)};
    if (opts->lse != nullptr && (overlaps(le, wse) || overlaps(le, oe)))
        return fail(SAGE_E_INVALID, "lse overlaps o or the workspace");
    const int64_t nqt = (P.m.Lq + query_rows_per_wg(P.pv) - 1) / query_rows_per_wg(P.pv);
    if (nqt * P.Hq * static_cast<int64_t>(P.B) * c->nsplit > INT32_MAX)
        return fail(SAGE_E_UNSUPPORTED, "too many workgroups for one launch with %d key ranges", c->nsplit);
    if (c->nsplit > 1) {
        if (P.Hq > 65535 || P.B > 65535)
            return fail(SAGE_E_UNSUPPORTED, "key splits need Hq and B <= 65535");
        const int64_t need = split_bytes(P, c->nsplit);
        if (opts->part == nullptr)
            return fail(SAGE_E_WORKSPACE, "%d key ranges need %lld bytes of split scratch; part is NULL", c->nsplit,
                        static_cast<long long>(need));
        if (reinterpret_cast<uintptr_t>(opts->part) % 256 != 0)
            return fail(SAGE_E_WORKSPACE, "split scratch must be 256-byte aligned");
        if (opts->part_bytes < static_cast<size_t>(need))
            return fail(SAGE_E_WORKSPACE, "split scratch has %zu bytes, %d key ranges need %lld", opts->part_bytes,
                        c->nsplit, static_cast<long long>(need));
        const Extent pe{reinterpret_cast<uintptr_t>(opts->part),
                        reinterpret_cast<uintptr_t>(opts->part) + static_cast<uintptr_t>(need)};
        if (overlaps(pe, wse) || overlaps(pe, oe) || (opts->lse != nullptr && overlaps(pe, le)))
            return fail(SAGE_E_INVALID, "split scratch overlaps o, lse or the workspace");
        c->part = opts->part;
    }
    if (opts->block_mask != nullptr) {
        if (P.m.cu_q != nullptr)
            return fail(SAGE_E_UNSUPPORTED, "block masks are supported for dense problems only");
        const int64_t n = static_cast<int64_t>(P.B) * P.Hq * ((P.m.Lq + sage::kMaskBlockQ - 1) / sage::kMaskBlockQ) *
                          ((P.m.Lk + sage::kBK - 1) / sage::kBK);
        const Extent me{reinterpret_cast<uintptr_t>(opts->block_mask),
                        reinterpret_cast<uintptr_t>(opts->block_mask) + static_cast<uintptr_t>(n)};
        const Extent pe{reinterpret_cast<uintptr_t>(c->part),
                        reinterpret_cast<uintptr_t>(c->part) + static_cast<uintptr_t>(c->part ? split_bytes(P, c->nsplit) : 0)};
        if (overlaps(me, wse) || overlaps(me, oe) || (opts->lse != nullptr && overlaps(me, le)) ||
            (c->part != nullptr && overlaps(me, pe)))
            return fail(SAGE_E_INVALID, "block_mask overlaps o, lse, the split scratch or the workspace");
        c->bmask = opts->block_mask;
    }
    return SAGE_OK;
}

Plan dense_plan(const sage_problem* p) {
    Plan P{};
    P.B = p->B; P.Hq = p->Hq; P.Hkv = p->Hkv; P.D = p->D; P.dtype = p->dtype; P.pv = p->pv;
    for (int i = 0; i < 3; ++i) {
        P.qs[i] = p->q_stride[i];
        P.ks[i] = p->k_stride[i];
        P.vs[i] = p->v_stride[i];
        P.os[i] = p->o_stride[i];
    }
    layout_of(p, &P.L);
    P.m = dense_map(p, P.L);
    P.nkb_max = P.L.nkb;
    P.nchunk_max = P.L.nchunk;
    P.qrows = static_cast<int64_t>(P.B) * P.Hq * P.L.Lq_pad;
    P.qtiles = (p->Lq + sage::kBQ - 1) / sage::kBQ * static_cast<int64_t>(P.Hq) * P.B;
    P.nb_max = (p->Lk + sage::kBK - 1) / sage::kBK;
    return P;
}

// ---- packed variable-length problems ----

int64_t varlen_qrows(const sage_varlen_problem* p) { return static_cast<int64_t>(p->total_q) + 256LL * p->B; }
int64_t varlen_kblocks(const sage_varlen_problem* p) { return (static_cast<int64_t>(p->total_k) + 127LL * p->B) / 64 + 2; }
int64_t varlen_chunks(const sage_varlen_problem* p) { return (static_cast<int64_t>(p->total_k) + 255LL * p->B) / 256 + 1; }

void varlen_layout_of(const sage_varlen_problem* p, sage_ws_layout* L) {
    const int64_t B = p->B, Hq = p->Hq, Hkv = p->Hkv;
    std::memset(L, 0, sizeof(*L));
    L->Dp = padded_dim(p->D);
    const int64_t Dp = L->Dp;
    const int64_t R = varlen_qrows(p), NKB = varlen_kblocks(p), NCH = varlen_chunks(p);
    L->Lq_pad = static_cast<int32_t>(R);
    L->Lk_pad = static_cast<int32_t>(64 * NKB);
    L->nkb = static_cast<int32_t>(NKB);
    L->nchunk = static_cast<int32_t>(NCH);
    const int64_t vb = p->pv == SAGE_PV_FP16 ? 2 : 1;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    L->qhat = take(Hq * R * Dp);
    L->sq = take(Hq * R * 4);
    L->khat = take(Hkv * NKB * 64 * Dp);
    L->sk = take(Hkv * NKB * 4);
    L->kbar = take(B * Hkv * Dp * 4);
    L->vhat = take(Hkv * NKB * Dp * 64 * vb);
    L->vmax = take(B * Hkv * Dp * 4);
    L->kpart = take(Hkv * NCH * Dp * 8);
    L->vpart = take(Hkv * NCH * Dp * 4);
    L->total_bytes = off;
}

// Byte extent of a packed [total, H, D] view with (token, head) strides s.
Extent extent2(const void* base, const int64_t s[2], int64_t total, int64_t H, int64_t D) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(base);
    if (total <= 0) return {p, p};
    return {p, p + 2 * static_cast<uintptr_t>(s[0] * (total - 1) + s[1] * (H - 1) + D)};
}

Plan varlen_plan(const sage_varlen_problem* p, const int32_t* cu_q, const int32_t* cu_k) {
    Plan P{};
    P.B = p->B; P.Hq = p->Hq; P.Hkv = p->Hkv; P.D = p->D; P.dtype = p->dtype; P.pv = p->pv;
    // (batch, head, token): entries are found through the map, not a batch stride
    P.qs[0] = 0; P.qs[1] = p->q_stride[1]; P.qs[2] = p->q_stride[0];
    P.ks[0] = 0; P.ks[1] = p->k_stride[1]; P.ks[2] = p->k_stride[0];
    P.vs[0] = 0; P.vs[1] = p->v_stride[1]; P.vs[2] = p->v_stride[0];
    P.os[0] = 0; P.os[1] = p->o_stride[1]; P.os[2] = p->o_stride[0];
    varlen_layout_of(p, &P.L);
    sage::SeqMap& m = P.m;
    m.cu_q = cu_q;
    m.cu_k = cu_k;
    m.Lq = p->max_seqlen_q;
    m.Lk = p->max_seqlen_k;
    m.total_q = p->total_q;
    m.total_k = p->total_k;
    m.q_bstride = 0;
    m.q_hstride = P.L.Lq_pad;
    m.kb_bstride = 0;
    m.kb_hstride = P.L.nkb;
    m.c_bstride = 0;
    m.c_hstride = P.L.nchunk;
    P.nkb_max = static_cast<int>((p->max_seqlen_k + 127LL) / 128 * 2);
    P.nchunk_max = static_cast<int>((p->max_seqlen_k + 255LL) / 256);
    P.qrows = static_cast<int64_t>(P.Hq) * P.L.Lq_pad;
    // every sequence's tiles, rounded up: at most total_q / 128 + B per head
    P.qtiles = (static_cast<int64_t>(p->total_q) / sage::kBQ + p->B) * P.Hq;
    P.nb_max = static_cast<int>((p->max_seqlen_k + sage::kBK - 1LL) / sage::kBK);
    return P;
}

// ---- the allocation-free entry point ----

// Library-owned scratch of sage_attn_noalloc: the workspace sections and,
// after them, the split partials. Each GPU holds its own copy from the first
// use until the process ends. In host code the array's name is only a
// stand-in for the symbol; its device address comes from hipGetSymbolAddress,
// once per device, and only that address reaches kernels.
static __device__ __align__(256) uint8_t scratch[SAGE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up on its first use).
int scratch_address(void* stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SAGE_E_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
    if (stream != nullptr) {
        int sdev = -1;
        e = hipStreamGetDevice(as_stream(stream), &sdev);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if (sdev != dev)
            return fail(SAGE_E_INVALID, "the stream belongs to device %d but device %d is current", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
            return fail(SAGE_E_HIP, "scratch symbol address is not 256-byte aligned");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SAGE_OK;
}

}  // namespace

extern "C" {

const char* sage_status_str(int status) {
    switch (status) {
        case SAGE_OK: return "ok";
        case SAGE_E_INVALID: return "invalid argument";
        case SAGE_E_UNSUPPORTED: return "unsupported problem";
        case SAGE_E_WORKSPACE: return "bad workspace";
        case SAGE_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* sage_last_error(void) { return g_err.c_str(); }

int sage_softmax_block_keys(void) { return sage::kBK; }

int sage_softmax_spec(int pv, int* block_keys, int* reference) {
    if (pv != SAGE_PV_FP8 && pv != SAGE_PV_FP16)
        return fail(SAGE_E_INVALID, "pv %d is neither SAGE_PV_FP8 nor SAGE_PV_FP16", pv);
    if (block_keys != nullptr) *block_keys = sage::kBK;
    if (reference != nullptr) *reference = pv == SAGE_PV_FP8 ? SAGE_REF_LAZY : SAGE_REF_MAX;
    return ok();
}

int sage_problem_check(const sage_problem* p) {
    if (p == nullptr) return fail(SAGE_E_INVALID, "problem pointer is NULL");
    if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Lq < 1 || p->Lk < 1 || p->D < 1)
        return fail(SAGE_E_INVALID, "B, Hq, Hkv, Lq, Lk, D must all be >= 1 (got %d %d %d %d %d %d)",
                    p->B, p->Hq, p->Hkv, p->Lq, p->Lk, p->D);
    if (p->D > 128)
        return fail(SAGE_E_UNSUPPORTED, "head dim %d > 128 is not supported", p->D);
    if (p->Hq % p->Hkv != 0)
        return fail(SAGE_E_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
    if (p->dtype != SAGE_FP16 && p->dtype != SAGE_BF16)
        return fail(SAGE_E_INVALID, "dtype %d is neither SAGE_FP16 nor SAGE_BF16", p->dtype);
    if (p->pv != SAGE_PV_FP8 && p->pv != SAGE_PV_FP16)
        return fail(SAGE_E_INVALID, "pv %d is neither SAGE_PV_FP8 nor SAGE_PV_FP16", p->pv);
    if (p->Lq > INT32_MAX - sage::kQPad || p->Lk > INT32_MAX - sage::kQPad)
        return fail(SAGE_E_UNSUPPORTED, "sequence length too large");
    int st;
    if ((st = check_strides("q", p->q_stride)) != SAGE_OK) return st;
    if ((st = check_strides("k", p->k_stride)) != SAGE_OK) return st;
    if ((st = check_strides("v", p->v_stride)) != SAGE_OK) return st;
    if ((st = check_strides("o", p->o_stride)) != SAGE_OK) return st;
    const int64_t on[3] = {p->B, p->Hq, p->Lq};
    if (!rows_disjoint(p->o_stride, on, p->D))
        return fail(SAGE_E_INVALID, "o strides make distinct output rows overlap");
    const int64_t nqt = (p->Lq + sage::kBQ - 1) / sage::kBQ;
    if (nqt * p->Hq * static_cast<int64_t>(p->B) > INT32_MAX)
        return fail(SAGE_E_UNSUPPORTED, "too many query tiles for one launch");
    return ok();
}

int sage_problem_init(sage_problem* p, int layout, int B, int Hq, int Hkv, int Lq, int Lk, int D,
                      int dtype) {
    if (p == nullptr) return fail(SAGE_E_INVALID, "problem pointer is NULL");
    if (layout != SAGE_HND && layout != SAGE_NHD)
        return fail(SAGE_E_INVALID, "layout %d is neither SAGE_HND nor SAGE_NHD", layout);
    std::memset(p, 0, sizeof(*p));
    p->B = B;
    p->Hq = Hq;
    p->Hkv = Hkv;
    p->Lq = Lq;
    p->Lk = Lk;
    p->D = D;
    p->dtype = dtype;
    auto fill = [&](int64_t s[3], int64_t H, int64_t L) {
        if (layout == SAGE_HND) {
            s[0] = H * L * D;
            s[1] = L * D;
            s[2] = D;
        } else {
            s[0] = L * H * D;
            s[1] = D;
            s[2] = H * D;
        }
    };
    fill(p->q_stride, Hq, Lq);
    fill(p->k_stride, Hkv, Lk);
    fill(p->v_stride, Hkv, Lk);
    fill(p->o_stride, Hq, Lq);
    return sage_problem_check(p);
}

size_t sage_workspace_bytes(const sage_problem* p) {
    if (sage_problem_check(p) != SAGE_OK) return 0;
    sage_ws_layout L;
    layout_of(p, &L);
    return static_cast<size_t>(L.total_bytes);
}

int sage_workspace_layout(const sage_problem* p, sage_ws_layout* out) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (out == nullptr) return fail(SAGE_E_INVALID, "layout pointer is NULL");
    layout_of(p, out);
    return ok();
}

int sage_quantize(const sage_problem* p, const void* q, const void* k, const void* v,
                  int smooth_k, void* ws, size_t ws_bytes, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (q == nullptr || k == nullptr || v == nullptr)
        return fail(SAGE_E_INVALID, "q, k and v must be non-NULL device pointers");
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    const Extent wse{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(L.total_bytes)};
    if (overlaps(wse, extent_of(q, p->q_stride, p->B, p->Hq, p->Lq, p->D)) ||
        overlaps(wse, extent_of(k, p->k_stride, p->B, p->Hkv, p->Lk, p->D)) ||
        overlaps(wse, extent_of(v, p->v_stride, p->B, p->Hkv, p->Lk, p->D)))
        return fail(SAGE_E_INVALID, "the workspace overlaps q, k or v");

    return launch_quantize(dense_plan(p), q, k, v, smooth_k, ws, as_stream(stream));
}

int sage_attn_quantized(const sage_problem* p, const void* ws, size_t ws_bytes, void* o,
                        int is_causal, float sm_scale, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (o == nullptr) return fail(SAGE_E_INVALID, "o must be a non-NULL device pointer");
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SAGE_E_INVALID, "sm_scale must be finite and > 0 (got %g)", static_cast<double>(sm_scale));
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    const Extent wse{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(L.total_bytes)};
    if (overlaps(wse, extent_of(o, p->o_stride, p->B, p->Hq, p->Lq, p->D)))
        return fail(SAGE_E_INVALID, "o overlaps the workspace");
    if (is_causal < 0 || is_causal > 2)
        return fail(SAGE_E_INVALID, "is_causal must be 0, 1 or 2 (got %d)", is_causal);
    return launch_attention(dense_plan(p), ws, o, one_pass(is_causal, sm_scale), as_stream(stream));
}

int sage_split_count(const sage_problem* p) {
    if (sage_problem_check(p) != SAGE_OK) return 0;
    return auto_split(dense_plan(p));
}

size_t sage_split_bytes(const sage_problem* p, int nsplit) {
    if (sage_problem_check(p) != SAGE_OK || nsplit < 0 || nsplit > sage::kMaxSplit) return 0;
    const Plan P = dense_plan(p);
    return static_cast<size_t>(split_bytes(P, nsplit == 0 ? auto_split(P) : nsplit));
}

int sage_attn_quantized_ex(const sage_problem* p, const void* ws, size_t ws_bytes, void* o,
                           const sage_attn_opts* opts, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (o == nullptr) return fail(SAGE_E_INVALID, "o must be a non-NULL device pointer");
    if ((st = check_opts(opts)) != SAGE_OK) return st;
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    const Extent wse{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(L.total_bytes)};
    const Extent oe = extent_of(o, p->o_stride, p->B, p->Hq, p->Lq, p->D);
    if (overlaps(wse, oe)) return fail(SAGE_E_INVALID, "o overlaps the workspace");
    const Plan P = dense_plan(p);
    AttnCall c;
    if ((st = plan_call(P, opts, wse, oe, static_cast<int64_t>(p->B) * p->Hq * p->Lq, &c)) != SAGE_OK) return st;
    c.ls[0] = static_cast<int64_t>(p->Hq) * p->Lq;
    c.ls[1] = p->Lq;
    c.ls[2] = 1;
    return launch_attention(P, ws, o, c, as_stream(stream));
}

int sage_attn(const sage_problem* p, const void* q, const void* k, const void* v, void* o,
              int is_causal, float sm_scale, int smooth_k, void* ws, size_t ws_bytes,
              void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (o == nullptr || q == nullptr || k == nullptr || v == nullptr)
        return fail(SAGE_E_INVALID, "q, k, v and o must be non-NULL device pointers");
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SAGE_E_INVALID, "sm_scale must be finite and > 0 (got %g)", static_cast<double>(sm_scale));
    if (is_causal < 0 || is_causal > 2)
        return fail(SAGE_E_INVALID, "is_causal must be 0, 1 or 2 (got %d)", is_causal);
    const Extent oe = extent_of(o, p->o_stride, p->B, p->Hq, p->Lq, p->D);
    if (overlaps(oe, extent_of(q, p->q_stride, p->B, p->Hq, p->Lq, p->D)) ||
        overlaps(oe, extent_of(k, p->k_stride, p->B, p->Hkv, p->Lk, p->D)) ||
        overlaps(oe, extent_of(v, p->v_stride, p->B, p->Hkv, p->Lk, p->D)))
        return fail(SAGE_E_INVALID, "o overlaps q, k or v");
    sage_attn_opts opts{};
    opts.is_causal = is_causal;
    opts.nsplit = 1;
    opts.sm_scale = sm_scale;
    return sage_attn_ex(p, q, k, v, o, smooth_k, ws, ws_bytes, &opts, stream);
}

int sage_attn_ex(const sage_problem* p, const void* q, const void* k, const void* v, void* o, int smooth_k,
                 void* ws, size_t ws_bytes, const sage_attn_opts* opts, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (o == nullptr || q == nullptr || k == nullptr || v == nullptr)
        return fail(SAGE_E_INVALID, "q, k, v and o must be non-NULL device pointers");
    if ((st = check_opts(opts)) != SAGE_OK) return st;
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    const Extent wse{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(L.total_bytes)};
    const Extent oe = extent_of(o, p->o_stride, p->B, p->Hq, p->Lq, p->D);
    const Extent in[3] = {extent_of(q, p->q_stride, p->B, p->Hq, p->Lq, p->D),
                          extent_of(k, p->k_stride, p->B, p->Hkv, p->Lk, p->D),
                          extent_of(v, p->v_stride, p->B, p->Hkv, p->Lk, p->D)};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(wse, in[i])) return fail(SAGE_E_INVALID, "the workspace overlaps q, k or v");
        if (overlaps(oe, in[i])) return fail(SAGE_E_INVALID, "o overlaps q, k or v");
    }
    if (overlaps(wse, oe)) return fail(SAGE_E_INVALID, "o overlaps the workspace");
    const Plan P = dense_plan(p);
    AttnCall c;
    if ((st = plan_call(P, opts, wse, oe, static_cast<int64_t>(p->B) * p->Hq * p->Lq, &c)) != SAGE_OK) return st;
    const Extent le{reinterpret_cast<uintptr_t>(c.lse),
                    reinterpret_cast<uintptr_t>(c.lse) + static_cast<uintptr_t>(c.lse ? 4LL * p->B * p->Hq * p->Lq : 0)};
    const Extent pe{reinterpret_cast<uintptr_t>(c.part),
                    reinterpret_cast<uintptr_t>(c.part) + static_cast<uintptr_t>(c.part ? split_bytes(P, c.nsplit) : 0)};
    for (int i = 0; i < 3; ++i)
        if ((c.lse != nullptr && overlaps(le, in[i])) || (c.part != nullptr && overlaps(pe, in[i])))
            return fail(SAGE_E_INVALID, "lse or the split scratch overlaps q, k or v");
    c.ls[0] = static_cast<int64_t>(p->Hq) * p->Lq;
    c.ls[1] = p->Lq;
    c.ls[2] = 1;
    const hipStream_t s = as_stream(stream);
    const bool fused = fuse_q(P, c.nsplit);
    if ((st = launch_quantize(P, q, k, v, smooth_k, ws, s, !fused)) != SAGE_OK) return st;
    return launch_attention(P, ws, o, c, s, fused ? q : nullptr);
}

size_t sage_noalloc_bytes(const sage_problem* p, int nsplit) {
    if (sage_problem_check(p) != SAGE_OK || nsplit < 0 || nsplit > sage::kMaxSplit) return 0;
    const Plan P = dense_plan(p);
    return static_cast<size_t>(round_up(P.L.total_bytes, 256) + split_bytes(P, nsplit == 0 ? auto_split(P) : nsplit));
}

int sage_attn_noalloc(const sage_problem* p, const void* q, const void* k, const void* v, void* o, int smooth_k,
                      const sage_attn_opts* opts, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (o == nullptr || q == nullptr || k == nullptr || v == nullptr)
        return fail(SAGE_E_INVALID, "q, k, v and o must be non-NULL device pointers");
    if ((st = check_opts(opts)) != SAGE_OK) return st;
    if (opts->part != nullptr || opts->part_bytes != 0)
        return fail(SAGE_E_INVALID, "opts->part must be NULL and part_bytes 0: the split partials use the library's scratch");
    const Plan P = dense_plan(p);
    const int nsplit = opts->nsplit == 0 ? auto_split(P) : opts->nsplit;
    const int64_t ws_bytes = round_up(P.L.total_bytes, 256);
    const int64_t need = ws_bytes + split_bytes(P, nsplit);
    if (need > static_cast<int64_t>(SAGE_NOALLOC_SCRATCH_BYTES))
        return fail(SAGE_E_WORKSPACE, "the problem needs %lld bytes of scratch (workspace %lld + split partials %lld), "
                    "more than the %lld bytes sage_attn_noalloc holds", static_cast<long long>(need),
                    static_cast<long long>(P.L.total_bytes), static_cast<long long>(need - ws_bytes),
                    static_cast<long long>(SAGE_NOALLOC_SCRATCH_BYTES));
    void* base = nullptr;
    if ((st = scratch_address(stream, &base)) != SAGE_OK) return st;
    sage_attn_opts o2 = *opts;
    o2.nsplit = nsplit;
    o2.part = nsplit > 1 ? static_cast<uint8_t*>(base) + ws_bytes : nullptr;
    o2.part_bytes = static_cast<size_t>(need - ws_bytes);
    return sage_attn_ex(p, q, k, v, o, smooth_k, base, static_cast<size_t>(ws_bytes), &o2, stream);
}

int sage_quantize_kv(const sage_problem* p, const void* k, const void* v, int smooth_k, void* ws, size_t ws_bytes,
                     void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (k == nullptr || v == nullptr) return fail(SAGE_E_INVALID, "k and v must be non-NULL device pointers");
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    const Extent wse{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(L.total_bytes)};
    if (overlaps(wse, extent_of(k, p->k_stride, p->B, p->Hkv, p->Lk, p->D)) ||
        overlaps(wse, extent_of(v, p->v_stride, p->B, p->Hkv, p->Lk, p->D)))
        return fail(SAGE_E_INVALID, "the workspace overlaps k or v");
    return launch_quantize(dense_plan(p), nullptr, k, v, smooth_k, ws, as_stream(stream), false);
}

int sage_attn_q_ex(const sage_problem* p, const void* q, const void* ws, size_t ws_bytes, void* o,
                   const sage_attn_opts* opts, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (o == nullptr || q == nullptr) return fail(SAGE_E_INVALID, "q and o must be non-NULL device pointers");
    if ((st = check_opts(opts)) != SAGE_OK) return st;
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    const Extent wse{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(L.total_bytes)};
    const Extent oe = extent_of(o, p->o_stride, p->B, p->Hq, p->Lq, p->D);
    const Extent qe = extent_of(q, p->q_stride, p->B, p->Hq, p->Lq, p->D);
    if (overlaps(wse, oe)) return fail(SAGE_E_INVALID, "o overlaps the workspace");
    if (overlaps(oe, qe)) return fail(SAGE_E_INVALID, "o overlaps q");
    const Plan P = dense_plan(p);
    AttnCall c;
    if ((st = plan_call(P, opts, wse, oe, static_cast<int64_t>(p->B) * p->Hq * p->Lq, &c)) != SAGE_OK) return st;
    const Extent le{reinterpret_cast<uintptr_t>(c.lse),
                    reinterpret_cast<uintptr_t>(c.lse) + static_cast<uintptr_t>(c.lse ? 4LL * p->B * p->Hq * p->Lq : 0)};
    const Extent pe{reinterpret_cast<uintptr_t>(c.part),
                    reinterpret_cast<uintptr_t>(c.part) + static_cast<uintptr_t>(c.part ? split_bytes(P, c.nsplit) : 0)};
    if ((c.lse != nullptr && overlaps(le, qe)) || (c.part != nullptr && overlaps(pe, qe)))
        return fail(SAGE_E_INVALID, "lse or the split scratch overlaps q");
    c.ls[0] = static_cast<int64_t>(p->Hq) * p->Lq;
    c.ls[1] = p->Lq;
    c.ls[2] = 1;
    return launch_attention(P, ws, o, c, as_stream(stream), q);
}

int sage_debug_qk_int32(const sage_problem* p, const void* ws, size_t ws_bytes, int b, int hq,
                        int32_t* out, void* stream) {
    int st = sage_problem_check(p);
    if (st != SAGE_OK) return st;
    if (b < 0 || b >= p->B || hq < 0 || hq >= p->Hq)
        return fail(SAGE_E_INVALID, "head (%d, %d) out of range", b, hq);
    if (out == nullptr) return fail(SAGE_E_INVALID, "out must be a non-NULL device pointer");
    sage_ws_layout L;
    if ((st = check_ws(p, ws, ws_bytes, &L)) != SAGE_OK) return st;
    sage::AttnArgs a;
    fill_attn_args(dense_plan(p), ws, &a);
    a.dump = out;
    a.dump_ld = L.Lk_pad;
    a.dump_b = b;
    a.dump_hq = hq;
    hipError_t e = sage::launch_attn_dump(a, L.Dp, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "debug launch");
    return ok();
}

int sage_varlen_problem_check(const sage_varlen_problem* p) {
    if (p == nullptr) return fail(SAGE_E_INVALID, "problem pointer is NULL");
    if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->D < 1)
        return fail(SAGE_E_INVALID, "B, Hq, Hkv, D must all be >= 1 (got %d %d %d %d)", p->B, p->Hq, p->Hkv, p->D);
    if (p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 1 || p->max_seqlen_k < 1)
        return fail(SAGE_E_INVALID, "totals must be >= 0 and max_seqlen >= 1 (got %d %d %d %d)", p->total_q,
                    p->total_k, p->max_seqlen_q, p->max_seqlen_k);
    if (p->D > 128) return fail(SAGE_E_UNSUPPORTED, "head dim %d > 128 is not supported", p->D);
    if (p->Hq % p->Hkv != 0)
        return fail(SAGE_E_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
    if (p->dtype != SAGE_FP16 && p->dtype != SAGE_BF16)
        return fail(SAGE_E_INVALID, "dtype %d is neither SAGE_FP16 nor SAGE_BF16", p->dtype);
    if (p->pv != SAGE_PV_FP8 && p->pv != SAGE_PV_FP16)
        return fail(SAGE_E_INVALID, "pv %d is neither SAGE_PV_FP8 nor SAGE_PV_FP16", p->pv);
    if (p->B > 65535 || p->Hkv > 65535)
        return fail(SAGE_E_UNSUPPORTED, "more than 65535 sequences or kv heads");
    const int64_t big = INT32_MAX / 2;
    if (varlen_qrows(p) * p->Hq > big || varlen_kblocks(p) * 64 * p->Hkv > big ||
        p->max_seqlen_q > INT32_MAX - 512 || p->max_seqlen_k > INT32_MAX - 512)
        return fail(SAGE_E_UNSUPPORTED, "packed problem too large");
    const int64_t nqt = (p->max_seqlen_q + sage::kBQ - 1) / sage::kBQ;
    if (nqt * p->Hq * static_cast<int64_t>(p->B) > INT32_MAX ||
        (p->max_seqlen_q + 255LL) / 64 * p->Hq * p->B + (p->max_seqlen_k + 255LL) / 256 * p->Hkv * p->B > INT32_MAX)
        return fail(SAGE_E_UNSUPPORTED, "too many workgroups for one launch");
    const int64_t* ss[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
    const char* nm[4] = {"q", "k", "v", "o"};
    for (int t = 0; t < 4; ++t)
        for (int i = 0; i < 2; ++i)
            if (ss[t][i] < 0)
                return fail(SAGE_E_UNSUPPORTED, "%s stride[%d] = %lld is negative", nm[t], i,
                            static_cast<long long>(ss[t][i]));
    const int64_t os3[3] = {0, p->o_stride[1], p->o_stride[0]};
    const int64_t on[3] = {1, p->Hq, p->total_q};
    if (!rows_disjoint(os3, on, p->D))
        return fail(SAGE_E_INVALID, "o strides make distinct output rows overlap");
    return ok();
}

int sage_varlen_problem_init(sage_varlen_problem* p, int B, int Hq, int Hkv, int total_q, int total_k,
                             int max_seqlen_q, int max_seqlen_k, int D, int dtype, int pv) {
    if (p == nullptr) return fail(SAGE_E_INVALID, "problem pointer is NULL");
    std::memset(p, 0, sizeof(*p));
    p->B = B; p->Hq = Hq; p->Hkv = Hkv; p->D = D; p->dtype = dtype; p->pv = pv;
    p->total_q = total_q; p->total_k = total_k;
    p->max_seqlen_q = max_seqlen_q; p->max_seqlen_k = max_seqlen_k;
    p->q_stride[0] = static_cast<int64_t>(Hq) * D; p->q_stride[1] = D;
    p->k_stride[0] = static_cast<int64_t>(Hkv) * D; p->k_stride[1] = D;
    p->v_stride[0] = static_cast<int64_t>(Hkv) * D; p->v_stride[1] = D;
    p->o_stride[0] = static_cast<int64_t>(Hq) * D; p->o_stride[1] = D;
    return sage_varlen_problem_check(p);
}

size_t sage_varlen_workspace_bytes(const sage_varlen_problem* p) {
    if (sage_varlen_problem_check(p) != SAGE_OK) return 0;
    sage_ws_layout L;
    varlen_layout_of(p, &L);
    return static_cast<size_t>(L.total_bytes);
}

int sage_varlen_workspace_layout(const sage_varlen_problem* p, sage_ws_layout* out) {
    int st = sage_varlen_problem_check(p);
    if (st != SAGE_OK) return st;
    if (out == nullptr) return fail(SAGE_E_INVALID, "layout pointer is NULL");
    varlen_layout_of(p, out);
    return ok();
}

// Argument checks shared by the packed entry points; fills *P and the
// extents of the workspace, o and the inputs (q, k, v).
static int varlen_prepare(const sage_varlen_problem* p, const void* q, const void* k, const void* v, void* o,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* ws, size_t ws_bytes,
                          Plan* P, Extent* wse, Extent* oe, Extent (&in)[3]) {
    int st = sage_varlen_problem_check(p);
    if (st != SAGE_OK) return st;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(SAGE_E_INVALID, "q, k, v and o must be non-NULL device pointers");
    if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)
        return fail(SAGE_E_INVALID, "cu_seqlens_q and cu_seqlens_k must be non-NULL device pointers");
    *P = varlen_plan(p, cu_seqlens_q, cu_seqlens_k);
    if (ws == nullptr) return fail(SAGE_E_WORKSPACE, "workspace pointer is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return fail(SAGE_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < static_cast<size_t>(P->L.total_bytes))
        return fail(SAGE_E_WORKSPACE, "workspace has %zu bytes, needs %lld", ws_bytes,
                    static_cast<long long>(P->L.total_bytes));
    *wse = Extent{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + static_cast<uintptr_t>(P->L.total_bytes)};
    const Extent qe = extent2(q, p->q_stride, p->total_q, p->Hq, p->D);
    const Extent ke = extent2(k, p->k_stride, p->total_k, p->Hkv, p->D);
    const Extent ve = extent2(v, p->v_stride, p->total_k, p->Hkv, p->D);
    in[0] = qe;
    in[1] = ke;
    in[2] = ve;
    *oe = extent2(o, p->o_stride, p->total_q, p->Hq, p->D);
    if (overlaps(*wse, qe) || overlaps(*wse, ke) || overlaps(*wse, ve))
        return fail(SAGE_E_INVALID, "the workspace overlaps q, k or v");
    if (overlaps(*oe, qe) || overlaps(*oe, ke) || overlaps(*oe, ve) || overlaps(*oe, *wse))
        return fail(SAGE_E_INVALID, "o overlaps q, k, v or the workspace");
    return SAGE_OK;
}

int sage_varlen_attn(const sage_varlen_problem* p, const void* q, const void* k, const void* v, void* o,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int is_causal, float sm_scale,
                     int smooth_k, void* ws, size_t ws_bytes, void* stream) {
    Plan P;
    Extent wse, oe, in[3];
    int st = varlen_prepare(p, q, k, v, o, cu_seqlens_q, cu_seqlens_k, ws, ws_bytes, &P, &wse, &oe, in);
    if (st != SAGE_OK) return st;
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SAGE_E_INVALID, "sm_scale must be finite and > 0 (got %g)", static_cast<double>(sm_scale));
    if (is_causal < 0 || is_causal > 2)
        return fail(SAGE_E_INVALID, "is_causal must be 0, 1 or 2 (got %d)", is_causal);
    const hipStream_t s = as_stream(stream);
    const bool fused = fuse_q(P, 1);
    if ((st = launch_quantize(P, q, k, v, smooth_k, ws, s, !fused)) != SAGE_OK) return st;
    return launch_attention(P, ws, o, one_pass(is_causal, sm_scale), s, fused ? q : nullptr);
}

int sage_varlen_split_count(const sage_varlen_problem* p) {
    if (sage_varlen_problem_check(p) != SAGE_OK) return 0;
    return auto_split(varlen_plan(p, nullptr, nullptr));
}

size_t sage_varlen_split_bytes(const sage_varlen_problem* p, int nsplit) {
    if (sage_varlen_problem_check(p) != SAGE_OK || nsplit < 0 || nsplit > sage::kMaxSplit) return 0;
    const Plan P = varlen_plan(p, nullptr, nullptr);
    return static_cast<size_t>(split_bytes(P, nsplit == 0 ? auto_split(P) : nsplit));
}

int sage_varlen_attn_ex(const sage_varlen_problem* p, const void* q, const void* k, const void* v, void* o,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int smooth_k, void* ws,
                        size_t ws_bytes, const sage_attn_opts* opts, void* stream) {
    Plan P;
    Extent wse, oe, in[3];
    int st = varlen_prepare(p, q, k, v, o, cu_seqlens_q, cu_seqlens_k, ws, ws_bytes, &P, &wse, &oe, in);
    if (st != SAGE_OK) return st;
    if ((st = check_opts(opts)) != SAGE_OK) return st;
    AttnCall c;
    if ((st = plan_call(P, opts, wse, oe, static_cast<int64_t>(p->Hq) * p->total_q, &c)) != SAGE_OK) return st;
    const Extent le{reinterpret_cast<uintptr_t>(c.lse),
                    reinterpret_cast<uintptr_t>(c.lse) + static_cast<uintptr_t>(c.lse ? 4LL * p->Hq * p->total_q : 0)};
    const Extent pe{reinterpret_cast<uintptr_t>(c.part),
                    reinterpret_cast<uintptr_t>(c.part) + static_cast<uintptr_t>(c.part ? split_bytes(P, c.nsplit) : 0)};
    for (int i = 0; i < 3; ++i)
        if ((c.lse != nullptr && overlaps(le, in[i])) || (c.part != nullptr && overlaps(pe, in[i])))
            return fail(SAGE_E_INVALID, "lse or the split scratch overlaps q, k or v");
    c.ls[0] = 0;
    c.ls[1] = p->total_q;
    c.ls[2] = 1;
    const hipStream_t s = as_stream(stream);
    const bool fused = fuse_q(P, c.nsplit);
    if ((st = launch_quantize(P, q, k, v, smooth_k, ws, s, !fused)) != SAGE_OK) return st;
    return launch_attention(P, ws, o, c, s, fused ? q : nullptr);
}

}  // extern "C"
