"""CPU oracle for SageAttention2-style quantized attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library. It shares no code
with the HIP path; the C source ``sage_oracle.c`` documents every step and the
passage of the pages it follows.

All tensors here are numpy arrays in the logical (batch, head, token, channel)
order ("HND"). Inputs are float32 arrays holding fp16/bf16 values exactly.
Heads are processed independently; a thread pool runs (batch, head, row-range)
work items in parallel (ctypes releases the GIL during each C call).
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

KBLOCK = 64          # tokens per K quantization block (per-block INT8 scale)
KMEAN_CHUNK = 256    # fixed summation chunk of the fp64 key mean
PSCALE = 256.0       # static power-of-two scale applied to P before FP8
PREF = {"max": 0, "pow2": 1, "lazy": 2}   # reference P is quantized against (see softmax_reference in the C source)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    f64 = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = f64
    lib.oracle_e4m3_encode.argtypes = [f64]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_padded_dim.argtypes = [i32]
    lib.oracle_padded_dim.restype = i32
    lib.oracle_k_mean.argtypes = [P, i32, i32, i32, P]
    lib.oracle_quant_q.argtypes = [P, i32, i32, i32, P, P]
    lib.oracle_quant_k.argtypes = [P, P, i32, i32, i32, P, P]
    lib.oracle_quant_v.argtypes = [P, i32, i32, i32, P, P]
    lib.oracle_qk_int32.argtypes = [P, i32, P, i32, i32, P]
    lib.oracle_attn_quantized.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, f64, i32,
                                          i32, i32, i32, i32, P]
    lib.oracle_attn_exact.argtypes = [P, P, P, i32, i32, i32, f64, i32, P, i32, i32, i32, i32, i32, P]
    lib.oracle_round_f16.argtypes = [f64]
    lib.oracle_round_f16.restype = f64
    lib.oracle_round_bf16.argtypes = [f64]
    lib.oracle_round_bf16.restype = f64
    lib.oracle_attn_quantized_pv16.argtypes = [P, P, i32, P, P, P, i32, i32, i32, f64, i32,
                                               i32, i32, i32, i32, P]
    lib.oracle_attn_general.argtypes = [P, P, i32, P, P, P, P, P, i32, i32, i32, f64, i32, i32,
                                        i32, i32, i32, P, i32, i32, i32, i32, i32, P, P]
    for name in ("oracle_k_mean", "oracle_quant_q", "oracle_quant_k", "oracle_quant_v",
                 "oracle_qk_int32", "oracle_attn_quantized", "oracle_attn_exact",
                 "oracle_attn_quantized_pv16", "oracle_attn_general"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _workers(n_items, threads):
    if threads is None:
        threads = os.cpu_count() or 1
    return max(1, min(threads, n_items))


# --------------------------------------------------------------------------
# FP8 E4M3FN codec
# --------------------------------------------------------------------------
def e4m3_decode(codes):
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_decode(int(c)) for c in codes.ravel()],
                    dtype=np.float64).reshape(codes.shape)


def e4m3_encode(values):
    lib = _load()
    values = np.asarray(values, dtype=np.float64)
    return np.array([lib.oracle_e4m3_encode(float(x)) for x in values.ravel()],
                    dtype=np.uint8).reshape(values.shape)


def round_f16(values):
    """Round fp64 values to IEEE binary16 (nearest, ties to even); returns fp64."""
    lib = _load()
    values = np.asarray(values, dtype=np.float64)
    return np.array([lib.oracle_round_f16(float(x)) for x in values.ravel()],
                    dtype=np.float64).reshape(values.shape)


def round_bf16(values):
    """Round fp64 values to bfloat16 (nearest, ties to even); returns fp64."""
    lib = _load()
    values = np.asarray(values, dtype=np.float64)
    return np.array([lib.oracle_round_bf16(float(x)) for x in values.ravel()],
                    dtype=np.float64).reshape(values.shape)


def padded_dim(d):
    return int(_load().oracle_padded_dim(int(d)))


# --------------------------------------------------------------------------
# Quantization prologue
# --------------------------------------------------------------------------
def quantize(q, k, v, smooth_k=True, threads=None):
    """Quantize logical-HND float32 inputs.

    q: [B, Hq, Lq, D]; k, v: [B, Hkv, Lk, D]. Returns a dict of numpy arrays:
    kbar [B,Hkv,Dp] f32, qhat [B,Hq,Lq,Dp] i8, sq [B,Hq,Lq] f32,
    khat [B,Hkv,Lk,Dp] i8, sk [B,Hkv,ceil(Lk/64)] f32,
    vhat [B,Hkv,Lk,Dp] u8 (token major, unpermuted), sv [B,Hkv,Dp] f32.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    Dp = padded_dim(D)
    nkb = (Lk + KBLOCK - 1) // KBLOCK
    out = dict(
        kbar=np.zeros((B, Hkv, Dp), np.float32),
        qhat=np.zeros((B, Hq, Lq, Dp), np.int8),
        sq=np.zeros((B, Hq, Lq), np.float32),
        khat=np.zeros((B, Hkv, Lk, Dp), np.int8),
        sk=np.zeros((B, Hkv, nkb), np.float32),
        vhat=np.zeros((B, Hkv, Lk, Dp), np.uint8),
        sv=np.zeros((B, Hkv, Dp), np.float32),
    )

    def kv_job(bh):
        b, h = bh
        kb = np.ascontiguousarray(k[b, h])
        vb = np.ascontiguousarray(v[b, h])
        kbar = out["kbar"][b, h]
        if smooth_k:
            lib.oracle_k_mean(_ptr(kb), Lk, D, Dp, _ptr(kbar))
        lib.oracle_quant_k(_ptr(kb), _ptr(kbar), Lk, D, Dp, _ptr(out["khat"][b, h]),
                           _ptr(out["sk"][b, h]))
        lib.oracle_quant_v(_ptr(vb), Lk, D, Dp, _ptr(out["vhat"][b, h]), _ptr(out["sv"][b, h]))

    def q_job(bh):
        b, h = bh
        qb = np.ascontiguousarray(q[b, h])
        lib.oracle_quant_q(_ptr(qb), Lq, D, Dp, _ptr(out["qhat"][b, h]), _ptr(out["sq"][b, h]))

    jobs_kv = [(b, h) for b in range(B) for h in range(Hkv)]
    jobs_q = [(b, h) for b in range(B) for h in range(Hq)]
    with ThreadPoolExecutor(_workers(len(jobs_kv) + len(jobs_q), threads)) as ex:
        list(ex.map(kv_job, jobs_kv))
        list(ex.map(q_job, jobs_q))
    out["D"] = D
    out["Dp"] = Dp
    return out


def qk_int32(qhat_bh, khat_bh):
    """Exact int32 logits of one head: qhat [Lq,Dp] i8, khat [Lk,Dp] i8 -> [Lq,Lk]."""
    lib = _load()
    qhat_bh = np.ascontiguousarray(qhat_bh, dtype=np.int8)
    khat_bh = np.ascontiguousarray(khat_bh, dtype=np.int8)
    Lq, Dp = qhat_bh.shape
    Lk = khat_bh.shape[0]
    out = np.zeros((Lq, Lk), np.int32)
    lib.oracle_qk_int32(_ptr(qhat_bh), Lq, _ptr(khat_bh), Lk, Dp, _ptr(out))
    return out


def _row_jobs(B, Hq, Lq, heads, rows, chunk):
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    if rows is None:
        rows = (0, Lq)
    r0, r1 = rows
    jobs = []
    for (b, h) in heads:
        for s in range(r0, r1, chunk):
            jobs.append((b, h, s, min(s + chunk, r1)))
    return heads, (r0, r1), jobs


def attn_quantized(qz, sm_scale, causal=False, bk=128, heads=None, rows=None,
                   threads=None, chunk=64, pref="max"):
    """Quantized attention from a ``quantize`` result, fp64 output.

    heads: list of (b, hq) to compute (default all); rows: (r0, r1) query range.
    bk: keys per online-softmax block; pref: the reference P is quantized
    against, "max" (the running maximum), "pow2" (power-of-two steps) or
    "lazy" (the maximum plus two factors of two, moved only when a block passes
    it by more than 0.75 of a factor of two).
    Returns an array [len(heads), r1-r0, D] float64 in the order of ``heads``.
    """
    lib = _load()
    B, Hq, Lq, Dp = qz["qhat"].shape
    Hkv = qz["khat"].shape[1]
    Lk = qz["khat"].shape[2]
    D = qz["D"]
    G = Hq // Hkv
    heads, (r0, r1), jobs = _row_jobs(B, Hq, Lq, heads, rows, chunk)
    out = np.zeros((len(heads), r1 - r0, D), np.float64)
    index = {hd: n for n, hd in enumerate(heads)}

    def job(j):
        b, h, s0, s1 = j
        hk = h // G
        dst = np.zeros((s1 - s0, D), np.float64)
        lib.oracle_attn_quantized(_ptr(qz["qhat"][b, h]), _ptr(qz["sq"][b, h]), Lq,
                                  _ptr(qz["khat"][b, hk]), _ptr(qz["sk"][b, hk]),
                                  _ptr(qz["vhat"][b, hk]), _ptr(qz["sv"][b, hk]), Lk,
                                  D, Dp, float(sm_scale), int(bool(causal)), int(bk), PREF[pref],
                                  s0, s1, _ptr(dst))
        out[index[(b, h)], s0 - r0:s1 - r0] = dst

    with ThreadPoolExecutor(_workers(len(jobs), threads)) as ex:
        list(ex.map(job, jobs))
    return out


def attn_quantized_pv16(qz, v, sm_scale, causal=False, fmt="fp16", bk=128, heads=None,
                        rows=None, threads=None, chunk=64):
    """INT8-QK / 16-bit-PV quantized attention (the "8+16" variant), fp64 output.

    qz: a ``quantize`` result (its Q/K codes and scales are used; its FP8 V is
    not); v: the logical-HND float32 V holding the 16-bit input values;
    fmt: "fp16" or "bf16", the format P is rounded to (the inputs' format).
    Returns [len(heads), r1-r0, D] float64 like ``attn_quantized``.
    """
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, Hq, Lq, Dp = qz["qhat"].shape
    Hkv = qz["khat"].shape[1]
    Lk = qz["khat"].shape[2]
    D = qz["D"]
    G = Hq // Hkv
    f = {"fp16": 0, "bf16": 1}[fmt]
    heads, (r0, r1), jobs = _row_jobs(B, Hq, Lq, heads, rows, chunk)
    out = np.zeros((len(heads), r1 - r0, D), np.float64)
    index = {hd: n for n, hd in enumerate(heads)}

    def job(j):
        b, h, s0, s1 = j
        hk = h // G
        dst = np.zeros((s1 - s0, D), np.float64)
        lib.oracle_attn_quantized_pv16(_ptr(qz["qhat"][b, h]), _ptr(qz["sq"][b, h]), Lq,
                                       _ptr(qz["khat"][b, hk]), _ptr(qz["sk"][b, hk]),
                                       _ptr(v[b, hk]), Lk, D, Dp, float(sm_scale),
                                       int(bool(causal)), int(bk), f, s0, s1, _ptr(dst))
        out[index[(b, h)], s0 - r0:s1 - r0] = dst

    with ThreadPoolExecutor(_workers(len(jobs), threads)) as ex:
        list(ex.map(job, jobs))
    return out


def _mask_args(block_mask, b, h, mask_block):
    """(pointer, mbq, mbk, row stride) of head (b, h) of a [B, Hq, nqb, nkb] block mask."""
    if block_mask is None:
        return None, 1, 1, 1
    m = block_mask[b, h]
    assert m.dtype == np.uint8 and m.flags["C_CONTIGUOUS"]
    return _ptr(m), int(mask_block[0]), int(mask_block[1]), m.shape[1]


def attn_general(qz, sm_scale, v=None, pv="fp8", fmt="fp16", causal=0, nsplit=1, bk=128,
                 heads=None, rows=None, threads=None, chunk=64, block_mask=None, mask_block=(128, 128),
                 pref="max"):
    """Quantized attention with key-range splits, causal alignment, block masks and the LSE.

    pv: "fp8" (uses qz's FP8 V) or "fp16" (uses v, P rounded to ``fmt``);
    causal: 0 none, 1 top-left, 2 bottom-right; nsplit: key ranges (see the C
    source); block_mask: None or uint8 [B, Hq, ceil(Lq/mbq), ceil(Lk/mbk)],
    nonzero = the block of mask_block = (mbq queries, mbk keys) is computed;
    pref: "max", "pow2" or "lazy", the reference P is quantized against (FP8 P).
    Returns (out [len(heads), r1-r0, D], lse [len(heads), r1-r0]) fp64.
    """
    lib = _load()
    B, Hq, Lq, Dp = qz["qhat"].shape
    Hkv = qz["khat"].shape[1]
    Lk = qz["khat"].shape[2]
    D = qz["D"]
    G = Hq // Hkv
    f = -1 if pv == "fp8" else {"fp16": 0, "bf16": 1}[fmt]
    if f >= 0:
        v = np.ascontiguousarray(v, dtype=np.float32)
    if block_mask is not None:
        block_mask = np.ascontiguousarray(block_mask, dtype=np.uint8)
        assert block_mask.shape == (B, Hq, -(-Lq // mask_block[0]), -(-Lk // mask_block[1])), block_mask.shape
    causal = int(causal)
    heads, (r0, r1), jobs = _row_jobs(B, Hq, Lq, heads, rows, chunk)
    out = np.zeros((len(heads), r1 - r0, D), np.float64)
    lse = np.zeros((len(heads), r1 - r0), np.float64)
    index = {hd: n for n, hd in enumerate(heads)}

    def job(j):
        b, h, s0, s1 = j
        hk = h // G
        dst = np.zeros((s1 - s0, D), np.float64)
        ls = np.zeros(s1 - s0, np.float64)
        vptr = _ptr(v[b, hk]) if f >= 0 else None
        lib.oracle_attn_general(_ptr(qz["qhat"][b, h]), _ptr(qz["sq"][b, h]), Lq,
                                _ptr(qz["khat"][b, hk]), _ptr(qz["sk"][b, hk]),
                                _ptr(qz["vhat"][b, hk]), _ptr(qz["sv"][b, hk]), vptr, Lk,
                                D, Dp, float(sm_scale), causal, int(bk), f, PREF[pref], int(nsplit),
                                *_mask_args(block_mask, b, h, mask_block), s0, s1, _ptr(dst), _ptr(ls))
        out[index[(b, h)], s0 - r0:s1 - r0] = dst
        lse[index[(b, h)], s0 - r0:s1 - r0] = ls

    with ThreadPoolExecutor(_workers(len(jobs), threads)) as ex:
        list(ex.map(job, jobs))
    return out, lse


def attn_exact(q, k, v, sm_scale, causal=False, heads=None, rows=None, threads=None,
               chunk=64, block_mask=None, mask_block=(128, 128)):
    """Exact fp64 attention on logical-HND float32 inputs (GQA: hkv = hq // G).

    causal: False/0 none, True/1 top-left, 2 bottom-right; block_mask as in
    attn_general."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if block_mask is not None:
        block_mask = np.ascontiguousarray(block_mask, dtype=np.uint8)
        assert block_mask.shape == (B, Hq, -(-Lq // mask_block[0]), -(-Lk // mask_block[1])), block_mask.shape
    heads, (r0, r1), jobs = _row_jobs(B, Hq, Lq, heads, rows, chunk)
    out = np.zeros((len(heads), r1 - r0, D), np.float64)
    index = {hd: n for n, hd in enumerate(heads)}

    def job(j):
        b, h, s0, s1 = j
        hk = h // G
        dst = np.zeros((s1 - s0, D), np.float64)
        lib.oracle_attn_exact(_ptr(q[b, h]), _ptr(k[b, hk]), _ptr(v[b, hk]), Lq, Lk, D,
                              float(sm_scale), int(causal), *_mask_args(block_mask, b, h, mask_block),
                              s0, s1, _ptr(dst))
        out[index[(b, h)], s0 - r0:s1 - r0] = dst

    with ThreadPoolExecutor(_workers(len(jobs), threads)) as ex:
        list(ex.map(job, jobs))
    return out
