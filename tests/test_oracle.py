"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one step of the oracle to a closed form, an invariant of the
mathematics, a brute-force computation on tiny inputs, a value printed by the
pages or a format specification, or an independent library routine (torch's
float8_e4m3fn cast), so that a dropped term, a wrong sign, a wrong index or a
transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import sage_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cos_rel(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    cos = float(a @ b / math.sqrt((a @ a) * (b @ b)))
    rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    return cos, rel


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


# ---------------------------------------------------------------------------
# FP8 E4M3FN codec
# ---------------------------------------------------------------------------
def test_e4m3_spec_points():
    g = _golden("ocp_e4m3_points.json")
    for code, val in g["points"]:
        c = int(code, 16)
        assert oracle.e4m3_decode([c])[0] == val
        assert oracle.e4m3_encode([val])[0] == c
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3_decode([int(code, 16)])[0])


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = _torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_encode_midpoints_and_neighbours_vs_torch():
    # every midpoint between adjacent finite codes and its two fp32 neighbours
    pos = np.sort(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                          pos.astype(np.float32)])
    pts = pts[np.abs(pts) <= 448]
    pts = np.concatenate([pts, -pts])
    ours = oracle.e4m3_encode(pts.astype(np.float64))
    assert np.array_equal(ours, _torch_e4m3(pts))


def test_e4m3_encode_random_vs_torch_and_brute_force():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 20000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    ours = oracle.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(ours, _torch_e4m3(x))
    # brute force on a subset: nearest finite code, ties to the even code
    table = _torch_e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = [c for c in range(256) if not np.isnan(table[c])]
    for xv, oc in zip(x[:500].astype(np.float64), ours[:500]):
        d = [abs(table[c] - xv) for c in finite]
        best = min(d)
        cands = [c for c, dd in zip(finite, d) if dd == best]
        if len(cands) > 1:   # tie: even mantissa; zeros keep the sign of x
            cands = [c for c in cands if (c & 1) == 0]
            if len(cands) > 1:
                cands = [c for c in cands if (c >> 7) == (1 if xv < 0 else 0)]
        assert oc == cands[0], (xv, oc, cands)


def test_e4m3_saturation_and_zero_sign():
    enc = oracle.e4m3_encode([448.0, 460.0, 1e6, -1e6, 1e-12, -1e-12, 0.0, -0.0])
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x00, 0x80]


# ---------------------------------------------------------------------------
# Head-dim padding (sd.cpp doc)
# ---------------------------------------------------------------------------
def test_padded_dim_matches_page_rule():
    g = _golden("sd_cpp_head_dim_padding.json")
    for lo, hi, p in g["ranges"]:
        for d in range(lo, hi + 1):
            assert oracle.padded_dim(d) == p


# ---------------------------------------------------------------------------
# INT8 quantizers
# ---------------------------------------------------------------------------
def _quant_q(q2d):
    q4 = q2d[None, None].astype(np.float32)
    qz = oracle.quantize(q4, q4, q4)
    return qz["qhat"][0, 0], qz["sq"][0, 0], qz["Dp"]


def test_quant_q_ties_round_to_even_and_zero_row():
    D = 8
    row = np.array([127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5], np.float32)   # amax 127 -> r = 1
    zero = np.zeros(D, np.float32)
    codes, s, Dp = _quant_q(np.stack([row, zero]))
    assert list(codes[0, :D]) == [127, 2, 4, -2, 0, 0, 2, -126]
    assert np.all(codes[0, D:] == 0) and Dp == 64
    assert s[0] == np.float32(1.0)
    assert np.all(codes[1] == 0) and s[1] == 0.0


def test_quant_q_invariants_fp16_rows():
    q, _, _, _ = si.make_inputs(dict(B=1, Hq=1, Hkv=1, Lq=300, Lk=4, D=80, dtype="fp16"), seed=11)
    q = q[0, 0] * np.float32(3.0)
    codes, s, Dp = _quant_q(q)
    assert Dp == 128
    c = codes[:, :80].astype(np.float64)
    assert np.all(np.abs(codes) <= 127) and np.all(codes[:, 80:] == 0)
    amax_idx = np.argmax(np.abs(q), axis=1)
    assert np.all(np.abs(c[np.arange(300), amax_idx]) == 127)
    assert np.all(np.sign(c) * np.sign(q) >= 0)            # no sign flips
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(q.astype(np.float64) - c * s64)
    # rne(q * r) with r = 127/a and s = a/127 each rounded once in fp32:
    # |q - c*s| <= s/2 + s * 127 * 2^-22
    assert np.all(err <= s64 / 2 * (1 + 2 ** -13) + 1e-30)
    # scale is amax/127 correctly rounded in fp32
    assert np.array_equal(s, (np.abs(q).max(axis=1) / np.float32(127.0)).astype(np.float32))


def _f32_nearest(fr):
    """Correctly rounded fp32 of an exact Fraction (ties to even)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def test_k_mean_is_exact_mean_for_fp16():
    # fp16 values are multiples of 2^-24 bounded by 65504: the fp64 sum of
    # 1000 of them is exact in any order, so the oracle's mean must be the
    # correctly rounded exact rational mean (up to the final double rounding
    # fp64 -> fp32, which this seed does not hit).
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=1000, D=24, dtype="fp16")
    _, k, v, _ = si.make_inputs(cfg, seed=5)
    k = k * np.float32(16.0) + np.float32(3.0)
    k = k.astype(np.float16).astype(np.float32)
    qz = oracle.quantize(k[:, :, :1], k, v, smooth_k=True)
    kbar = qz["kbar"][0, 0]
    for d in range(24):
        exact = sum(Fraction(float(x)) for x in k[0, 0, :, d]) / 1000
        assert kbar[d] == _f32_nearest(exact), d
    assert np.all(kbar[24:] == 0)
    qz0 = oracle.quantize(k[:, :, :1], k, v, smooth_k=False)
    assert np.all(qz0["kbar"] == 0)


def test_quant_k_blocks_smoothing_and_tail():
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=150, D=64, dtype="fp16", kbias_var=4.0)
    q, k, v, _ = si.make_inputs(cfg, seed=9)
    k = k.copy()
    k[0, 0, 64:128] *= np.float32(4.0)          # second block has a larger range
    qz = oracle.quantize(q, k, v, smooth_k=True)
    kbar = qz["kbar"][0, 0]
    kt = k[0, 0] - kbar[None, :]                # fp32 subtraction, as specified
    sk = qz["sk"][0, 0]
    assert sk.shape == (3,)
    for b, (j0, j1) in enumerate([(0, 64), (64, 128), (128, 150)]):
        a = np.abs(kt[j0:j1]).max()
        assert sk[b] == np.float32(a) / np.float32(127.0)
        codes = qz["khat"][0, 0, j0:j1].astype(np.float64)
        err = np.abs(kt[j0:j1].astype(np.float64) - codes * np.float64(sk[b]))
        assert np.all(err <= np.float64(sk[b]) / 2 * (1 + 2 ** -13))
        assert np.abs(codes).max() == 127
    assert sk[1] > 2 * sk[0]
    # with a dominant per-channel bias, smoothing removes it and every block scale shrinks
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=150, D=64, dtype="fp16", kbias_var=16.0)
    q, k, v, _ = si.make_inputs(cfg, seed=9)
    on = oracle.quantize(q, k, v, smooth_k=True)["sk"][0, 0]
    off = oracle.quantize(q, k, v, smooth_k=False)["sk"][0, 0]
    assert np.all(on < 0.6 * off)


def test_quant_v_per_channel():
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=130, D=40, dtype="bf16")
    q, k, v, _ = si.make_inputs(cfg, seed=3)
    v = v.copy()
    v[0, 0, :, 5] = 0.0                          # an all-zero channel
    qz = oracle.quantize(q, k, v)
    sv = qz["sv"][0, 0]
    codes = qz["vhat"][0, 0]
    assert codes.shape == (130, 64)
    c = np.abs(v[0, 0]).max(axis=0)
    assert np.array_equal(sv[:40], (c / np.float32(448.0)).astype(np.float32))
    assert sv[5] == 0 and np.all(codes[:, 5] == 0)
    assert np.all(sv[40:] == 0) and np.all(codes[:, 40:] == 0)
    dec = _torch_e4m3_decode(codes)[:, :40]
    # the channel max lands on +-448
    idx = np.argmax(np.abs(v[0, 0]), axis=0)
    for d in range(40):
        if d != 5:
            assert abs(dec[idx[d], d]) == 448.0
    # relative error of each code is at most half a step of the format (2^-4),
    # absolute error at most half the subnormal step below 2^-6
    rec = dec * sv[None, :40].astype(np.float64)
    err = np.abs(rec - v[0, 0])
    bound = np.maximum(np.abs(v[0, 0]) * 2.0 ** -4, sv[None, :40] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


# ---------------------------------------------------------------------------
# int32 logits
# ---------------------------------------------------------------------------
def test_qk_int32_brute_force():
    rng = np.random.default_rng(1)
    qh = rng.integers(-127, 128, (5, 64), dtype=np.int64).astype(np.int8)
    kh = rng.integers(-127, 128, (7, 64), dtype=np.int64).astype(np.int8)
    out = oracle.qk_int32(qh, kh)
    for i in range(5):
        for j in range(7):
            assert out[i, j] == sum(int(qh[i, d]) * int(kh[j, d]) for d in range(64))
    # extreme values stay exact
    big = np.full((1, 128), 127, np.int8)
    assert oracle.qk_int32(big, -big)[0, 0] == -127 * 127 * 128


# ---------------------------------------------------------------------------
# Exact attention
# ---------------------------------------------------------------------------
def _numpy_attention(q, k, v, sm, causal):
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Lq, D))
    for b in range(B):
        for h in range(Hq):
            s = sm * (q[b, h].astype(np.float64) @ k[b, h // G].astype(np.float64).T)
            if causal:
                s = np.where(np.triu(np.ones_like(s, bool), 1), -np.inf, s)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h] = (p / p.sum(axis=1, keepdims=True)) @ v[b, h // G].astype(np.float64)
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_exact_attention_vs_numpy(causal):
    cfg = dict(B=2, Hq=4, Hkv=2, Lq=37, Lk=37, D=24, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=21)
    ours = oracle.attn_exact(q, k, v, 0.3, causal=causal)
    ref = _numpy_attention(q, k, v, 0.3, causal).reshape(8, 37, 24)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_exact_attention_special_cases():
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=6, Lk=6, D=16, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=2)
    # causal row 0 sees only key 0
    o = oracle.attn_exact(q, k, v, 0.25, causal=True)
    assert np.array_equal(o[0, 0], v[0, 0, 0].astype(np.float64))
    # zero query: uniform weights -> mean of v (prefix means when causal)
    z = np.zeros_like(q)
    o = oracle.attn_exact(z, k, v, 0.25, causal=False)
    assert np.allclose(o[0], v[0, 0].astype(np.float64).mean(axis=0)[None], atol=1e-14)
    o = oracle.attn_exact(z, k, v, 0.25, causal=True)
    pref = np.cumsum(v[0, 0].astype(np.float64), axis=0) / np.arange(1, 7)[:, None]
    assert np.allclose(o[0], pref, atol=1e-14)
    # one key
    o = oracle.attn_exact(q, k[:, :, :1], v[:, :, :1], 0.25)
    assert np.array_equal(o[0], np.repeat(v[0, 0, :1].astype(np.float64), 6, axis=0))


def test_exact_attention_key_shift_invariance():
    # Smoothing K adds the row constant q . kbar to every logit of a row:
    # softmax is unchanged (the reason smoothing is lossless before quantization).
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=40, Lk=70, D=32, dtype="fp16", kbias_var=4.0)
    q, k, v, _ = si.make_inputs(cfg, seed=4)
    kbar = k.astype(np.float64).mean(axis=2, keepdims=True)
    o1 = oracle.attn_exact(q, k, v, 0.2)
    o2 = oracle.attn_exact(q, (k - kbar).astype(np.float32), v, 0.2)
    # k - kbar rounded to fp32 perturbs logits by ~1e-7 relative
    assert np.max(np.abs(o1 - o2)) < 1e-5
    # exact version of the identity in fp64 on the numpy side
    r1 = _numpy_attention(q.astype(np.float64), k.astype(np.float64), v, 0.2, False)
    r2 = _numpy_attention(q.astype(np.float64), k.astype(np.float64) - kbar, v, 0.2, False)
    assert np.max(np.abs(r1 - r2)) < 1e-12


# ---------------------------------------------------------------------------
# Quantized attention
# ---------------------------------------------------------------------------
def _qattn(q, k, v, sm, causal=False, bk=128, smooth=True):
    qz = oracle.quantize(q, k, v, smooth_k=smooth)
    return oracle.attn_quantized(qz, sm, causal=causal, bk=bk), qz


def test_quantized_zero_query_gives_mean_of_quantized_v():
    # q = 0 -> every logit 0 -> P~ = 1 -> P^ = E4M3(256) = 256 exactly, so the
    # output is s_v times the mean of the decoded V codes (prefix means when causal).
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=50, Lk=50, D=16, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=8)
    z = np.zeros_like(q)
    for causal in (False, True):
        o, qz = _qattn(z, k, v, 0.25, causal=causal, bk=16)
        vd = _torch_e4m3_decode(qz["vhat"][0, 0])[:, :16] * qz["sv"][0, 0, :16].astype(np.float64)
        if causal:
            ref = np.cumsum(vd, axis=0) / np.arange(1, 51)[:, None]
        else:
            ref = np.repeat(vd.mean(axis=0, keepdims=True), 50, axis=0)
        assert np.allclose(o[0], ref, rtol=1e-13, atol=1e-15)


def test_quantized_dominant_key_selects_its_value():
    # Row i has one key (index perm[i]) with a logit far above the rest:
    # every other P~ underflows the FP8 grid and the output is that key's
    # dequantized value row exactly.
    Lq, Lk, D = 12, 40, 16
    rng = np.random.default_rng(3)
    perm = rng.permutation(Lk)[:Lq]
    q = np.zeros((1, 1, Lq, D), np.float32)
    k = np.zeros((1, 1, Lk, D), np.float32)
    for i in range(Lq):
        q[0, 0, i, i] = 1.0
        k[0, 0, perm[i], i] = 1.0
    v = si.make_inputs(dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=Lk, D=D, dtype="fp16"), seed=6)[2]
    o, qz = _qattn(q, k, v, 60.0, bk=16, smooth=False)
    vd = _torch_e4m3_decode(qz["vhat"][0, 0])[:, :D] * qz["sv"][0, 0, :D].astype(np.float64)
    assert np.allclose(o[0], vd[perm], rtol=1e-14, atol=0)


def test_quantized_single_key():
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=9, Lk=1, D=8, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=12)
    o, qz = _qattn(q, k, v, 0.5)
    vd = _torch_e4m3_decode(qz["vhat"][0, 0, 0])[:8] * qz["sv"][0, 0, :8]
    assert np.allclose(o[0], np.repeat(vd[None], 9, axis=0), rtol=1e-14)


def test_quantized_online_blocks_carry_rescale():
    # Different key-block sizes only change which running maximum P is
    # quantized against; a missing or wrong alpha rescale would break this.
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=64, Lk=300, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=13)
    q = q * np.float32(2.0)
    qz = oracle.quantize(q, k, v)
    o_small = oracle.attn_quantized(qz, 0.125, bk=16)
    o_one = oracle.attn_quantized(qz, 0.125, bk=1024)
    cos, rel = _cos_rel(o_small, o_one)
    assert cos > 0.9995 and rel < 0.03
    ex = oracle.attn_exact(q, k, v, 0.125)
    for o in (o_small, o_one):
        assert _cos_rel(o, ex)[0] > 0.999


def test_quantized_scale_invariance_q_times_two():
    # q -> 2q doubles s_q exactly and keeps the codes, so with sm_scale/2 the
    # logits, and therefore the outputs, are bit-identical.
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=33, Lk=90, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=14)
    o1, qz1 = _qattn(q, k, v, 0.125)
    o2, qz2 = _qattn(q * np.float32(2.0), k, v, 0.0625)
    assert np.array_equal(qz1["qhat"], qz2["qhat"])
    assert np.array_equal(o1, o2)


def test_quantized_gqa_equals_repeated_kv_heads():
    cfg = dict(B=2, Hq=4, Hkv=2, Lq=20, Lk=70, D=32, dtype="bf16")
    q, k, v, _ = si.make_inputs(cfg, seed=15)
    o_gqa, _ = _qattn(q, k, v, 0.2)
    o_rep, _ = _qattn(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), 0.2)
    assert np.array_equal(o_gqa, o_rep)


def test_quantized_head_dim_padding_equals_manual_zero_pad():
    # D = 80 is padded to 128 inside; padding the inputs by hand with zeros
    # and keeping the 1/sqrt(80) scale gives the same codes and outputs.
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=30, Lk=75, D=80, dtype="bf16", kbias_var=2.0)
    q, k, v, _ = si.make_inputs(cfg, seed=16)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:3] + (48,), np.float32)], axis=3)
    sm = 1 / math.sqrt(80)
    o1, qz1 = _qattn(q, k, v, sm)
    o2, qz2 = _qattn(pad(q), pad(k), pad(v), sm)
    for key in ("qhat", "sq", "khat", "sk", "vhat", "sv", "kbar"):
        assert np.array_equal(qz1[key], qz2[key]), key
    assert np.array_equal(o1, o2[..., :80])


@pytest.mark.parametrize("name", ["c1", "c2", "c2c"])
def test_quantized_vs_exact_within_page_envelope(name):
    # the accuracy bar: cosine >= 0.999 vs fp64 on random fp16; the page's fp8-PV
    # backend shows rel_l2 0.0345-0.0381 and cos >= 0.99927 (used as a loose envelope).
    env = _golden("sm120a_accuracy_table.json")["sageattn_qk_int8_pv_fp8_cuda"]
    q, k, v, cfg = si.make_inputs(name)
    sm = 1 / math.sqrt(cfg["D"])
    o, _ = _qattn(q, k, v, sm, causal=cfg["causal"])
    e = oracle.attn_exact(q, k, v, sm, causal=cfg["causal"])
    cos, rel = _cos_rel(o, e)
    assert cos >= 0.999
    assert 0.5 * env["rel_l2"][0] <= rel <= 1.25 * env["rel_l2"][1]


def test_smoothing_helps_with_key_channel_bias():
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=128, Lk=512, D=128, dtype="fp16", kbias_var=4.0)
    q, k, v, _ = si.make_inputs(cfg, seed=17)
    sm = 1 / math.sqrt(128)
    e = oracle.attn_exact(q, k, v, sm)
    on, _ = _qattn(q, k, v, sm, smooth=True)
    off, _ = _qattn(q, k, v, sm, smooth=False)
    c_on, r_on = _cos_rel(on, e)
    c_off, r_off = _cos_rel(off, e)
    assert c_on >= 0.999 and r_on < r_off


def test_large_magnitude_causal_is_finite():
    # sm_120a page, accuracy section: large-magnitude causal inputs give no NaN/Inf.
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=96, Lk=96, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=18)
    o, _ = _qattn(q * np.float32(30.0), k * np.float32(30.0), v * np.float32(30.0), 0.125, causal=True)
    assert np.all(np.isfinite(o))


def test_p_quantization_uses_static_2_pow_8_scale():
    # Two keys with P~ = (1, 1.5 * 2^-14): scaled by 2^8 both land exactly on
    # E4M3 codes (256 and 1.5 * 2^-6), so the output ratio between the two
    # one-hot value channels is exactly 1.5 * 2^-14. Any other scale would push
    # the small weight into the subnormal grid and change the ratio.
    D = 16
    q = np.zeros((1, 1, 1, D), np.float32)
    k = np.zeros((1, 1, 2, D), np.float32)
    v = np.zeros((1, 1, 2, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 1, 0] = -1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, 1] = 1.0
    gap = 14 * math.log(2.0) - math.log(1.5)     # logit difference for P~ = 1.5 * 2^-14
    o, _ = _qattn(q, k, v, gap / 2.0, smooth=False)
    ratio = o[0, 0, 1] / o[0, 0, 0]
    assert abs(ratio / (1.5 * 2.0 ** -14) - 1.0) < 1e-6


# ---------------------------------------------------------------------------
# 16-bit float rounding and the INT8-QK / 16-bit-PV variant ("8+16")
# ---------------------------------------------------------------------------
def test_round_16bit_spec_points():
    g = _golden("ieee_binary16_bfloat16_points.json")
    for fn, key in ((oracle.round_f16, "binary16"), (oracle.round_bf16, "bfloat16")):
        for x, y in g[key]:
            assert fn([x])[0] == float(y), (key, x, y)


def test_round_f16_vs_numpy_and_all_codes():
    # every binary16 value rounds to itself; random fp64 values (normal,
    # subnormal, overflow) round like numpy's float64 -> float16 cast
    allv = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    fin = allv[np.isfinite(allv)]
    assert np.array_equal(oracle.round_f16(fin), fin)
    rng = np.random.default_rng(21)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-25, 12, 200000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_f16(x), ref)
    # the midpoints between neighbouring binary16 values go to the even one
    pos = np.sort(fin[fin > 0])
    mid = (pos[:-1] + pos[1:]) / 2.0
    got = oracle.round_f16(mid)
    even = np.where((pos[:-1].astype(np.float16).view(np.uint16) & 1) == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, even)


def test_round_bf16_vs_torch():
    # bfloat16 rounding of fp32-representable values, against torch's
    # float32 -> bfloat16 cast (round to nearest even)
    rng = np.random.default_rng(22)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def _qattn16(q, k, v, sm, fmt="fp16", causal=False, bk=128, smooth=True):
    qz = oracle.quantize(q, k, v, smooth_k=smooth)
    return oracle.attn_quantized_pv16(qz, v, sm, causal=causal, fmt=fmt, bk=bk), qz


def test_pv16_zero_query_gives_mean_of_v():
    # q = 0 -> P~ = 1 -> P^ = 1 exactly: the output is the (prefix) mean of V itself
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=40, Lk=40, D=16, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=23)
    z = np.zeros_like(q)
    for causal in (False, True):
        o, _ = _qattn16(z, k, v, 0.25, causal=causal, bk=16)
        vd = v[0, 0].astype(np.float64)
        ref = (np.cumsum(vd, axis=0) / np.arange(1, 41)[:, None]) if causal else np.repeat(vd.mean(0, keepdims=True), 40, 0)
        assert np.allclose(o[0], ref, rtol=1e-13, atol=1e-15)


def test_pv16_single_key_and_dominant_key():
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=5, Lk=1, D=8, dtype="bf16")
    q, k, v, _ = si.make_inputs(cfg, seed=24)
    o, _ = _qattn16(q, k, v, 0.5, fmt="bf16")
    assert np.array_equal(o[0], np.repeat(v[0, 0].astype(np.float64), 5, axis=0))
    # one key per row far above the rest: the others round to 0 in binary16
    Lq, Lk, D = 10, 30, 16
    perm = np.random.default_rng(4).permutation(Lk)[:Lq]
    q = np.zeros((1, 1, Lq, D), np.float32)
    k = np.zeros((1, 1, Lk, D), np.float32)
    for i in range(Lq):
        q[0, 0, i, i] = 1.0
        k[0, 0, perm[i], i] = 1.0
    v = si.make_inputs(dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=Lk, D=D, dtype="fp16"), seed=7)[2]
    o, _ = _qattn16(q, k, v, 60.0, bk=16, smooth=False)
    assert np.array_equal(o[0], v[0, 0, perm].astype(np.float64))


def test_pv16_rounds_p_to_the_input_format():
    # Two keys, one-hot values: out = (P0, P1) / (P0 + P1) with P0 = 1 and P1
    # the 16-bit rounding of exp(-gap). The expected weights use numpy's and
    # torch's casts; leaving P unrounded, or rounding it to the other format
    # or to FP8, changes the ratio.
    D = 16
    q = np.zeros((1, 1, 1, D), np.float32)
    k = np.zeros((1, 1, 2, D), np.float32)
    v = np.zeros((1, 1, 2, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 1, 0] = -1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, 1] = 1.0
    for sm in (0.61, 1.37, 2.9):
        qz = oracle.quantize(q, k, v, smooth_k=False)
        a = oracle.qk_int32(qz["qhat"][0, 0], qz["khat"][0, 0])[0]
        lg = a.astype(np.float64) * float(qz["sq"][0, 0, 0]) * qz["sk"][0, 0, 0].astype(np.float64) * sm
        p1 = math.exp(lg[1] - lg[0])
        for fmt, cast in (("fp16", lambda x: float(np.float64(x).astype(np.float16))),
                          ("bf16", lambda x: float(torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double()))):
            o = oracle.attn_quantized_pv16(qz, v, sm, fmt=fmt)[0, 0]
            w1 = cast(p1)
            assert abs(o[1] / o[0] - w1) <= 1e-15 * w1, (fmt, sm)
            assert w1 != p1


def test_pv16_vs_exact_and_more_accurate_than_fp8():
    # sm_120a accuracy table: the FP16-PV backend has rel_l2 0.0092-0.0112 and
    # cos >= 0.99994 against float64, about 3.7x below the FP8-PV backend.
    env16 = _golden("sm120a_accuracy_table.json")["sageattn_qk_int8_pv_fp16_cuda"]
    for name in ("c1", "c2", "c2c"):
        q, k, v, cfg = si.make_inputs(name)
        sm = 1 / math.sqrt(cfg["D"])
        qz = oracle.quantize(q, k, v)
        o16 = oracle.attn_quantized_pv16(qz, v, sm, causal=cfg["causal"])
        o8 = oracle.attn_quantized(qz, sm, causal=cfg["causal"])
        e = oracle.attn_exact(q, k, v, sm, causal=cfg["causal"])
        c16, r16 = _cos_rel(o16, e)
        c8, r8 = _cos_rel(o8, e)
        assert c16 >= env16["cos_min"] - 5e-5
        assert r16 <= 1.5 * env16["rel_l2"][1]
        assert r16 < r8 / 2.0


def test_pv16_gqa_blocks_and_causal_row0():
    cfg = dict(B=1, Hq=4, Hkv=2, Lq=70, Lk=70, D=32, dtype="bf16")
    q, k, v, _ = si.make_inputs(cfg, seed=25)
    qz = oracle.quantize(q, k, v)
    o = oracle.attn_quantized_pv16(qz, v, 0.2, fmt="bf16", causal=True)
    assert np.array_equal(o[:, 0], v[0, [0, 0, 1, 1], 0].astype(np.float64))
    qr = oracle.quantize(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1))
    o_rep = oracle.attn_quantized_pv16(qr, np.repeat(v, 2, axis=1), 0.2, fmt="bf16", causal=True)
    assert np.array_equal(o, o_rep)
    # different block sizes only change the maxima P is rounded against
    o_small = oracle.attn_quantized_pv16(qz, v, 0.2, fmt="bf16", bk=16)
    o_big = oracle.attn_quantized_pv16(qz, v, 0.2, fmt="bf16", bk=1024)
    assert _cos_rel(o_small, o_big)[0] > 0.99999


# ---------------------------------------------------------------------------
# Key-range splits, causal alignment, log-sum-exp (attn_general)
# ---------------------------------------------------------------------------
def test_general_reduces_to_the_unsplit_variants():
    cfg = dict(B=1, Hq=2, Hkv=1, Lq=90, Lk=300, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=31)
    qz = oracle.quantize(q, k, v)
    for causal in (False, True):
        ref8 = oracle.attn_quantized(qz, 0.125, causal=causal)
        g8, _ = oracle.attn_general(qz, 0.125, causal=int(causal))
        assert np.allclose(g8, ref8, rtol=1e-12, atol=1e-14)
        ref16 = oracle.attn_quantized_pv16(qz, v, 0.125, causal=causal)
        g16, _ = oracle.attn_general(qz, 0.125, v=v, pv="fp16", causal=int(causal))
        assert np.allclose(g16, ref16, rtol=1e-12, atol=1e-14)


def _two_keys(gap_over_2):
    # query e_0 against keys +e_0 and -e_0 (one 128-key block each when the
    # second sits at position 128), one-hot values
    D = 16
    q = np.zeros((1, 1, 1, D), np.float32)
    k = np.zeros((1, 1, 129, D), np.float32)
    v = np.zeros((1, 1, 129, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 128, 0] = -1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 128, 1] = 1.0
    k[0, 0, 1:128, 0] = -1.0e4          # other keys: weight exp(-huge) = 0 exactly
    return q, k, v


def test_split_combines_the_ranges_exactly():
    # Keys 0 and 128 in different ranges (nsplit = 2, bk = 128): each range
    # has one visible weight P~ = 1, quantized exactly, so the combination is
    # the exact two-way softmax, and the LSE is log(e^x0 + e^x128). Without
    # the split the smaller weight goes through E4M3 and the ratio changes.
    q, k, v = _two_keys(None)
    qz = oracle.quantize(q, k, v, smooth_k=False)
    sm = 0.9
    a = oracle.qk_int32(qz["qhat"][0, 0], qz["khat"][0, 0])[0]
    x0 = a[0] * float(qz["sq"][0, 0, 0]) * float(qz["sk"][0, 0, 0]) * sm
    x1 = a[128] * float(qz["sq"][0, 0, 0]) * float(qz["sk"][0, 0, 2]) * sm
    ratio = math.exp(x1 - x0)
    for pv in ("fp8", "fp16"):
        # (the FP8 V scale 1/448 is rounded to fp32, which scales both outputs alike)
        o2, l2 = oracle.attn_general(qz, sm, v=v, pv=pv, nsplit=2)
        assert abs(o2[0, 0, 1] / o2[0, 0, 0] / ratio - 1.0) < 1e-14
        assert abs(o2[0, 0, 0] + o2[0, 0, 1] - 1.0) < (1e-7 if pv == "fp8" else 1e-15)
        assert abs(l2[0, 0] - math.log(math.exp(x0) + math.exp(x1))) < 1e-13
        o1, _ = oracle.attn_general(qz, sm, v=v, pv=pv, nsplit=1)
        assert abs(o1[0, 0, 1] / o1[0, 0, 0] / ratio - 1.0) > 1e-5


def test_lse_closed_forms_and_empty_rows():
    # q = 0: every visible logit is 0, P~ = 1 is exact in both formats, so the
    # LSE is log(number of visible keys) exactly (prefix counts when causal)
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=40, Lk=300, D=16, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=32)
    qz = oracle.quantize(np.zeros_like(q), k, v)
    for pv in ("fp8", "fp16"):
        for nsplit in (1, 3):
            _, l0 = oracle.attn_general(qz, 0.3, v=v, pv=pv, nsplit=nsplit)
            assert np.allclose(l0[0], math.log(300), rtol=0, atol=1e-13)
            _, l1 = oracle.attn_general(qz, 0.3, v=v, pv=pv, causal=1, nsplit=nsplit)
            assert np.allclose(l1[0], np.log(np.arange(1, 41)), atol=1e-13)
            o2, l2 = oracle.attn_general(qz, 0.3, v=v, pv=pv, causal=2, nsplit=nsplit)
            assert np.allclose(l2[0], np.log(np.arange(261, 301)), atol=1e-13)
    # bottom-right with Lq > Lk: the first Lq - Lk rows see no key
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=50, Lk=20, D=16, dtype="bf16")
    q, k, v, _ = si.make_inputs(cfg, seed=33)
    qz = oracle.quantize(q, k, v)
    o, l = oracle.attn_general(qz, 0.25, causal=2, nsplit=2)
    assert not o[0, :30].any() and np.all(np.isneginf(l[0, :30]))
    assert np.all(np.isfinite(l[0, 30:]))
    e = oracle.attn_exact(q, k, v, 0.25, causal=2)
    assert not e[0, :30].any()
    assert _cos_rel(o[0, 30:], e[0, 30:])[0] > 0.999


def test_bottom_right_causal_exact_vs_numpy_and_special_cases():
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=33, Lk=70, D=32, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=34)
    sm = 0.2
    got = oracle.attn_exact(q, k, v, sm, causal=2)[0]
    s = (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T) * sm
    i = np.arange(33)[:, None]
    j = np.arange(70)[None, :]
    s[j > i + 70 - 33] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ v[0, 0].astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    # Lq == Lk: bottom-right is top-left
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=60, Lk=60, D=32, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=35)
    assert np.array_equal(oracle.attn_exact(q, k, v, sm, causal=2), oracle.attn_exact(q, k, v, sm, causal=1))
    qz = oracle.quantize(q, k, v)
    a, _ = oracle.attn_general(qz, sm, causal=2)
    b, _ = oracle.attn_general(qz, sm, causal=1)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_splits_stay_within_the_envelope(pv):
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=64, Lk=1000, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=36)
    sm = 0.125
    qz = oracle.quantize(q, k, v)
    e = oracle.attn_exact(q, k, v, sm)
    o1, l1 = oracle.attn_general(qz, sm, v=v, pv=pv, nsplit=1)
    for ns in (2, 3, 8):
        o, l = oracle.attn_general(qz, sm, v=v, pv=pv, nsplit=ns)
        assert _cos_rel(o, e)[0] >= (0.999 if pv == "fp8" else 0.9999)
        assert _cos_rel(o, o1)[0] > 0.9995
        assert np.abs(l - l1).max() < 0.02


# ---------------------------------------------------------------------------
# Block-sparse patterns (block_mask)
# ---------------------------------------------------------------------------
def _rand_mask(rng, B, H, Lq, Lk, density):
    return (rng.random((B, H, -(-Lq // 128), -(-Lk // 128))) < density).astype(np.uint8)


def test_block_mask_all_ones_and_key_subset():
    cfg = dict(B=1, Hq=2, Hkv=1, Lq=200, Lk=600, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=41)
    qz = oracle.quantize(q, k, v)
    ones = np.ones((1, 2, 2, 5), np.uint8)
    for pv in ("fp8", "fp16"):
        a, la = oracle.attn_general(qz, 0.125, v=v, pv=pv, nsplit=2)
        b, lb = oracle.attn_general(qz, 0.125, v=v, pv=pv, nsplit=2, block_mask=ones)
        assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert np.array_equal(oracle.attn_exact(q, k, v, 0.125), oracle.attn_exact(q, k, v, 0.125, block_mask=ones))
    # key blocks 1 and 2 only (keys 128..383), for every query block: the same
    # as attention over those keys alone, with the same quantized codes
    sub = np.zeros_like(ones)
    sub[..., 1:3] = 1
    ks, vs = k[:, :, 128:384], v[:, :, 128:384]
    assert np.array_equal(oracle.attn_exact(q, k, v, 0.125, block_mask=sub), oracle.attn_exact(q, ks, vs, 0.125))
    qz_sub = dict(qz)
    qz_sub["khat"] = np.ascontiguousarray(qz["khat"][:, :, 128:384])
    qz_sub["vhat"] = np.ascontiguousarray(qz["vhat"][:, :, 128:384])
    qz_sub["sk"] = np.ascontiguousarray(qz["sk"][:, :, 2:6])
    for pv in ("fp8", "fp16"):
        a, la = oracle.attn_general(qz, 0.125, v=v, pv=pv, block_mask=sub)
        b, lb = oracle.attn_general(qz_sub, 0.125, v=np.ascontiguousarray(vs), pv=pv)
        assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_block_mask_lower_triangle_is_causal_and_empty_rows():
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=300, Lk=300, D=32, dtype="bf16")
    q, k, v, _ = si.make_inputs(cfg, seed=42)
    qz = oracle.quantize(q, k, v)
    tri = np.tril(np.ones((3, 3), np.uint8))[None, None].repeat(2, axis=1)
    for pv in ("fp8", "fp16"):
        a, la = oracle.attn_general(qz, 0.2, v=v, pv=pv, fmt="bf16", causal=1)
        b, lb = oracle.attn_general(qz, 0.2, v=v, pv=pv, fmt="bf16", causal=1, block_mask=tri)
        assert np.array_equal(a, b) and np.array_equal(la, lb)
    # a query block without any block: zero rows, LSE -inf (exact attention too)
    m = np.ones((1, 2, 3, 3), np.uint8)
    m[0, 1, 1] = 0
    o, l = oracle.attn_general(qz, 0.2, block_mask=m)
    assert not o[1, 128:256].any() and np.all(np.isneginf(l[1, 128:256]))
    assert np.all(np.isfinite(l[0])) and np.all(np.isfinite(l[1, :128])) and np.all(np.isfinite(l[1, 256:]))
    e = oracle.attn_exact(q, k, v, 0.2, block_mask=m)
    assert not e[1, 128:256].any()
    assert np.array_equal(e[0], oracle.attn_exact(q, k, v, 0.2)[0])


def test_block_mask_is_elementwise_minus_inf_and_per_head():
    # exact attention with a random block pattern equals the softmax with -inf
    # on the skipped (query, key) blocks; each q head reads its own pattern
    cfg = dict(B=2, Hq=4, Hkv=2, Lq=260, Lk=400, D=16, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=43)
    rng = np.random.default_rng(5)
    m = _rand_mask(rng, 2, 4, 260, 400, 0.6)
    m[:, :, :, 0] = 1                            # every query sees some key
    got = oracle.attn_exact(q, k, v, 0.3, block_mask=m).reshape(2, 4, 260, 16)
    for b in range(2):
        for h in range(4):
            s = q[b, h].astype(np.float64) @ k[b, h // 2].astype(np.float64).T * 0.3
            full = np.kron(m[b, h], np.ones((128, 128), np.uint8))[:260, :400]
            s[full == 0] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            ref = p / p.sum(axis=1, keepdims=True) @ v[b, h // 2].astype(np.float64)
            assert np.allclose(got[b, h], ref, rtol=1e-12, atol=1e-14)
    # the quantized scheme under the same pattern stays within the envelope
    qz = oracle.quantize(q, k, v)
    for pv in ("fp8", "fp16"):
        o, _ = oracle.attn_general(qz, 0.3, v=v, pv=pv, nsplit=3, block_mask=m)
        assert _cos_rel(o.reshape(got.shape), got)[0] > (0.999 if pv == "fp8" else 0.9999)


# ---------------------------------------------------------------------------
# The normaliser reading: l is the sum of the quantized weights that multiply V
# ---------------------------------------------------------------------------
# The pages do not say which weights the softmax denominator sums (topgit.dev,
# "SageAttention vs FlashAttention": blockwise softmax, no formula). The reading
# taken is the sum of the same quantized weights that multiply V, so the output
# is a convex combination of the dequantized values. These pins use one query
# against two keys in one softmax block with one-hot values: the smaller
# weight exp(-gap) lies strictly between two codes of the P format, so the sum
# of the quantized weights and the sum of the unquantized ones differ, and
# every assertion below fails under the other reading.
def _norm_case():
    D = 16
    q = np.zeros((1, 1, 1, D), np.float32)
    k = np.zeros((1, 1, 2, D), np.float32)
    v = np.zeros((1, 1, 2, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 1, 0] = -1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, 1] = 1.0
    qz = oracle.quantize(q, k, v, smooth_k=False)
    a = oracle.qk_int32(qz["qhat"][0, 0], qz["khat"][0, 0])[0]
    unit = float(a[0]) * float(qz["sq"][0, 0, 0]) * float(qz["sk"][0, 0, 0])   # logit of key 0 at sm = 1
    assert a[1] == -a[0]
    return q, k, v, qz, unit


def _e4m3_round(x):
    """E4M3FN value nearest to x (torch's cast, an independent routine)."""
    return float(_torch_e4m3_decode(_torch_e4m3([x]))[0])


def _f16_round(x):
    return float(np.float64(x).astype(np.float16))


def _bf16_round(x):
    return float(torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).double())


# target unquantized weights exp(-gap): each sits well inside a gap between two
# codes of every P format (FP8 as 256 * w, binary16 and bfloat16 as w)
_NORM_TARGETS = (0.3, 0.0123, 0.71)


def test_normaliser_is_sum_of_fp8_weights():
    q, k, v, qz, unit = _norm_case()
    sv = float(qz["sv"][0, 0, 0])                 # 1/448 rounded to fp32 (both channels)
    vdec = 448.0 * sv                             # dequantized value 1 of channels 0 and 1
    assert float(qz["sv"][0, 0, 1]) == sv
    for target in _NORM_TARGETS:
        gap = -math.log(target)
        sm = gap / (2.0 * unit)
        x0 = unit * sm
        p1 = math.exp(-2.0 * x0)
        w1 = _e4m3_round(256.0 * p1)              # dec(P^) of the smaller weight, times 2^8
        assert abs(w1 / (256.0 * p1) - 1.0) > 1e-3   # quantization visibly moves it
        den = 256.0 + w1                          # sum of dec(P^): the reading
        exp0, exp1 = vdec * 256.0 / den, vdec * w1 / den
        o = oracle.attn_quantized(qz, sm)[0, 0]
        assert abs(o[0] - exp0) <= 1e-15 and abs(o[1] - exp1) <= 1e-15, target
        assert abs(o[0] + o[1] - vdec) <= 1e-15
        og, lse = oracle.attn_general(qz, sm)
        assert abs(og[0, 0, 0] - exp0) <= 1e-15 and abs(og[0, 0, 1] - exp1) <= 1e-15
        # the LSE in the unit of the weights actually used: x0 + ln(sum dec(P^) / 2^8)
        assert abs(lse[0, 0] - (x0 + math.log(den / 256.0))) <= 1e-14
        assert abs(lse[0, 0] - (x0 + math.log(1.0 + p1))) > 1e-4


@pytest.mark.parametrize("fmt", ["fp16", "bf16"])
def test_normaliser_is_sum_of_16bit_weights(fmt):
    q, k, v, qz, unit = _norm_case()
    rnd = _f16_round if fmt == "fp16" else _bf16_round
    for target in _NORM_TARGETS:
        gap = -math.log(target)
        sm = gap / (2.0 * unit)
        x0 = unit * sm
        p1 = math.exp(-2.0 * x0)
        w1 = rnd(p1)
        assert abs(w1 / p1 - 1.0) > (2e-5 if fmt == "fp16" else 2e-4)
        den = 1.0 + w1
        o = oracle.attn_quantized_pv16(qz, v, sm, fmt=fmt)[0, 0]
        assert abs(o[0] - 1.0 / den) <= 1e-15 and abs(o[1] - w1 / den) <= 1e-15, (fmt, target)
        assert abs(o[0] + o[1] - 1.0) <= 2e-16
        og, lse = oracle.attn_general(qz, sm, v=v, pv="fp16", fmt=fmt)
        assert abs(og[0, 0, 0] - 1.0 / den) <= 1e-15 and abs(og[0, 0, 1] - w1 / den) <= 1e-15
        assert abs(lse[0, 0] - (x0 + math.log(den))) <= 1e-14
        assert abs(lse[0, 0] - (x0 + math.log(1.0 + p1))) > 1e-9


# ---------------------------------------------------------------------------
# The reference P is quantized against: the running maximum, or power-of-two
# steps above it (softmax_reference in the oracle's C source)
# ---------------------------------------------------------------------------
def _two_block_case(gap_log2, x0=9.0, sub=None, sub_ref=None):
    # one query against key 0 (block 0, logit x0), keys 1..63 (block 0, logit
    # -x0: weights below the smallest FP8 code), key 64 (block 1, logit about
    # x0 + gap_log2 * ln 2) and, when sub is given, key 65 (block 1, logit
    # chosen so that 2^8 times its weight against the power-of-two reference
    # is about sub, in the subnormal range of E4M3); one-hot values on keys
    # 0, 64 and 65
    D = 16
    Lk = 66 if sub else 65
    q = np.zeros((1, 1, 1, D), np.float32)
    k = np.zeros((1, 1, Lk, D), np.float32)
    v = np.zeros((1, 1, Lk, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 1:64, 0] = -1.0
    c = (x0 + gap_log2 * math.log(2.0)) / x0
    k[0, 0, 64, 0] = np.float32(c)
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 64, 1] = 1.0
    if sub:
        # sub_ref: the reference of block 1 in factors of two above x0
        n = math.ceil(gap_log2) if sub_ref is None else sub_ref
        x65 = x0 + n * math.log(2.0) + math.log(sub / 256.0)
        k[0, 0, 65, 0] = np.float32(x65 / x0)
        v[0, 0, 65, 2] = 1.0
    qz = oracle.quantize(q, k, v, smooth_k=False)
    a = oracle.qk_int32(qz["qhat"][0, 0], qz["khat"][0, 0])[0]
    sq = float(qz["sq"][0, 0, 0])
    sm = x0 / (float(a[0]) * sq * float(qz["sk"][0, 0, 0]))
    xs = [float(a[j]) * sq * float(qz["sk"][0, 0, j // 64]) * sm for j in range(Lk)]
    vdec = 448.0 * float(qz["sv"][0, 0, 0])
    for ch in range(1, 3 if sub else 2):
        assert float(qz["sv"][0, 0, ch]) == float(qz["sv"][0, 0, 0])
    return qz, sm, xs, vdec


@pytest.mark.parametrize("gap", [0.4, 1.3, 1.9, 3.6])
def test_pow2_reference_closed_form(gap):
    # 2^8 times the third key's weight lands at about 2.7 steps of the E4M3
    # subnormal grid (2^-9), where rounding is not invariant under a factor 2;
    # gap 1.9 would put the second key's weight above 448 (saturation) under
    # a reference one factor of two lower: both expose a wrong step count
    qz, sm, xs, vdec = _two_block_case(gap, sub=2.7 * 2.0 ** -9)
    x0, xm, x64, x65 = xs[0], xs[1], xs[64], xs[65]
    assert _e4m3_round(256.0 * math.exp(xm - x0)) == 0.0      # keys 1..63 drop out
    assert x65 < x64
    n = math.ceil((x64 - x0) / math.log(2.0))
    assert n == math.ceil(gap)
    # power-of-two steps: block 0 is quantized against x0 (its maximum), then
    # the reference rises by n factors of two; block 1 against x0 + n ln 2
    ref1 = x0 + n * math.log(2.0)
    w0 = 256.0 * 2.0 ** -n
    w64 = _e4m3_round(256.0 * math.exp(x64 - ref1))
    w65 = _e4m3_round(256.0 * math.exp(x65 - ref1))
    assert 128.0 < w64 <= 256.0 and 0.0 < w65 < 2.0 ** -6
    den = w0 + w64 + w65
    o = oracle.attn_quantized(qz, sm, bk=64, pref="pow2")[0, 0]
    og, lse = oracle.attn_general(qz, sm, bk=64, pref="pow2")
    for out in (o, og[0, 0]):
        assert abs(out[0] - vdec * w0 / den) <= 1e-15, gap
        assert abs(out[1] - vdec * w64 / den) <= 1e-15, gap
        assert abs(out[2] - vdec * w65 / den) <= 1e-17, gap
    assert abs(lse[0, 0] - (ref1 + math.log(den / 256.0))) <= 1e-13
    # the running maximum: block 1 is quantized against x64 itself (weight 256)
    # and block 0's exact 256 is rescaled by e^(x0 - x64)
    m0, m64, m65 = 256.0 * math.exp(x0 - x64), 256.0, _e4m3_round(256.0 * math.exp(x65 - x64))
    om = oracle.attn_quantized(qz, sm, bk=64, pref="max")[0, 0]
    dm = m0 + m64 + m65
    assert abs(om[0] - vdec * m0 / dm) <= 1e-15
    assert abs(om[1] - vdec * m64 / dm) <= 1e-15
    assert abs(o[1] / o[0] - om[1] / om[0]) > 1e-3 * (om[1] / om[0])


def test_pow2_reference_agrees_when_the_first_block_holds_the_maximum():
    # the first block sets the reference to its own maximum and later blocks
    # below it do not move it: one block, and a falling second block, give the
    # same bits under both rules
    qz, sm, _, _ = _two_block_case(-2.5)
    a = oracle.attn_quantized(qz, sm, bk=64, pref="pow2")
    b = oracle.attn_quantized(qz, sm, bk=64, pref="max")
    assert np.array_equal(a, b)
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=40, Lk=64, D=64, dtype="fp16")
    q, k, v, _ = si.make_inputs(cfg, seed=41)
    qz = oracle.quantize(q, k, v)
    assert np.array_equal(oracle.attn_quantized(qz, 0.125, bk=64, pref="pow2"),
                          oracle.attn_quantized(qz, 0.125, bk=64, pref="max"))


@pytest.mark.parametrize("name", ["c1", "c2", "c2c"])
def test_pow2_reference_within_page_envelope(name):
    # only the rounding point of P moves: the result stays within the pages'
    # FP8-PV envelope against fp64 and close to the running-maximum rule
    env = _golden("sm120a_accuracy_table.json")["sageattn_qk_int8_pv_fp8_cuda"]
    q, k, v, cfg = si.make_inputs(name)
    sm = 1 / math.sqrt(cfg["D"])
    qz = oracle.quantize(q, k, v)
    p2 = oracle.attn_quantized(qz, sm, causal=cfg["causal"], bk=64, pref="pow2")
    mx = oracle.attn_quantized(qz, sm, causal=cfg["causal"], bk=64, pref="max")
    e = oracle.attn_exact(q, k, v, sm, causal=cfg["causal"])
    cos, rel = _cos_rel(p2, e)
    assert cos >= 0.999 and 0.5 * env["rel_l2"][0] <= rel <= 1.25 * env["rel_l2"][1]
    assert _cos_rel(p2, mx)[0] > 0.9995
    assert not np.array_equal(p2, mx)
    g, _ = oracle.attn_general(qz, sm, causal=int(cfg["causal"]), bk=64, pref="pow2")
    assert np.allclose(g, p2, rtol=1e-12, atol=1e-14)


def test_pow2_reference_rising_logits_and_lse():
    # logits that rise by several factors of two per block and then jump: the
    # power-of-two reference follows them (the weights stay in range) and the
    # result stays close to the exact softmax; q = 0 gives LSE = log(count)
    Lk, D = 640, 32
    rng = np.random.default_rng(42)
    q = np.zeros((1, 1, 8, D), np.float32)
    q[0, 0, :, 0] = 1.0
    k = rng.standard_normal((1, 1, Lk, D)).astype(np.float32) * np.float32(0.1)
    k[0, 0, :, 0] = np.linspace(0.0, 6.0, Lk, dtype=np.float32)
    k[0, 0, 600:, 0] += np.float32(20.0)
    v = rng.standard_normal((1, 1, Lk, D)).astype(np.float32)
    qz = oracle.quantize(q, k, v, smooth_k=False)
    o = oracle.attn_quantized(qz, 2.0, bk=64, pref="pow2")
    om = oracle.attn_quantized(qz, 2.0, bk=64, pref="max")
    e = oracle.attn_exact(q, k, v, 2.0)
    # a handful of keys carry the softmax here, so FP8 V dominates the error
    # of both rules against fp64 (about 0.995); the rules agree closely
    assert np.all(np.isfinite(o)) and _cos_rel(o, om)[0] > 0.9995
    assert _cos_rel(o, e)[0] > 0.99 and _cos_rel(om, e)[0] > 0.99
    qz0 = oracle.quantize(np.zeros_like(q), k, v)
    for nsplit in (1, 3):
        _, l0 = oracle.attn_general(qz0, 0.3, bk=64, pref="pow2", nsplit=nsplit)
        assert np.allclose(l0[0], math.log(Lk), rtol=0, atol=1e-13)
        _, l1 = oracle.attn_general(qz0, 0.3, bk=64, pref="pow2", nsplit=nsplit, causal=1)
        assert np.allclose(l1[0], np.log(np.arange(1, 9)), atol=1e-13)


LAZY_OVER, LAZY_SLACK = 2.0, 0.75


@pytest.mark.parametrize("gap", [0.5, 2.6, 2.9, 4.2])
def test_lazy_reference_closed_form(gap):
    # the lazy rule: block 0 is quantized against its maximum plus two factors
    # of two (weight 2^-2); block 1 keeps that reference while its maximum is
    # within 0.75 of a factor of two of it (gaps 0.5 and 2.6: the second key's
    # weight 2^(gap - 2) goes up to 2^0.6), and otherwise moves it to its own
    # maximum plus two factors of two (gaps 2.9 and 4.2), rescaling block 0
    # by e^(old - new). A slack of 0.5 or 1.0, or an overshoot of 1 or 3,
    # changes the weights of one of the four cases; the third key sits in the
    # E4M3 subnormal range against the reference block 1 uses.
    moved = gap > LAZY_SLACK + LAZY_OVER
    r1 = gap + LAZY_OVER if moved else LAZY_OVER
    qz, sm, xs, vdec = _two_block_case(gap, sub=2.7 * 2.0 ** -9, sub_ref=r1)
    x0, xm, x64, x65 = xs[0], xs[1], xs[64], xs[65]
    ln2 = math.log(2.0)
    assert _e4m3_round(256.0 * math.exp(xm - x0)) == 0.0      # keys 1..63 drop out
    ref0 = x0 + LAZY_OVER * ln2
    assert ((x64 - ref0) > LAZY_SLACK * ln2) == moved
    ref1 = x64 + LAZY_OVER * ln2 if moved else ref0
    alpha = math.exp(ref0 - ref1)
    w0 = _e4m3_round(256.0 * math.exp(x0 - ref0))
    assert w0 == 64.0
    w64 = _e4m3_round(256.0 * math.exp(x64 - ref1))
    w65 = _e4m3_round(256.0 * math.exp(x65 - ref1))
    assert 0.0 < w65 < 2.0 ** -6
    assert w64 == 64.0 if moved else 64.0 < w64 <= 448.0
    den = alpha * w0 + w64 + w65
    o = oracle.attn_quantized(qz, sm, bk=64, pref="lazy")[0, 0]
    og, lse = oracle.attn_general(qz, sm, bk=64, pref="lazy")
    for out in (o, og[0, 0]):
        assert abs(out[0] - vdec * alpha * w0 / den) <= 1e-15, gap
        assert abs(out[1] - vdec * w64 / den) <= 1e-15, gap
        assert abs(out[2] - vdec * w65 / den) <= 1e-17, gap
    assert abs(lse[0, 0] - (ref1 + math.log(den / 256.0))) <= 1e-13
    # the running maximum gives other weights: when block 1 keeps the lazy
    # reference its key has weight 2^(gap - 2) there but 2^0 under the
    # maximum; when the reference moves, both rules scale the two normal
    # weights alike and only the subnormal third key rounds differently
    om = oracle.attn_quantized(qz, sm, bk=64, pref="max")[0, 0]
    if moved:
        assert o[2] != om[2]
    else:
        assert abs(o[1] / o[0] - om[1] / om[0]) > 1e-3 * (om[1] / om[0])


def test_lazy_reference_weights_stay_in_range_and_lse():
    # logits that rise by several factors of two per block and then jump: the
    # reference moves only on some blocks, every weight stays below 448 / 256
    # (no saturation), the result stays close to the running-maximum rule and
    # to the exact softmax, and q = 0 gives LSE = log(count)
    Lk, D = 640, 32
    rng = np.random.default_rng(43)
    q = np.zeros((1, 1, 8, D), np.float32)
    q[0, 0, :, 0] = 1.0
    k = rng.standard_normal((1, 1, Lk, D)).astype(np.float32) * np.float32(0.1)
    k[0, 0, :, 0] = np.linspace(0.0, 6.0, Lk, dtype=np.float32)
    k[0, 0, 600:, 0] += np.float32(20.0)
    v = rng.standard_normal((1, 1, Lk, D)).astype(np.float32)
    qz = oracle.quantize(q, k, v, smooth_k=False)
    o = oracle.attn_quantized(qz, 2.0, bk=64, pref="lazy")
    om = oracle.attn_quantized(qz, 2.0, bk=64, pref="max")
    e = oracle.attn_exact(q, k, v, 2.0)
    assert np.all(np.isfinite(o)) and _cos_rel(o, om)[0] > 0.9995
    assert _cos_rel(o, e)[0] > 0.99
    qz0 = oracle.quantize(np.zeros_like(q), k, v)
    for nsplit in (1, 3):
        _, l0 = oracle.attn_general(qz0, 0.3, bk=64, pref="lazy", nsplit=nsplit)
        assert np.allclose(l0[0], math.log(Lk), rtol=0, atol=1e-13)
        _, l1 = oracle.attn_general(qz0, 0.3, bk=64, pref="lazy", nsplit=nsplit, causal=1)
        assert np.allclose(l1[0], np.log(np.arange(1, 9)), atol=1e-13)


@pytest.mark.parametrize("name", ["c1", "c2", "c2c"])
def test_lazy_reference_within_page_envelope(name):
    # only the rounding point of P moves: the result stays within the pages'
    # FP8-PV envelope against fp64 and close to the running-maximum rule
    env = _golden("sm120a_accuracy_table.json")["sageattn_qk_int8_pv_fp8_cuda"]
    q, k, v, cfg = si.make_inputs(name)
    sm = 1 / math.sqrt(cfg["D"])
    qz = oracle.quantize(q, k, v)
    lz = oracle.attn_quantized(qz, sm, causal=cfg["causal"], bk=128, pref="lazy")
    mx = oracle.attn_quantized(qz, sm, causal=cfg["causal"], bk=128, pref="max")
    e = oracle.attn_exact(q, k, v, sm, causal=cfg["causal"])
    cos, rel = _cos_rel(lz, e)
    assert cos >= 0.999 and 0.5 * env["rel_l2"][0] <= rel <= 1.25 * env["rel_l2"][1]
    assert _cos_rel(lz, mx)[0] > 0.9995
    # one block of keys (c1): every weight is the maximum rule's times 2^-2,
    # which E4M3 rounds alike while no weight is subnormal, so the bits agree;
    # over several blocks the reference lags and they do not
    assert np.array_equal(lz, mx) == (cfg["Lk"] <= 128)
    g, _ = oracle.attn_general(qz, sm, causal=int(cfg["causal"]), bk=128, pref="lazy")
    assert np.allclose(g, lz, rtol=1e-12, atol=1e-14)
