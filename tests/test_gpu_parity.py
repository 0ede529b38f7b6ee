"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bar (from the project statement of the method): the quantized workspace
(key mean, INT8 Q/K codes and scales, FP8 V codes and scales) and the int32
QK^T tiles are bit-exact; the output is within max-abs 2e-2 and cosine 0.999
of the oracle's quantized result, and within cosine 0.999 of exact fp64
attention. Every call goes through the C ABI (quantized_attention_sage_amd).

The INT8-QK / 16-bit-PV variant is held to the same bar, with its 16-bit V^T
bit-exact against the input values, and to the tighter accuracy the pages'
table gives that backend (cosine 0.9999 against fp64 on the configs).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_attention_sage_amd as qa
import sage_inputs as si

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
COS_MIN = 0.999
TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}
PERM = np.array([qa.vhat_position(j) for j in range(64)])


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def to_dev(x, dtype, layout):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(TDT[dtype])
    if layout == "NHD":
        t = t.permute(0, 2, 1, 3).contiguous()
    return t.cuda()


def from_dev(o, layout):
    o = o.float()
    if layout == "NHD":
        o = o.permute(0, 2, 1, 3)
    return o.cpu().double().numpy()


class Run:
    """One GPU run: quantize + attention through the C ABI, plus workspace copies."""

    def __init__(self, q, k, v, cfg, causal, smooth=True, sm=None, pv="fp8"):
        layout = cfg.get("layout", "HND")
        self.layout = layout
        self.pv = pv
        self.sm = sm if sm is not None else 1.0 / math.sqrt(cfg["D"])
        self.qd, self.kd, self.vd = (to_dev(x, cfg["dtype"], layout) for x in (q, k, v))
        self.od = torch.empty_like(self.qd)
        self.p = qa.make_problem(self.qd, self.kd, self.vd, self.od, layout, pv=pv)
        self.ws = qa.new_workspace(self.p)
        qa.quantize(self.p, self.qd, self.kd, self.vd, self.ws, smooth_k=smooth)
        qa.attn_quantized(self.p, self.ws, self.od, is_causal=causal, sm_scale=self.sm)
        torch.cuda.synchronize()
        self.o = from_dev(self.od, layout)
        self.views = {k_: (v_.cpu().numpy() if torch.is_tensor(v_) else v_)
                      for k_, v_ in qa.workspace_views(self.p, self.ws).items()}


PERM16 = np.array([qa.vhat_position(j, "fp16") for j in range(64)])


def check_workspace16(run, qz, v, dtype):
    """16-bit variant: Q/K sections as in the FP8 one; V^T holds the input bits."""
    w = run.views
    B, H, nkb, Dp, _ = w["vhat"].shape
    Lk, D = v.shape[2], v.shape[3]
    tok = w["vhat"][..., PERM16].transpose(0, 1, 2, 4, 3).reshape(B, H, nkb * 64, Dp)
    bits = torch.from_numpy(np.ascontiguousarray(v)).to(TDT[dtype]).view(torch.int16).numpy()
    assert np.array_equal(tok[:, :, :Lk, :D], bits)
    assert not tok[:, :, Lk:].any() and not tok[..., D + 1:].any()
    if D < Dp:
        # the normaliser channel: 1.0 in the input format for every real token
        one = torch.ones(1, dtype=TDT[dtype]).view(torch.int16).item()
        assert np.all(tok[:, :, :Lk, D] == one)
    assert np.array_equal(w["kbar"], qz["kbar"])
    assert np.array_equal(w["qhat"][:, :, :qz["qhat"].shape[2]], qz["qhat"])
    assert np.array_equal(w["khat"][:, :, :Lk], qz["khat"])
    nb = qz["sk"].shape[2]
    assert np.array_equal(w["sk"][:, :, :nb], qz["sk"])


def check_output16(run, qz, q, k, v, cfg, causal, heads=None, rows=None, cos_fp64=0.9999):
    bk = qa.softmax_block_keys()
    ref = oracle.attn_quantized_pv16(qz, v, run.sm, causal=causal, fmt=cfg["dtype"], bk=bk,
                                     heads=heads, rows=rows)
    ex = oracle.attn_exact(q, k, v, run.sm, causal=causal, heads=heads, rows=rows)
    r0, r1 = rows if rows is not None else (0, cfg["Lq"])
    hs = heads if heads is not None else [(b, h) for b in range(cfg["B"]) for h in range(cfg["Hq"])]
    got = np.stack([run.o[b, h, r0:r1] for (b, h) in hs])
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    c_q, c_e = _cos(got, ref), _cos(got, ex)
    print("pv16 max_abs %.3g cos_vs_oracle %.7f cos_vs_fp64 %.7f (oracle vs fp64 %.7f)"
          % (err, c_q, c_e, _cos(ref, ex)))
    assert err <= MAX_ABS
    assert c_q >= COS_MIN
    assert c_e >= cos_fp64
    return got, ref


def check_workspace(run, qz, Lq, Lk):
    w = run.views
    L = w["layout"]
    assert np.array_equal(w["kbar"], qz["kbar"])
    assert np.array_equal(w["qhat"][:, :, :Lq], qz["qhat"])
    assert not w["qhat"][:, :, Lq:].any()
    assert np.array_equal(w["sq"][:, :, :Lq], qz["sq"])
    assert not w["sq"][:, :, Lq:].any()
    assert np.array_equal(w["khat"][:, :, :Lk], qz["khat"])
    assert not w["khat"][:, :, Lk:].any()
    nb = qz["sk"].shape[2]
    assert np.array_equal(w["sk"][:, :, :nb], qz["sk"])
    assert not w["sk"][:, :, nb:].any()
    B, H, nkb, Dp, _ = w["vhat"].shape
    tok = w["vhat"][..., PERM].transpose(0, 1, 2, 4, 3).reshape(B, H, nkb * 64, Dp)
    D = qz["D"]
    assert np.array_equal(tok[:, :, :Lk, :D], qz["vhat"][..., :D])
    assert not tok[:, :, Lk:].any() and not tok[..., D + 1:].any()
    if D < Dp:
        assert np.all(tok[:, :, :Lk, D] == 0x38)       # the normaliser channel: E4M3 1.0
    assert np.array_equal((w["vmax"] / np.float32(448.0)).astype(np.float32), qz["sv"])
    assert L.Lk_pad == nkb * 64


def check_output(run, qz, q, k, v, cfg, causal, heads=None, rows=None):
    bk, pref = qa.softmax_spec("fp8")
    ref = oracle.attn_quantized(qz, run.sm, causal=causal, bk=bk, pref=pref, heads=heads, rows=rows)
    ex = oracle.attn_exact(q, k, v, run.sm, causal=causal, heads=heads, rows=rows)
    r0, r1 = rows if rows is not None else (0, cfg["Lq"])
    hs = heads if heads is not None else [(b, h) for b in range(cfg["B"]) for h in range(cfg["Hq"])]
    got = np.stack([run.o[b, h, r0:r1] for (b, h) in hs])
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    c_q, c_e = _cos(got, ref), _cos(got, ex)
    print("max_abs %.3g cos_vs_oracle %.6f cos_vs_fp64 %.6f (oracle vs fp64 %.6f)"
          % (err, c_q, c_e, _cos(ref, ex)))
    assert err <= MAX_ABS
    assert c_q >= COS_MIN
    assert c_e >= COS_MIN
    return got, ref


_CACHE = {}
_QZ = {}


def config_inputs(name):
    if name not in _CACHE:
        _CACHE[name] = si.make_inputs(name)
    return _CACHE[name]


def config_quantized(name):
    """The oracle's quantization of a config's inputs (computed once per session)."""
    if name not in _QZ:
        q, k, v, _ = config_inputs(name)
        _QZ[name] = oracle.quantize(q, k, v)
    return _QZ[name]


@pytest.mark.parametrize("name", ["c1", "c2", "c2c"])
def test_small_configs_full(name):
    q, k, v, cfg = config_inputs(name)
    qz = config_quantized(name)
    run = Run(q, k, v, cfg, cfg["causal"])
    check_workspace(run, qz, cfg["Lq"], cfg["Lk"])
    check_output(run, qz, q, k, v, cfg, cfg["causal"])


# Regression bar on the large shapes: the measured agreement with the
# oracle's quantized result is cos ~ 0.999999 there, so a slip in a block
# scale or in the normaliser (which the 0.999 bar would still let through)
# fails this one.
COS_REGRESS = 0.99999


def strided_windows(Lq, n=8, w=16):
    """n windows of w query rows spread over [0, Lq), the last ending at Lq
    (the ragged last tile when Lq is not a multiple of 128)."""
    starts = sorted({min(i * (Lq // n) + (37 * i) % max(Lq // n - w, 1), Lq - w) for i in range(n - 1)} | {Lq - w})
    return [(s, s + w) for s in starts]


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_large_configs_all_heads(name):
    # full-size run; the workspace is compared in full and the output on every
    # head, on windows of rows spread over the whole query range: max-abs and
    # cosine against the oracle's quantized result (with the regression bar),
    # cosine, relative L2 and max-abs against exact fp64 attention
    q, k, v, cfg = config_inputs(name)
    qz = config_quantized(name)
    run = Run(q, k, v, cfg, cfg["causal"])
    check_workspace(run, qz, cfg["Lq"], cfg["Lk"])
    bk, pref = qa.softmax_spec("fp8")
    got, ref, ex = [], [], []
    for (r0, r1) in strided_windows(cfg["Lq"]):
        ref.append(oracle.attn_quantized(qz, run.sm, causal=cfg["causal"], bk=bk, pref=pref, rows=(r0, r1)))
        ex.append(oracle.attn_exact(q, k, v, run.sm, causal=cfg["causal"], rows=(r0, r1)))
        got.append(run.o[:, :, r0:r1].reshape(ref[-1].shape))
    got, ref, ex = (np.concatenate(x, axis=1) for x in (got, ref, ex))
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    c_q, c_e = _cos(got, ref), _cos(got, ex)
    rel = float(np.linalg.norm(got - ex) / np.linalg.norm(ex))
    print("%s: %d heads x %d rows: max_abs %.3g cos_vs_oracle %.7f | vs fp64: cos %.6f rel_l2 %.4g "
          "max_abs %.3g" % (name, got.shape[0], got.shape[1], err, c_q, c_e, rel, np.abs(got - ex).max()))
    assert err <= MAX_ABS
    assert c_q >= COS_REGRESS
    assert c_e >= COS_MIN
    del run
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,heads", [("c1", [(0, 0), (0, 1)]), ("c2", [(0, 3)]),
                                        ("c3", [(1, 17)]), ("c4", [(0, 9)]), ("c5", [(0, 2)])])
def test_int32_logits_bit_exact(name, heads):
    q, k, v, cfg = config_inputs(name)
    G = cfg["Hq"] // cfg["Hkv"]
    kvh = sorted({h // G for _, h in heads})
    qz = oracle.quantize(q[:, sorted({h for _, h in heads})], k[:, kvh], v[:, kvh])
    qd, kd, vd = (to_dev(x, cfg["dtype"], cfg["layout"]) for x in (q, k, v))
    p = qa.make_problem(qd, kd, vd, torch.empty_like(qd), cfg["layout"])
    ws = qa.new_workspace(p)
    qa.quantize(p, qd, kd, vd, ws)
    hq_idx = sorted({h for _, h in heads})
    for b, h in heads:
        dump = qa.debug_qk_int32(p, ws, b, h).cpu().numpy()
        ref = oracle.qk_int32(qz["qhat"][b, hq_idx.index(h)], qz["khat"][b, kvh.index(h // G)])
        assert np.array_equal(dump[:cfg["Lq"], :cfg["Lk"]], ref)
        assert not dump[:cfg["Lq"], cfg["Lk"]:].any()


EDGE = [
    ("ragged_gqa_nhd", dict(B=2, Hq=6, Hkv=3, Lq=200, Lk=333, D=80, dtype="bf16", layout="NHD", kbias_var=2.0), False),
    ("ragged_gqa_nhd_causal", dict(B=2, Hq=6, Hkv=3, Lq=333, Lk=333, D=80, dtype="bf16", layout="NHD"), True),
    ("odd_dim_scalar_path", dict(B=1, Hq=2, Hkv=2, Lq=70, Lk=70, D=37, dtype="fp16", layout="HND"), False),
    ("single_token", dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=1, D=64, dtype="fp16", layout="HND"), False),
    ("lq_gt_lk_causal", dict(B=1, Hq=2, Hkv=1, Lq=300, Lk=64, D=128, dtype="fp16", layout="HND"), True),
    ("lq_lt_lk_causal", dict(B=1, Hq=2, Hkv=2, Lq=64, Lk=1000, D=128, dtype="bf16", layout="HND"), True),
    ("d16", dict(B=1, Hq=3, Hkv=1, Lq=130, Lk=129, D=16, dtype="fp16", layout="NHD"), False),
    ("d128_long_ragged", dict(B=1, Hq=2, Hkv=2, Lq=257, Lk=2049, D=128, dtype="fp16", layout="HND", kbias_var=4.0), False),
    # 131072 keys: the statistics finished by their own launch (512 chunks),
    # 1024 key blocks per query tile, cut by the automatic split into 16 ranges
    ("long_keys_131072", dict(B=1, Hq=2, Hkv=1, Lq=64, Lk=131072, D=128, dtype="fp16", layout="HND",
                              kbias_var=4.0), False),
    # many short entries (384 query tiles of one partial block each), causal
    ("many_short_entries", dict(B=96, Hq=4, Hkv=2, Lq=65, Lk=65, D=64, dtype="bf16", layout="NHD"), True),
    # short fp16 heads on more than one K/V workgroup per CU (640): the codes
    # kernel sums the statistics itself and loads its rows after them
    ("d128_short_heads_full_grid", dict(B=2, Hq=20, Hkv=20, Lq=40, Lk=1000, D=128, dtype="fp16", layout="HND",
                                        kbias_var=4.0), False),
]


@pytest.mark.parametrize("name,cfg,causal", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, cfg, causal):
    q, k, v, cfg = si.make_inputs(cfg, seed=0x5A6E1000 + len(name))
    qz = oracle.quantize(q, k, v)
    run = Run(q, k, v, cfg, causal)
    check_workspace(run, qz, cfg["Lq"], cfg["Lk"])
    check_output(run, qz, q, k, v, cfg, causal)


def test_smooth_off_and_zero_rows():
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=150, Lk=150, D=64, dtype="fp16", layout="HND")
    q, k, v, cfg = si.make_inputs(cfg, seed=77)
    q = q.copy()
    v = v.copy()
    q[0, 0, 5] = 0.0                  # zero query row: scale 0, uniform weights
    v[0, 1, :, 3] = 0.0               # zero value channel: scale 0, codes 0
    qz = oracle.quantize(q, k, v, smooth_k=False)
    run = Run(q, k, v, cfg, False, smooth=False)
    check_workspace(run, qz, 150, 150)
    check_output(run, qz, q, k, v, cfg, False)


def test_e4m3_rounding_midpoints_through_v():
    # Channel maxima of 448 make the V scale exactly 1, so the prologue's
    # hardware conversion sees the fp16 values themselves: every midpoint
    # between adjacent E4M3 codes below 448 and its two fp16 neighbours.
    pos = np.sort(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([mids, np.nextafter(mids.astype(np.float16), np.float16(0)).astype(np.float64),
                           np.nextafter(mids.astype(np.float16), np.float16(500)).astype(np.float64), pos])
    vals = vals[np.abs(vals) <= 448]
    vals = np.concatenate([vals, -vals]).astype(np.float16).astype(np.float32)
    n = len(vals)
    Lk = ((n + 63) // 64) * 64
    v = np.zeros((1, 1, Lk, 64), np.float32)
    v[0, 0, :n, 0] = vals
    v[0, 0, n:, 0] = 448.0
    v[0, 0, :, 1] = -448.0
    k = np.zeros_like(v)
    q = np.zeros((1, 1, 1, 64), np.float32)
    cfg = dict(B=1, Hq=1, Hkv=1, Lq=1, Lk=Lk, D=64, dtype="fp16", layout="HND")
    qz = oracle.quantize(q, k, v)
    run = Run(q, k, v, cfg, False)
    check_workspace(run, qz, 1, Lk)


def test_invariants_layout_gqa_views_padding_determinism():
    cfg = dict(B=2, Hq=4, Hkv=2, Lq=96, Lk=200, D=80, dtype="bf16", layout="HND", kbias_var=2.0)
    q, k, v, cfg = si.make_inputs(cfg, seed=91)
    dt = torch.bfloat16
    qd, kd, vd = (torch.from_numpy(x).to(dt).cuda() for x in (q, k, v))
    o_hnd = qa.sageattn(qd, kd, vd, "HND")
    # determinism
    assert torch.equal(o_hnd, qa.sageattn(qd, kd, vd, "HND"))
    # NHD holds the same values permuted
    o_nhd = qa.sageattn(*(x.permute(0, 2, 1, 3).contiguous() for x in (qd, kd, vd)), tensor_layout="NHD")
    assert torch.equal(o_hnd, o_nhd.permute(0, 2, 1, 3))
    # GQA equals the same call with each kv head repeated for its q heads
    o_rep = qa.sageattn(qd, kd.repeat_interleave(2, dim=1), vd.repeat_interleave(2, dim=1), "HND")
    assert torch.equal(o_hnd, o_rep)
    # fused qkv projection views (token stride 3*H*D, NHD) equal contiguous copies
    H, L, D = 4, 96, 80
    qkv = torch.from_numpy(si.gen_tensor(5, 0, 2, 3 * H, L, D, "bf16")).to(dt).cuda()
    qkv = qkv.view(2, 3, H, L, D).permute(0, 3, 1, 2, 4).contiguous()      # [B, L, 3, H, D]
    qv, kv_, vv = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert qv.stride(1) == 3 * H * D
    o_view = qa.sageattn(qv, kv_, vv, "NHD")
    o_copy = qa.sageattn(qv.contiguous(), kv_.contiguous(), vv.contiguous(), "NHD")
    assert torch.equal(o_view, o_copy)
    # head dim 80 equals a manual zero pad to 128 with the 1/sqrt(80) scale
    pad = lambda x: torch.nn.functional.pad(x, (0, 48))
    o_pad = qa.sageattn(pad(qd), pad(kd), pad(vd), "HND", sm_scale=1 / math.sqrt(80))
    assert torch.equal(o_hnd, o_pad[..., :80])
    assert not o_pad[..., 80:].any()


# (q scale, input seed): ~1.7k and ~2k (one-FMA form, just under the limit;
# the second is the worst of the probed seeds there), ~4k (exact form; with
# the one-FMA form up to 4096 this input broke the max-abs bar at 0.031) and
# ~14k (exact form)
FORMS = [(1.0, 0x0DE9A001), (1.15, 0x0DE9B001), (2.3, 0x0DE9B002), (8.0, 0x0DE9A008)]


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("qscale,seed", FORMS, ids=["q1", "q1.15", "q2.3", "q8"])
def test_dequantization_forms_at_the_regression_bar(qscale, seed, pv):
    # The attention kernel dequantizes a logit with one FMA whose addend
    # carries the accumulator bias (one rounding, at most 2^-14 in P's
    # exponent) while kMagic * scale stays below 2048, and subtracts the bias
    # exactly first above that. Rows where one key dominates (sharper logits,
    # q scaled up) are where a P rounding that differs from the oracle's
    # shows; every case is held to the regression bar against the oracle.
    cfg = dict(B=1, Hq=4, Hkv=2, Lq=1024, Lk=1024, D=128, dtype="fp16", layout="HND", kbias_var=4.0)
    q, k, v, cfg = si.make_inputs(cfg, seed=seed)
    q = (q * np.float32(qscale)).astype(np.float16).astype(np.float32)
    qz = oracle.quantize(q, k, v)
    run = Run(q, k, v, cfg, False, pv=pv)
    if pv == "fp8":
        check_workspace(run, qz, cfg["Lq"], cfg["Lk"])
        got, ref = check_output(run, qz, q, k, v, cfg, False)
    else:
        check_workspace16(run, qz, v, cfg["dtype"])
        # sharper logits than the pages' workloads: the method itself (the
        # oracle) is further from fp64 than the 16-bit table's 0.9999 here
        got, ref = check_output16(run, qz, q, k, v, cfg, False, cos_fp64=COS_MIN)
    assert _cos(got, ref) >= COS_REGRESS


def test_large_magnitude_causal_finite():
    cfg = dict(B=1, Hq=4, Hkv=4, Lq=512, Lk=512, D=128, dtype="fp16", layout="HND")
    q, k, v, cfg = si.make_inputs(cfg, seed=31)
    q, k, v = (x * np.float32(30.0) for x in (q, k, v))
    q, k, v = (x.astype(np.float16).astype(np.float32) for x in (q, k, v))
    qz = oracle.quantize(q, k, v)
    run = Run(q, k, v, cfg, True)
    assert np.all(np.isfinite(run.o))
    check_workspace(run, qz, 512, 512)
    bk, pref = qa.softmax_spec("fp8")
    ref = oracle.attn_quantized(qz, run.sm, causal=True, bk=bk, pref=pref)
    got = run.o.reshape(ref.shape)
    assert _cos(got, ref) >= COS_MIN and np.abs(got - ref).max() <= MAX_ABS * 30


def test_workspace_reuse_between_shapes():
    # one workspace serves a large call and then a smaller one
    big = dict(B=1, Hq=2, Hkv=2, Lq=300, Lk=700, D=128, dtype="fp16", layout="HND")
    small = dict(B=1, Hq=1, Hkv=1, Lq=33, Lk=65, D=64, dtype="fp16", layout="HND")
    qb, kb, vb, _ = si.make_inputs(big, seed=1)
    qs, ks, vs, _ = si.make_inputs(small, seed=2)
    dev = lambda x: torch.from_numpy(x).half().cuda()
    pb = qa.make_problem(dev(qb), dev(kb), dev(vb), None, "HND")
    ws = qa.new_workspace(pb)
    o1 = qa.sageattn(dev(qb), dev(kb), dev(vb), workspace=ws)
    o2 = qa.sageattn(dev(qs), dev(ks), dev(vs), workspace=ws)
    assert torch.equal(o2, qa.sageattn(dev(qs), dev(ks), dev(vs)))
    assert torch.equal(o1, qa.sageattn(dev(qb), dev(kb), dev(vb)))


# ---------------------------------------------------------------------------
# INT8-QK / 16-bit-PV variant
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c1", "c2", "c2c"])
def test_pv16_small_configs_full(name):
    q, k, v, cfg = config_inputs(name)
    qz = config_quantized(name)
    run = Run(q, k, v, cfg, cfg["causal"], pv="fp16")
    check_workspace16(run, qz, v, cfg["dtype"])
    check_output16(run, qz, q, k, v, cfg, cfg["causal"])


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_pv16_large_configs_all_heads(name):
    # every head, on the same windows of rows as the FP8 path
    q, k, v, cfg = config_inputs(name)
    qz = config_quantized(name)
    run = Run(q, k, v, cfg, cfg["causal"], pv="fp16")
    check_workspace16(run, qz, v, cfg["dtype"])
    for rows in strided_windows(cfg["Lq"]):
        check_output16(run, qz, q, k, v, cfg, cfg["causal"], rows=rows)
    del run
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,cfg,causal", EDGE, ids=[e[0] for e in EDGE])
def test_pv16_edge_shapes(name, cfg, causal):
    q, k, v, cfg = si.make_inputs(cfg, seed=0x5A6E1000 + len(name))
    qz = oracle.quantize(q, k, v)
    run = Run(q, k, v, cfg, causal, pv="fp16")
    check_workspace16(run, qz, v, cfg["dtype"])
    # single-key and tiny shapes: the INT8 logit error alone sets the accuracy
    check_output16(run, qz, q, k, v, cfg, causal, cos_fp64=0.999)


def test_pv16_more_accurate_than_fp8_and_invariants():
    cfg = dict(B=2, Hq=4, Hkv=2, Lq=96, Lk=200, D=80, dtype="bf16", layout="HND", kbias_var=2.0)
    q, k, v, cfg = si.make_inputs(cfg, seed=92)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    o16 = qa.sageattn_qk_int8_pv_fp16(qd, kd, vd)
    o8 = qa.sageattn_qk_int8_pv_fp8(qd, kd, vd)
    assert torch.equal(o8, qa.sageattn(qd, kd, vd))
    assert torch.equal(o16, qa.sageattn_qk_int8_pv_fp16(qd, kd, vd))          # deterministic
    ex = oracle.attn_exact(q, k, v, 1 / math.sqrt(80)).reshape(2, 4, 96, 80)
    e16 = np.linalg.norm(o16.double().cpu().numpy() - ex) / np.linalg.norm(ex)
    e8 = np.linalg.norm(o8.double().cpu().numpy() - ex) / np.linalg.norm(ex)
    assert e16 < e8 / 2
    o_rep = qa.sageattn_qk_int8_pv_fp16(qd, kd.repeat_interleave(2, dim=1), vd.repeat_interleave(2, dim=1))
    assert torch.equal(o16, o_rep)
    o_nhd = qa.sageattn_qk_int8_pv_fp16(*(x.permute(0, 2, 1, 3).contiguous() for x in (qd, kd, vd)),
                                        tensor_layout="NHD")
    assert torch.equal(o16, o_nhd.permute(0, 2, 1, 3))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_pv16_lazy_running_max(dtype):
    # Key magnitudes ramp up along the sequence and triple at key 640: the
    # per-block maxima of the logits rise by 1-2 (log2 units) from block to
    # block, which the 16-bit variant absorbs without a rescale (its running
    # maxima lag by up to 8, so P reaches 2^8), then by about 15, which forces
    # one. Output and LSE against the oracle, whose maxima are exact, in one
    # pass and in 2 key ranges.
    cfg = dict(B=1, Hq=2, Hkv=1, Lq=200, Lk=1000, D=64, dtype=dtype, layout="HND")
    q, k, v, cfg = si.make_inputs(cfg, seed=123)
    j = np.arange(cfg["Lk"])
    ramp = ((1.0 + 2.0 * j / cfg["Lk"]) * np.where(j >= 640, 3.0, 1.0)).astype(np.float32)
    k = torch.from_numpy(k * ramp[None, None, :, None]).to(TDT[dtype]).float().numpy()
    qz = oracle.quantize(q, k, v)
    run = Run(q, k, v, cfg, False, pv="fp16")
    check_workspace16(run, qz, v, dtype)
    check_output16(run, qz, q, k, v, cfg, False, cos_fp64=0.999)
    for nsplit in (1, 2):
        o = torch.empty_like(run.qd)
        lse = torch.empty((1, 2, cfg["Lq"]), dtype=torch.float32, device="cuda")
        qa.attn_quantized_ex(run.p, run.ws, o, is_causal=0, sm_scale=run.sm, nsplit=nsplit, lse=lse)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attn_general(qz, run.sm, v=v, pv="fp16", fmt=dtype, causal=0, nsplit=nsplit,
                                           bk=qa.softmax_block_keys())
        got = o.float().cpu().double().numpy().reshape(ref_o.shape)
        d = np.abs(lse.cpu().double().numpy().reshape(ref_l.shape) - ref_l)
        print("nsplit %d max_abs %.3g cos %.7f lse max %.3g mean %.3g"
              % (nsplit, np.abs(got - ref_o).max(), _cos(got, ref_o), d.max(), d.mean()))
        assert np.abs(got - ref_o).max() <= MAX_ABS and _cos(got, ref_o) >= COS_MIN
        assert d.max() <= 1e-2 and d.mean() <= 2e-4
