"""GPU parity of block-sparse attention (block_mask; needs an MI355X).

A flag per block of 128 queries x 128 keys decides whether the block is
computed; the oracle's attn_general / attn_exact take the same mask. Bar: the
output bar of the dense path against the oracle and against exact fp64
attention under the same mask, rows of query blocks without any flag exactly
0 with LSE -inf, the LSE bar of the split tests. Invariants, bit for bit: an
all-ones mask equals no mask; the lower block triangle with a causal mask
equals the causal mask alone. Every call goes through the C ABI.
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
LSE_MAX = 1e-2
LSE_MEAN = 2e-4
TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = math.sqrt(a @ a), math.sqrt(b @ b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    return float(a @ b / (na * nb))


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


def make_mask(cfg, density, seed, empty_qblocks=()):
    rng = np.random.default_rng(seed)
    shape = (cfg["B"], cfg["Hq"], -(-cfg["Lq"] // 128), -(-cfg["Lk"] // 128))
    m = (rng.random(shape) < density).astype(np.uint8)
    for (b, h, i) in empty_qblocks:
        m[b, h, i] = 0
    return m


class Sparse:
    """Prologue once, then attention calls with options through the C ABI."""

    def __init__(self, q, k, v, cfg, pv):
        self.cfg = cfg
        self.layout = cfg.get("layout", "HND")
        self.sm = 1.0 / math.sqrt(cfg["D"])
        self.qd, self.kd, self.vd = (to_dev(x, cfg["dtype"], self.layout) for x in (q, k, v))
        self.p = qa.make_problem(self.qd, self.kd, self.vd, torch.empty_like(self.qd), self.layout, pv=pv)
        self.ws = qa.new_workspace(self.p)
        qa.quantize(self.p, self.qd, self.kd, self.vd, self.ws)

    def run(self, mask=None, causal=0, nsplit=1):
        o = torch.empty_like(self.qd)
        lse = torch.empty((self.p.B, self.p.Hq, self.p.Lq), dtype=torch.float32, device="cuda")
        md = torch.from_numpy(mask).cuda() if mask is not None else None
        qa.attn_quantized_ex(self.p, self.ws, o, is_causal=causal, sm_scale=self.sm, nsplit=nsplit, lse=lse,
                             block_mask=md)
        torch.cuda.synchronize()
        return o, lse


def check(o_t, l_t, q, k, v, cfg, mask, causal, nsplit, pv, heads=None, rows=None, qz=None):
    layout = cfg.get("layout", "HND")
    got_o = from_dev(o_t, layout)
    got_l = l_t.cpu().double().numpy()
    qz = qz if qz is not None else oracle.quantize(q, k, v)
    sm = 1.0 / math.sqrt(cfg["D"])
    bk, pref = qa.softmax_spec(pv)
    ref_o, ref_l = oracle.attn_general(qz, sm, v=v, pv=pv, fmt=cfg["dtype"], causal=causal, nsplit=nsplit,
                                       bk=bk, pref=pref, heads=heads, rows=rows, block_mask=mask)
    ex = oracle.attn_exact(q, k, v, sm, causal=causal, heads=heads, rows=rows, block_mask=mask)
    r0, r1 = rows if rows is not None else (0, cfg["Lq"])
    hs = heads if heads is not None else [(b, h) for b in range(cfg["B"]) for h in range(cfg["Hq"])]
    o = np.stack([got_o[b, h, r0:r1] for (b, h) in hs])
    lse = np.stack([got_l[b, h, r0:r1] for (b, h) in hs])
    assert np.all(np.isfinite(o))
    empty = ~np.isfinite(ref_l)
    assert np.all(o[empty] == 0.0)
    assert np.array_equal(np.isneginf(lse), empty)
    err = np.abs(o - ref_o).max()
    c_q, c_e = _cos(o, ref_o), _cos(o, ex)
    d = np.abs(lse[~empty] - ref_l[~empty])
    print("mask density %.2f causal %d nsplit %d pv %s: empty rows %d max_abs %.3g cos_vs_oracle %.6f "
          "cos_vs_fp64 %.6f lse max %.3g mean %.3g" % (mask.mean(), causal, nsplit, pv, empty.sum(), err, c_q, c_e,
                                                       d.max(), d.mean()))
    assert d.max() <= LSE_MAX and d.mean() <= LSE_MEAN
    assert err <= MAX_ABS
    assert c_q >= COS_MIN
    assert c_e >= COS_MIN


CASES = [
    # name, shape, density, causal, nsplit, pv, empty query blocks
    ("fp8_half", dict(B=2, Hq=2, Hkv=2, Lq=384, Lk=640, D=64, dtype="fp16", layout="HND"), 0.5, 0, 1, "fp8",
     [(0, 1, 1)]),
    ("pv16_two_qblocks_per_tile", dict(B=1, Hq=3, Hkv=1, Lq=520, Lk=900, D=128, dtype="bf16", layout="NHD"), 0.4, 0, 1,
     "fp16", [(0, 0, 1), (0, 2, 4)]),
    ("fp8_causal_split", dict(B=1, Hq=4, Hkv=2, Lq=700, Lk=700, D=80, dtype="bf16", layout="NHD", kbias_var=2.0),
     0.6, 1, 3, "fp8", [(0, 3, 2)]),
    ("pv16_bottom_right_split", dict(B=1, Hq=2, Hkv=2, Lq=200, Lk=1300, D=64, dtype="fp16", layout="HND"), 0.3, 2, 2,
     "fp16", []),
    ("fp8_sparse_tail_d37", dict(B=1, Hq=2, Hkv=2, Lq=150, Lk=1000, D=37, dtype="fp16", layout="HND"), 0.5, 0, 1,
     "fp8", [(0, 0, 0)]),
]


@pytest.mark.parametrize("name,cfg,density,causal,nsplit,pv,empty", CASES, ids=[c[0] for c in CASES])
def test_block_sparse_against_oracle(name, cfg, density, causal, nsplit, pv, empty):
    q, k, v, cfg = si.make_inputs(cfg, seed=0x5A6E4000 + len(name))
    mask = make_mask(cfg, density, seed=len(name), empty_qblocks=empty)
    # besides the emptied query blocks, every query block has work
    for b in range(cfg["B"]):
        for h in range(cfg["Hq"]):
            for i in range(mask.shape[2]):
                if (b, h, i) not in empty and not mask[b, h, i].any():
                    mask[b, h, i, -1] = 1
    s = Sparse(q, k, v, cfg, pv)
    o, lse = s.run(mask, causal, nsplit)
    check(o, lse, q, k, v, cfg, mask, causal, nsplit, pv)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_block_sparse_invariants_bit_exact(pv):
    cfg = dict(B=1, Hq=2, Hkv=1, Lq=600, Lk=600, D=128, dtype="fp16", layout="HND")
    q, k, v, cfg = si.make_inputs(cfg, seed=77)
    s = Sparse(q, k, v, cfg, pv)
    nq, nk = -(-600 // 128), -(-600 // 128)
    ones = np.ones((1, 2, nq, nk), np.uint8)
    for nsplit in (1, 2):
        o0, l0 = s.run(None, 0, nsplit)
        o1, l1 = s.run(ones, 0, nsplit)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    tri = np.tril(np.ones((nq, nk), np.uint8))[None, None].repeat(2, axis=1)
    oc, lc = s.run(None, 1, 1)
    ot, lt = s.run(np.ascontiguousarray(tri), 1, 1)
    assert torch.equal(oc, ot) and torch.equal(lc, lt)
    # all blocks off: zero output, LSE -inf
    oz, lz = s.run(np.zeros_like(ones), 0, 1)
    assert not oz.any() and torch.isneginf(lz).all()


def test_block_sparse_full_size_sampled():
    # B2 H24 L4096 D128 fp16 with half of the blocks on, sampled heads and rows
    q, k, v, cfg = si.make_inputs("c3")
    mask = make_mask(cfg, 0.5, seed=3)
    s = Sparse(q, k, v, cfg, "fp8")
    o, lse = s.run(mask, 0, 1)
    qz = oracle.quantize(q, k, v)
    check(o, lse, q, k, v, cfg, mask, 0, 1, "fp8", heads=[(0, 0), (1, 23)], rows=(0, 64), qz=qz)
    check(o, lse, q, k, v, cfg, mask, 0, 1, "fp8", heads=[(1, 7)], rows=(4096 - 64, 4096), qz=qz)
    del s
    torch.cuda.empty_cache()


def test_block_mask_refusals():
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=200, Lk=300, D=64, dtype="fp16", layout="HND")
    q, k, v, cfg = si.make_inputs(cfg, seed=5)
    s = Sparse(q, k, v, cfg, "fp8")
    with pytest.raises(qa.SageError):                               # wrong shape
        s.run(np.ones((1, 2, 2, 2), np.uint8))
    o = torch.zeros_like(s.qd)
    with pytest.raises(qa.SageError) as e:                          # mask inside o
        lib = qa.lib()
        op = qa._opts(0, 0.125, 1, None, None)
        op.block_mask = o.data_ptr()
        qa._check(lib.sage_attn_quantized_ex(qa.ctypes.byref(s.p), qa._ptr(s.ws), s.ws.numel(), qa._ptr(o),
                                             qa.ctypes.byref(op), qa._stream()))
    assert e.value.status == qa.SAGE_E_INVALID
    torch.cuda.synchronize()
    assert not o.any()
