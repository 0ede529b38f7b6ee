"""GPU: the one-call path, whose attention kernel quantizes Q itself
(sage_attn / sage_attn_ex), against the two-call path (sage_quantize, then
sage_attn_quantized / sage_attn_quantized_ex); needs an MI355X.

Both compute each query's INT8 codes and scale by the same per-token rule
(s_q = amax / 127, codes rne(q * 127 / amax) clamped to +-127), so the bar is
bit for bit: output and LSE identical, and the K/V workspace sections
identical, while the one-call path leaves the Q sections unwritten. The
two-call path's Q codes are themselves checked against the oracle bit for bit
in test_gpu_parity. Every call goes through the C ABI.
"""
import math

import numpy as np
import pytest
import torch

import quantized_attention_sage_amd as qa
import sage_inputs as si

pytestmark = pytest.mark.gpu

TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def device_inputs(cfg, seed, pad_rows=0):
    """q, k, v on the device in cfg's layout. pad_rows > 0: q is a view into
    rows of D + pad_rows channels (a strided input)."""
    q, k, v, cfg = si.make_inputs(cfg, seed=seed)
    out = []
    for i, x in enumerate((q, k, v)):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(TDT[cfg["dtype"]])
        if cfg["layout"] == "NHD":
            t = t.permute(0, 2, 1, 3).contiguous()
        t = t.cuda()
        if i == 0 and pad_rows:
            big = torch.zeros(t.shape[:-1] + (t.shape[-1] + pad_rows,), dtype=t.dtype, device="cuda")
            big[..., :t.shape[-1]] = t
            t = big[..., :t.shape[-1]]
        out.append(t)
    return out, cfg


def run_both(cfg, seed, pv, causal=0, nsplit=1, with_lse=False, mask=None, pad_rows=0, fused=None):
    fused = fused if fused is not None else []
    (qd, kd, vd), cfg = device_inputs(cfg, seed, pad_rows)
    sm = 1.0 / math.sqrt(cfg["D"])
    res = []
    # two calls (sage_quantize, sage_attn_quantized_ex); one call (sage_attn_ex);
    # its two parts (sage_quantize_kv, sage_attn_q_ex); the fused-Q attention on
    # the two-call workspace
    for mode in ("two", "one", "parts", "q_on_full_ws"):
        o = torch.empty(qd.shape, dtype=qd.dtype, device="cuda")
        p = qa.make_problem(qd, kd, vd, o, cfg["layout"], pv=pv)
        ws = qa.new_workspace(p)
        ws.fill_(0x5A)
        lse = torch.empty((p.B, p.Hq, p.Lq), dtype=torch.float32, device="cuda") if with_lse else None
        md = torch.from_numpy(mask).cuda() if mask is not None else None
        kw = dict(is_causal=causal, sm_scale=sm, nsplit=nsplit, lse=lse, block_mask=md)
        if mode == "one":
            qa.attn_ex(p, qd, kd, vd, o, ws, **kw)
        elif mode == "parts":
            qa.quantize_kv(p, kd, vd, ws)
            qa.attn_q_ex(p, qd, ws, o, **kw)
        else:
            qa.quantize(p, qd, kd, vd, ws)
            if mode == "two":
                qa.attn_quantized_ex(p, ws, o, **kw)
            else:
                qa.attn_q_ex(p, qd, ws, o, **kw)
        torch.cuda.synchronize()
        res.append((mode, o, lse, ws))
    p_ = p
    _, o0, l0, ws0 = res[0]
    w0 = qa.workspace_views(p_, ws0)
    for mode, o1, l1, ws1 in res[1:]:
        assert torch.equal(o0, o1), (mode, (o0.float() - o1.float()).abs().max().item())
        if with_lse:
            assert torch.equal(l0, l1), mode
        w1 = qa.workspace_views(p_, ws1)
        for name in ("khat", "sk", "kbar", "vhat", "vmax"):
            assert torch.equal(w0[name], w1[name]), (mode, name)
        untouched = bool((w1["qhat"].view(torch.uint8) == 0x5A).all() and (w1["sq"].view(torch.uint8) == 0x5A).all())
        if mode == "parts":
            # the explicit fused-Q calls leave the Q sections as they were
            assert untouched, mode
        elif mode == "one":
            # the one-call path fuses Q when the launch needs more than one round
            # of workgroups or the K/V statistics need no launch of their own
            # (short fp16 heads); otherwise its prologue writes the Q codes
            if not untouched:
                Lq = w0["layout"].Lq_pad
                assert torch.equal(w0["qhat"][:, :, :Lq], w1["qhat"][:, :, :Lq])
                assert torch.equal(w0["sq"][:, :, :Lq], w1["sq"][:, :, :Lq])
            fused.append(untouched)
    return res[1][1]


CASES = [
    # name, shape, pv, causal, nsplit, lse, q row padding
    ("c1_fp8", "c1", "fp8", 0, 1, False, 0),
    ("c2c_fp16", "c2c", "fp16", 1, 1, True, 0),
    ("d80_bf16_nhd_ragged", dict(B=2, Hq=3, Hkv=3, Lq=300, Lk=777, D=80, dtype="bf16", layout="NHD"),
     "fp8", 0, 1, True, 0),
    ("d37_unaligned_pv16", dict(B=1, Hq=2, Hkv=1, Lq=150, Lk=400, D=37, dtype="fp16", layout="HND"),
     "fp16", 2, 1, True, 0),
    ("gqa_bottom_right_split3", dict(B=1, Hq=8, Hkv=2, Lq=200, Lk=900, D=128, dtype="fp16", layout="HND"),
     "fp8", 2, 3, True, 0),
    ("strided_q_rows", dict(B=1, Hq=4, Hkv=4, Lq=260, Lk=260, D=64, dtype="bf16", layout="HND"),
     "fp8", 1, 1, True, 8),
    ("strided_q_rows_unaligned", dict(B=1, Hq=2, Hkv=2, Lq=130, Lk=200, D=64, dtype="fp16", layout="HND"),
     "fp16", 0, 2, False, 3),
]


@pytest.mark.parametrize("name,cfg,pv,causal,nsplit,with_lse,pad", CASES, ids=[c[0] for c in CASES])
def test_fused_q_equals_two_calls(name, cfg, pv, causal, nsplit, with_lse, pad):
    run_both(cfg, 0x5A6E5000 + len(name), pv, causal, nsplit, with_lse, pad_rows=pad)


def test_fused_q_block_mask_split():
    cfg = dict(B=1, Hq=2, Hkv=2, Lq=384, Lk=640, D=128, dtype="fp16", layout="HND")
    rng = np.random.default_rng(11)
    mask = (rng.random((1, 2, 3, 5)) < 0.5).astype(np.uint8)
    mask[0, 1, 2] = 0                                 # a query block without keys
    run_both(cfg, 31, "fp8", 0, 2, True, mask=mask)


@pytest.mark.parametrize("name,pv,fuses", [("c3", "fp8", True), ("c3", "fp16", True), ("c4", "fp8", False),
                                           ("c2", "fp8", True)])
def test_fused_q_full_size(name, pv, fuses):
    # the benchmark shapes, whole outputs (c4 in the library's split); the
    # one-call path quantizes Q in the attention kernel at c3 (1536 tiles,
    # three rounds) and in the prologue at c4 (256 tiles x 2 key ranges = one
    # round of the 512 workgroup slots); at c2 (one round as well) the fp16
    # heads of 512 keys need no K/V statistics launch, so Q is fused there
    fused = []
    run_both(name, None, pv, 0, 0, True, fused=fused)
    assert fused == [fuses]
    torch.cuda.empty_cache()


def test_sageattn_uses_the_one_call_path():
    # sageattn() == sage_attn (one pass) through the C ABI, and == the two calls
    (qd, kd, vd), cfg = device_inputs("c2", 5)
    o = qa.sageattn(qd, kd, vd, nsplit=1)
    p = qa.make_problem(qd, kd, vd, None, "HND")
    ws = qa.new_workspace(p)
    o2 = torch.empty_like(qd)
    qa._check(qa.lib().sage_attn(qa.ctypes.byref(p), qa._ptr(qd), qa._ptr(kd), qa._ptr(vd), qa._ptr(o2), 0,
                                 1.0 / math.sqrt(cfg["D"]), 1, qa._ptr(ws), ws.numel(), qa._stream()))
    o3 = torch.empty_like(qd)
    qa.quantize(p, qd, kd, vd, ws)
    qa.attn_quantized(p, ws, o3)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(o, o3)
