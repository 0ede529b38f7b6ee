"""GPU: the allocation-free entry point (sage_attn_noalloc) against the one-call
path with a caller-allocated workspace (sage_attn_ex); needs an MI355X.

Both run the same launches on the same quantized sections, so the bar is bit
for bit on the output and the LSE. Two calls in a row share the library's
static scratch, the second on a smaller problem (with key ranges, whose
partials also live in the scratch), and a third repeats the first, so stale
contents of a larger call cannot leak into a smaller one or back. Every call
goes through the C ABI.
"""
import math

import numpy as np
import pytest
import torch

import quantized_attention_sage_amd as qa
import sage_inputs as si

pytestmark = pytest.mark.gpu

TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _device_inputs(cfg, seed):
    q, k, v, cfg = si.make_inputs(cfg, seed=seed)
    out = []
    for x in (q, k, v):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(TDT[cfg["dtype"]])
        if cfg["layout"] == "NHD":
            t = t.permute(0, 2, 1, 3).contiguous()
        out.append(t.cuda())
    return out, cfg


def _both(cfg, seed, causal, nsplit, pv="fp8"):
    print("noalloc case:", cfg if isinstance(cfg, str) else dict(cfg), "seed", seed, "causal", causal,
          "nsplit", nsplit, "pv", pv, flush=True)
    (qd, kd, vd), cfg = _device_inputs(cfg, seed)
    sm = 1.0 / math.sqrt(cfg["D"])
    res = []
    for mode in ("ws", "noalloc"):
        o = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device="cuda")
        p = qa.make_problem(qd, kd, vd, o, cfg["layout"], pv=pv)
        lse = torch.full((p.B, p.Hq, p.Lq), float("nan"), dtype=torch.float32, device="cuda")
        kw = dict(is_causal=causal, sm_scale=sm, nsplit=nsplit, lse=lse)
        if mode == "ws":
            ws = qa.new_workspace(p)
            qa.attn_ex(p, qd, kd, vd, o, ws, **kw)
        else:
            assert qa.noalloc_bytes(p, nsplit) <= qa.NOALLOC_SCRATCH_BYTES
            qa.attn_noalloc(p, qd, kd, vd, o, **kw)
        torch.cuda.synchronize()
        res.append((o, lse))
    (o0, l0), (o1, l1) = res
    assert torch.isfinite(o0.float()).all()
    assert torch.equal(o0, o1), (o0.float() - o1.float()).abs().max().item()
    assert torch.equal(torch.nan_to_num(l0, neginf=-1e30), torch.nan_to_num(l1, neginf=-1e30))
    return o1


def test_noalloc_equals_workspace_call_twice_then_smaller():
    big = dict(B=2, Hq=24, Hkv=24, Lq=4096, Lk=4096, D=128, dtype="fp16", layout="HND", kbias_var=4.0)
    small = dict(B=1, Hq=4, Hkv=2, Lq=300, Lk=700, D=80, dtype="bf16", layout="NHD", kbias_var=2.0)
    first = _both(big, 0x5A6E0003, causal=0, nsplit=1)
    _both(small, 11, causal=2, nsplit=3)
    _both(small, 12, causal=1, nsplit=1, pv="fp16")
    again = _both(big, 0x5A6E0003, causal=0, nsplit=1)
    assert torch.equal(first, again)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    c5 = qa.contiguous_problem("NHD", 1, 40, 40, 14040, 14040, 80, torch.bfloat16)
    x = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qa.SageError) as e:
        qa.attn_noalloc(c5, x, x, x, x)
    assert e.value.status == qa.SAGE_E_WORKSPACE
