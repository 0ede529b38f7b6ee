"""GPU parity of packed variable-length calls (sageattn_varlen; needs an MI355X).

Each packed sequence is an attention problem of its own, so its output must
equal, bit for bit, the dense call on that sequence alone, and meet the
parity bar against the oracle run on that sequence alone (the oracle's
per-head functions composed sequence by sequence). A sequence without keys
gets zero rows. Every call goes through the C ABI.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_attention_sage_amd as qa
import sage_inputs as si

pytestmark = pytest.mark.gpu

TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def _make(cfg, lens, seed):
    """Per-sequence logical inputs [1, H, L, D] and their packed device tensors [total, H, D]."""
    seqs = []
    for n, (lq, lk) in enumerate(lens):
        c = dict(B=1, Hq=cfg["Hq"], Hkv=cfg["Hkv"], Lq=max(lq, 1), Lk=max(lk, 1), D=cfg["D"],
                 dtype=cfg["dtype"], kbias_var=cfg.get("kbias_var", 0.0))
        q, k, v, _ = si.make_inputs(c, seed=seed + 17 * n)
        seqs.append((q[:, :, :lq], k[:, :, :lk], v[:, :, :lk]))
    dt = TDT[cfg["dtype"]]
    pack = lambda xs: torch.from_numpy(np.ascontiguousarray(
        np.concatenate([x[0].transpose(1, 0, 2) for x in xs], axis=0))).to(dt).cuda()
    qp = pack([s[0] for s in seqs])
    kp = pack([s[1] for s in seqs])
    vp = pack([s[2] for s in seqs])
    cu = lambda ls: torch.tensor(np.concatenate([[0], np.cumsum(ls)]), dtype=torch.int32).cuda()
    return seqs, qp, kp, vp, cu([l[0] for l in lens]), cu([l[1] for l in lens])


CASES = [
    ("mixed_fp16_pv16", dict(Hq=4, Hkv=2, D=64, dtype="fp16"),
     [(100, 100), (1, 1), (300, 129), (128, 128), (0, 5), (7, 0), (257, 400)], False, "fp16"),
    ("mixed_bf16_fp8_causal", dict(Hq=6, Hkv=3, D=80, dtype="bf16", kbias_var=2.0),
     [(200, 200), (64, 64), (129, 129), (1, 1), (513, 513)], True, "fp8"),
    ("d128_fp8_long", dict(Hq=2, Hkv=2, D=128, dtype="fp16", kbias_var=4.0),
     [(1000, 1500), (37, 2000), (256, 256)], False, "fp8"),
    ("d128_bf16_pv16_causal", dict(Hq=4, Hkv=1, D=128, dtype="bf16"),
     [(333, 333), (90, 90), (1, 1), (640, 640)], True, "fp16"),
]


@pytest.mark.parametrize("name,cfg,lens,causal,pv", CASES, ids=[c[0] for c in CASES])
def test_varlen_equals_dense_per_sequence_and_oracle(name, cfg, lens, causal, pv):
    seqs, qp, kp, vp, cq, ck = _make(cfg, lens, seed=0x5A6E2000 + len(name))
    mq = max(l[0] for l in lens)
    mk = max(l[1] for l in lens)
    sm = 1.0 / math.sqrt(cfg["D"])
    o = qa.sageattn_varlen(qp, kp, vp, cq, ck, mq, mk, is_causal=causal, pv=pv, nsplit=1)
    assert torch.equal(o, qa.sageattn_varlen(qp, kp, vp, cq, ck, mq, mk, is_causal=causal, pv=pv, nsplit=1))
    torch.cuda.synchronize()
    ofs = 0
    for (lq, lk), (q, k, v) in zip(lens, seqs):
        got_t = o[ofs:ofs + lq]
        ofs += lq
        if lq == 0:
            continue
        if lk == 0:
            assert not got_t.any()
            continue
        # the dense call on this sequence alone (NHD views of the packed rows)
        nhd = lambda x: torch.from_numpy(np.ascontiguousarray(x[0].transpose(1, 0, 2))).to(got_t.dtype).cuda()[None]
        dense = qa.sageattn(nhd(q), nhd(k), nhd(v), tensor_layout="NHD", is_causal=causal, pv=pv, nsplit=1)
        assert torch.equal(got_t, dense[0]), (lq, lk)
        # parity against the oracle on this sequence alone
        got = got_t.float().permute(1, 0, 2).unsqueeze(0).cpu().double().numpy()
        qz = oracle.quantize(q, k, v)
        bk, pref = qa.softmax_spec(pv)
        if pv == "fp8":
            ref = oracle.attn_quantized(qz, sm, causal=causal, bk=bk, pref=pref)
        else:
            ref = oracle.attn_quantized_pv16(qz, v, sm, causal=causal, fmt=cfg["dtype"], bk=bk)
        ex = oracle.attn_exact(q, k, v, sm, causal=causal)
        got = got.reshape(ref.shape)
        assert np.abs(got - ref).max() <= 2e-2
        assert _cos(got, ref) >= 0.999
        assert _cos(got, ex) >= (0.999 if pv == "fp8" or lk < 8 else 0.9999)


def test_varlen_strided_views_and_smooth_off():
    # packed q, k, v as views into one fused [total, 3, H, D] projection
    cfg = dict(Hq=4, Hkv=4, D=64, dtype="fp16")
    lens = [(150, 150), (40, 40), (300, 300)]
    seqs, qp, kp, vp, cq, ck = _make(cfg, lens, seed=77)
    fused = torch.stack([qp, kp, vp], dim=1).contiguous()        # [total, 3, H, D]
    qv, kv_, vv = fused[:, 0], fused[:, 1], fused[:, 2]
    assert qv.stride(0) == 3 * 4 * 64
    for pv in ("fp8", "fp16"):
        o_view = qa.sageattn_varlen(qv, kv_, vv, cq, ck, 300, 300, pv=pv, smooth_k=False)
        o_copy = qa.sageattn_varlen(qp, kp, vp, cq, ck, 300, 300, pv=pv, smooth_k=False)
        assert torch.equal(o_view, o_copy)
        assert torch.isfinite(o_view.float()).all()


SPLIT_CASES = [
    ("bottom_right_fp8_3", dict(Hq=4, Hkv=2, D=64, dtype="fp16"),
     [(100, 300), (1, 1), (300, 129), (0, 5), (7, 0), (64, 900), (257, 400)], 2, "fp8", 3),
    ("top_left_pv16_5", dict(Hq=2, Hkv=1, D=128, dtype="bf16", kbias_var=2.0),
     [(333, 333), (90, 700), (1, 1), (640, 640)], 1, "fp16", 5),
    ("no_mask_pv16_auto", dict(Hq=4, Hkv=4, D=80, dtype="bf16"),
     [(50, 2000), (20, 1500), (128, 128)], 0, "fp16", 0),
]


@pytest.mark.parametrize("name,cfg,lens,causal,pv,nsplit", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_varlen_split_lse_equals_dense_per_sequence(name, cfg, lens, causal, pv, nsplit):
    # packed call with key ranges, an LSE and per-sequence causal alignment:
    # every sequence equals, bit for bit, the dense call on it alone with the
    # same range count, and meets the bar against the oracle's split scheme
    seqs, qp, kp, vp, cq, ck = _make(cfg, lens, seed=0x5A6E3000 + len(name))
    mq = max(l[0] for l in lens)
    mk = max(l[1] for l in lens)
    sm = 1.0 / math.sqrt(cfg["D"])
    o, lse = qa.sageattn_varlen(qp, kp, vp, cq, ck, mq, mk, is_causal=causal, pv=pv, nsplit=nsplit,
                                return_lse=True)
    if nsplit == 0:
        op = torch.empty_like(qp)
        nsplit = qa.varlen_split_count(qa.make_varlen_problem(qp, kp, vp, op, len(lens), mq, mk, pv=pv))
        assert nsplit > 1
    torch.cuda.synchronize()
    assert lse.shape == (cfg["Hq"], qp.shape[0])
    ofs = 0
    for (lq, lk), (q, k, v) in zip(lens, seqs):
        got_t, got_l = o[ofs:ofs + lq], lse[:, ofs:ofs + lq]
        ofs += lq
        if lq == 0:
            continue
        if lk == 0:
            assert not got_t.any()
            assert torch.isneginf(got_l).all()
            continue
        nhd = lambda x: torch.from_numpy(np.ascontiguousarray(x[0].transpose(1, 0, 2))).to(got_t.dtype).cuda()[None]
        dense, dl = qa.sageattn(nhd(q), nhd(k), nhd(v), tensor_layout="NHD", is_causal=causal, pv=pv,
                                nsplit=nsplit, return_lse=True)
        assert torch.equal(got_t, dense[0]), (lq, lk)
        assert torch.equal(got_l, dl[0]), (lq, lk)
        qz = oracle.quantize(q, k, v)
        bk, pref = qa.softmax_spec(pv)
        ref, ref_l = oracle.attn_general(qz, sm, v=v, pv=pv, fmt=cfg["dtype"], causal=causal, nsplit=nsplit,
                                         bk=bk, pref=pref)
        got = got_t.float().permute(1, 0, 2).unsqueeze(0).cpu().double().numpy().reshape(ref.shape)
        gl = got_l.cpu().double().numpy().reshape(ref_l.shape)
        empty = ~np.isfinite(ref_l)
        assert np.array_equal(np.isneginf(gl), empty)
        assert np.all(got[empty] == 0.0)
        if (~empty).any():
            assert np.abs(gl[~empty] - ref_l[~empty]).max() <= 1e-2
            assert np.abs(got - ref).max() <= 2e-2
            assert _cos(got, ref) >= 0.999


# A packed call whose launch needs more than one round of workgroups, so the
# one-call path quantizes Q inside the attention kernel (from the packed q rows
# at each sequence's offset) instead of in the prologue: 24 heads, 8192 query
# tokens in sequences of mixed lengths. The packed grid has
# (total_q / 128 + B) * Hq query tiles of 128 rows, against 512 resident FP8
# workgroups (256 compute units x 2) or 256 of 256 rows for the 16-bit P.V.
FUSED_LENS = [3000, 2000, 1200, 900, 500, 300, 200, 92]
FUSED_CASES = [
    ("fp16_fp8_gqa", dict(Hq=24, Hkv=8, D=128, dtype="fp16", kbias_var=4.0), False, "fp8"),
    ("bf16_pv16_d80_causal", dict(Hq=24, Hkv=24, D=80, dtype="bf16", kbias_var=2.0), True, "fp16"),
]


@pytest.mark.parametrize("name,cfg,causal,pv", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_varlen_fused_q_many_tiles(name, cfg, causal, pv):
    lens = [(n, n) for n in FUSED_LENS]
    tiles = (sum(FUSED_LENS) // 128 + len(lens)) * cfg["Hq"]
    rows_per_wg, slots = (128, 512) if pv == "fp8" else (256, 256)
    assert tiles * 128 // rows_per_wg > slots          # more than one round: Q is coded in the kernel
    seqs, qp, kp, vp, cq, ck = _make(cfg, lens, seed=0x5A6E4000 + len(name))
    mq = mk = max(FUSED_LENS)
    sm = 1.0 / math.sqrt(cfg["D"])
    o = qa.sageattn_varlen(qp, kp, vp, cq, ck, mq, mk, is_causal=causal, pv=pv, nsplit=1)
    torch.cuda.synchronize()
    ofs = 0
    heads = [(0, 0), (0, cfg["Hq"] // 2 + 1), (0, cfg["Hq"] - 1)]
    for (lq, lk), (q, k, v) in zip(lens, seqs):
        got_t = o[ofs:ofs + lq]
        ofs += lq
        # bit for bit against the dense call on this sequence alone
        nhd = lambda x: torch.from_numpy(np.ascontiguousarray(x[0].transpose(1, 0, 2))).to(got_t.dtype).cuda()[None]
        dense = qa.sageattn(nhd(q), nhd(k), nhd(v), tensor_layout="NHD", is_causal=causal, pv=pv, nsplit=1)
        assert torch.equal(got_t, dense[0]), (lq, lk)
        # against the oracle on three heads, first and last rows of the sequence
        qz = oracle.quantize(q, k, v)
        bk, pref = qa.softmax_spec(pv)
        got = got_t.float().permute(1, 0, 2).cpu().double().numpy()
        for rows in ((0, min(lq, 48)), (max(lq - 48, 0), lq)):
            if pv == "fp8":
                ref = oracle.attn_quantized(qz, sm, causal=causal, bk=bk, pref=pref, heads=heads, rows=rows)
            else:
                ref = oracle.attn_quantized_pv16(qz, v, sm, causal=causal, fmt=cfg["dtype"], bk=bk,
                                                 heads=heads, rows=rows)
            ex = oracle.attn_exact(q, k, v, sm, causal=causal, heads=heads, rows=rows)
            g = np.stack([got[h, rows[0]:rows[1]] for (_, h) in heads])
            assert np.abs(g - ref).max() <= 2e-2, (lq, rows)
            assert _cos(g, ref) >= 0.999
            assert _cos(g, ex) >= (0.999 if pv == "fp8" else 0.9999)
