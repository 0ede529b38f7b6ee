"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/sage_attn.h declares,
lay the workspace out as documented, and refuse every malformed call before
it touches the device (so these calls are safe without a GPU).
"""
import ctypes
import os
import re

import pytest

import quantized_attention_sage_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qa.LIB_PATH), reason="libsage_attn.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    L = qa.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qa.EXPORTED)


def test_status_strings():
    L = qa.lib()
    for s in range(5):
        assert L.sage_status_str(s)
    assert L.sage_status_str(99) == b"unknown status"


def _p(layout="HND", B=2, Hq=4, Hkv=2, Lq=100, Lk=300, D=80, dtype=None):
    import torch
    return qa.contiguous_problem(layout, B, Hq, Hkv, Lq, Lk, D, dtype or torch.float16)


def test_problem_init_strides():
    p = _p("HND")
    assert list(p.q_stride) == [4 * 100 * 80, 100 * 80, 80]
    assert list(p.k_stride) == [2 * 300 * 80, 300 * 80, 80]
    p = _p("NHD")
    assert list(p.q_stride) == [100 * 4 * 80, 80, 4 * 80]
    assert list(p.v_stride) == [300 * 2 * 80, 80, 2 * 80]


@pytest.mark.parametrize("kw,status", [
    (dict(D=129), qa.SAGE_E_UNSUPPORTED),
    (dict(D=0), qa.SAGE_E_INVALID),
    (dict(Hq=3, Hkv=2), qa.SAGE_E_INVALID),
    (dict(Lq=0), qa.SAGE_E_INVALID),
    (dict(Lk=0), qa.SAGE_E_INVALID),
    (dict(B=0), qa.SAGE_E_INVALID),
])
def test_problem_init_refusals(kw, status):
    with pytest.raises(qa.SageError) as ei:
        _p(**kw)
    assert ei.value.status == status
    assert qa.lib().sage_last_error()


def test_bad_dtype_and_layout():
    p = qa.Problem()
    st = qa.lib().sage_problem_init(ctypes.byref(p), 0, 1, 1, 1, 8, 8, 64, 7)
    assert st == qa.SAGE_E_INVALID and b"dtype" in qa.lib().sage_last_error()
    st = qa.lib().sage_problem_init(ctypes.byref(p), 5, 1, 1, 1, 8, 8, 64, 0)
    assert st == qa.SAGE_E_INVALID and b"layout" in qa.lib().sage_last_error()


def test_negative_and_overlapping_strides():
    p = _p()
    p.k_stride[2] = -80
    with pytest.raises(qa.SageError) as ei:
        qa.check_problem(p)
    assert ei.value.status == qa.SAGE_E_UNSUPPORTED
    p = _p()
    p.o_stride[2] = 40          # rows of 80 elements 40 apart overlap
    with pytest.raises(qa.SageError) as ei:
        qa.check_problem(p)
    assert ei.value.status == qa.SAGE_E_INVALID
    # fused qkv view (token stride 3*H*D) is accepted
    p = _p(Hq=4, Hkv=4)
    for s in (p.q_stride, p.k_stride, p.v_stride):
        s[0], s[1], s[2] = 100 * 3 * 4 * 80, 80, 3 * 4 * 80
    p.Lk = 100
    qa.check_problem(p)


def test_workspace_layout_arithmetic():
    p = _p(B=2, Hq=4, Hkv=2, Lq=100, Lk=300, D=80)
    L = qa.workspace_layout(p)
    assert (L.Dp, L.Lq_pad, L.Lk_pad, L.nkb, L.nchunk) == (128, 256, 384, 6, 2)
    offs = [L.qhat, L.sq, L.khat, L.sk, L.kbar, L.vhat, L.vmax, L.kpart, L.vpart]
    sizes = [2 * 4 * 256 * 128, 2 * 4 * 256 * 4, 2 * 2 * 384 * 128, 2 * 2 * 6 * 4,
             2 * 2 * 128 * 4, 2 * 2 * 6 * 128 * 64, 2 * 2 * 128 * 4, 2 * 2 * 2 * 128 * 8,
             2 * 2 * 2 * 128 * 4]
    assert offs[0] == 0
    for a, n, b in zip(offs, sizes, offs[1:] + [L.total_bytes]):
        assert a % 256 == 0
        assert b >= a + n and b - (a + n) < 256
    assert qa.workspace_bytes(p) == L.total_bytes
    assert qa.softmax_block_keys() == 128
    assert qa.softmax_spec("fp8") == (128, "lazy") and qa.softmax_spec("fp16") == (128, "max")
    assert qa.lib().sage_softmax_spec(7, None, None) == qa.SAGE_E_INVALID
    p64 = _p(D=64, Lq=1, Lk=1)
    L64 = qa.workspace_layout(p64)
    assert (L64.Dp, L64.Lq_pad, L64.Lk_pad, L64.nkb, L64.nchunk) == (64, 256, 128, 2, 1)


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_calls_refused_before_any_device_work():
    L = qa.lib()
    p = _p()
    need = qa.workspace_bytes(p)
    pp = ctypes.byref(p)
    q, k, v, o, ws = (_fake(0x10000000 * (i + 1)) for i in range(5))
    cases = [
        (L.sage_quantize(pp, None, k, v, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_quantize(pp, q, k, v, 1, None, need, None), qa.SAGE_E_WORKSPACE),
        (L.sage_quantize(pp, q, k, v, 1, _fake(0x50000010), need, None), qa.SAGE_E_WORKSPACE),
        (L.sage_quantize(pp, q, k, v, 1, ws, need - 1, None), qa.SAGE_E_WORKSPACE),
        (L.sage_quantize(pp, q, k, _fake(0x50000000 + 512), 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized(pp, ws, need, o, 0, 0.0, None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized(pp, ws, need, o, 0, float("nan"), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized(pp, ws, need, o, 0, float("inf"), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized(pp, ws, need, None, 0, 0.1, None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized(pp, ws, need, _fake(0x50000000 + 4096), 0, 0.1, None), qa.SAGE_E_INVALID),
        (L.sage_attn(pp, q, k, v, q, 0, 0.1, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_attn(pp, q, k, v, o, 0, -1.0, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_debug_qk_int32(pp, ws, need, 2, 0, o, None), qa.SAGE_E_INVALID),
        (L.sage_debug_qk_int32(pp, ws, need, 0, 4, o, None), qa.SAGE_E_INVALID),
        (L.sage_debug_qk_int32(pp, ws, need, 0, 0, None, None), qa.SAGE_E_INVALID),
        (L.sage_debug_qk_int32(pp, ws, 16, 0, 0, o, None), qa.SAGE_E_WORKSPACE),
    ]
    for n, (got, want) in enumerate(cases):
        assert got == want, (n, got, want, L.sage_last_error())
        assert L.sage_last_error(), n
    bad = _p()
    bad.D = 200
    assert L.sage_attn(ctypes.byref(bad), q, k, v, o, 0, 0.1, 1, ws, need, None) == qa.SAGE_E_UNSUPPORTED
    assert L.sage_workspace_bytes(ctypes.byref(bad)) == 0


def test_one_call_and_fused_q_entry_points_refused():
    # sage_attn_ex, sage_quantize_kv and sage_attn_q_ex validate everything
    # before any launch (the pointers here are never dereferenced)
    L = qa.lib()
    p = _p()
    need = qa.workspace_bytes(p)
    pp = ctypes.byref(p)
    q, k, v, o, ws = (_fake(0x10000000 * (i + 1)) for i in range(5))

    def op(**kw):
        x = qa._opts(0, kw.get("sm", 0.125), kw.get("nsplit", 1), None, None)
        x.is_causal = kw.get("causal", 0)           # raw value: the C side must refuse 3
        if "lse" in kw:
            x.lse = kw["lse"]
        return ctypes.byref(x)

    cases = [
        (L.sage_attn_ex(pp, None, k, v, o, 1, ws, need, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_ex(pp, q, k, v, o, 1, ws, need, None, None), qa.SAGE_E_INVALID),
        (L.sage_attn_ex(pp, q, k, v, o, 1, ws, need, op(causal=3), None), qa.SAGE_E_INVALID),
        (L.sage_attn_ex(pp, q, k, v, o, 1, ws, need, op(sm=float("nan")), None), qa.SAGE_E_INVALID),
        (L.sage_attn_ex(pp, q, k, v, o, 1, ws, need - 1, op(), None), qa.SAGE_E_WORKSPACE),
        (L.sage_attn_ex(pp, q, k, v, _fake(0x30000000 + 64), 1, ws, need, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_ex(pp, q, k, v, o, 1, _fake(0x10000000), need, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_ex(pp, q, k, v, o, 1, ws, need, op(lse=0x20000000), None), qa.SAGE_E_INVALID),
        (L.sage_quantize_kv(pp, None, v, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_quantize_kv(pp, k, v, 1, ws, need - 1, None), qa.SAGE_E_WORKSPACE),
        (L.sage_quantize_kv(pp, k, _fake(0x50000000 + 256), 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_attn_q_ex(pp, None, ws, need, o, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_q_ex(pp, q, ws, need, None, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_q_ex(pp, q, ws, need, o, op(nsplit=17), None), qa.SAGE_E_INVALID),
        (L.sage_attn_q_ex(pp, q, ws, need, _fake(0x10000000 + 128), op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_q_ex(pp, q, ws, need, _fake(0x50000000 + 4096), op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_q_ex(pp, q, ws, need, o, op(lse=0x10000000 + 16), None), qa.SAGE_E_INVALID),
    ]
    for n, (got, want) in enumerate(cases):
        assert got == want, (n, got, want, L.sage_last_error())
    bad = _p()
    bad.D = 200
    assert L.sage_attn_ex(ctypes.byref(bad), q, k, v, o, 1, ws, need, op(), None) == qa.SAGE_E_UNSUPPORTED


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(qa.SageError):
        qa.sageattn(x, x, x)


def test_pv_field_checked_and_sizes_16bit_v():
    import torch
    p8 = _p(B=2, Hq=4, Hkv=2, Lq=100, Lk=300, D=80)
    p16 = qa.contiguous_problem("HND", 2, 4, 2, 100, 300, 80, torch.bfloat16, pv="fp16")
    assert p8.pv == qa.SAGE_PV_FP8 and p16.pv == qa.SAGE_PV_FP16
    L8, L16 = qa.workspace_layout(p8), qa.workspace_layout(p16)
    # the 16-bit V^T section is twice the FP8 one; everything before it is unchanged
    assert (L16.qhat, L16.sq, L16.khat, L16.sk, L16.kbar, L16.vhat) == (L8.qhat, L8.sq, L8.khat, L8.sk, L8.kbar, L8.vhat)
    assert L16.vmax - L16.vhat == 2 * 2 * 6 * 128 * 64 * 2
    assert L16.total_bytes > L8.total_bytes
    bad = _p()
    bad.pv = 2
    with pytest.raises(qa.SageError) as ei:
        qa.check_problem(bad)
    assert ei.value.status == qa.SAGE_E_INVALID and b"pv" in qa.lib().sage_last_error()
    with pytest.raises(qa.SageError):
        qa.contiguous_problem("HND", 1, 1, 1, 8, 8, 64, torch.float16, pv="fp4")
    # 16-bit V^T positions: bits 2 and 3 of the token index swap (a permutation)
    pos = [qa.vhat_position(j, "fp16") for j in range(64)]
    assert sorted(pos) == list(range(64))
    assert pos[4] == 8 and pos[8] == 4 and pos[12] == 12 and pos[3] == 3


# ---------------------------------------------------------------------------
# Packed variable-length problems
# ---------------------------------------------------------------------------
def _vp(B=3, Hq=4, Hkv=2, tq=300, tk=500, mq=200, mk=300, D=80, dtype=0, pv=1):
    p = qa.VarlenProblem()
    st = qa.lib().sage_varlen_problem_init(ctypes.byref(p), B, Hq, Hkv, tq, tk, mq, mk, D, dtype, pv)
    return p, st


def test_varlen_problem_init_and_refusals():
    p, st = _vp()
    assert st == qa.SAGE_OK
    assert list(p.q_stride) == [4 * 80, 80] and list(p.k_stride) == [2 * 80, 80]
    for kw, status in [(dict(D=129), qa.SAGE_E_UNSUPPORTED), (dict(B=0), qa.SAGE_E_INVALID),
                       (dict(Hq=3), qa.SAGE_E_INVALID), (dict(tq=-1), qa.SAGE_E_INVALID),
                       (dict(mk=0), qa.SAGE_E_INVALID), (dict(pv=5), qa.SAGE_E_INVALID),
                       (dict(dtype=3), qa.SAGE_E_INVALID)]:
        _, st = _vp(**kw)
        assert st == status, (kw, st)
        assert qa.lib().sage_last_error()
    p, _ = _vp()
    p.o_stride[0] = 40                  # token rows of 4 heads x 80 overlap
    assert qa.lib().sage_varlen_problem_check(ctypes.byref(p)) == qa.SAGE_E_INVALID


def test_varlen_workspace_layout_holds_every_sequence():
    # The documented rule places sequence b's rows of head h at
    #   Q row   h*Lq_pad + cu_q[b] + 255 b      (its rows rounded up to 256)
    #   K block h*nkb    + (cu_k[b] + 127 b)//64 (its tokens rounded up to 128)
    #   chunk   h*nchunk + (cu_k[b] + 255 b)//256
    # For random lengths these ranges stay inside the per-head sizes the
    # library reports and never overlap.
    import random
    rng = random.Random(5)
    for _ in range(3000):
        B = rng.randint(1, 9)
        mx = rng.choice([1, 63, 64, 127, 128, 129, 256, 257, 700])
        lq = [rng.randint(0, mx) for _ in range(B)]
        lk = [rng.randint(0, mx) for _ in range(B)]
        cq = [0] + list(__import__("itertools").accumulate(lq))
        ck = [0] + list(__import__("itertools").accumulate(lk))
        p, st = _vp(B=B, Hq=2, Hkv=1, tq=cq[-1], tk=ck[-1], mq=max(1, mx), mk=max(1, mx), D=64, pv=0)
        assert st == qa.SAGE_OK
        L = qa.varlen_workspace_layout(p)
        ranges = {"q": [], "k": [], "c": []}
        for b in range(B):
            q0 = cq[b] + 255 * b
            ranges["q"].append((q0, q0 + -(-lq[b] // 256) * 256))
            k0 = (ck[b] + 127 * b) // 64
            ranges["k"].append((k0, k0 + 2 * -(-lk[b] // 128)))
            c0 = (ck[b] + 255 * b) // 256
            ranges["c"].append((c0, c0 + -(-lk[b] // 256)))
        for key, total in (("q", L.Lq_pad), ("k", L.nkb), ("c", L.nchunk)):
            r = [x for x in ranges[key] if x[1] > x[0]]
            assert all(0 <= a and e <= total for a, e in r), (key, r, total)
            assert all(r[i][1] <= r[i + 1][0] for i in range(len(r) - 1)), (key, r)
        assert L.Lk_pad == 64 * L.nkb
        offs = [L.qhat, L.sq, L.khat, L.sk, L.kbar, L.vhat, L.vmax, L.kpart, L.vpart, L.total_bytes]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs[:-1])
        assert L.sq - L.qhat >= 2 * L.Lq_pad * 64 and L.vmax - L.vhat >= 1 * L.nkb * 64 * 64
    assert qa.varlen_workspace_bytes(p) == L.total_bytes


def test_varlen_calls_refused_before_any_device_work():
    L = qa.lib()
    p, _ = _vp()
    need = qa.varlen_workspace_bytes(p)
    pp = ctypes.byref(p)
    q, k, v, o, ws, cq, ck = (_fake(0x10000000 * (i + 1)) for i in range(7))
    cases = [
        (L.sage_varlen_attn(pp, q, k, v, o, None, ck, 0, 0.1, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_varlen_attn(pp, q, k, v, o, cq, None, 0, 0.1, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_varlen_attn(pp, None, k, v, o, cq, ck, 0, 0.1, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_varlen_attn(pp, q, k, v, o, cq, ck, 0, 0.0, 1, ws, need, None), qa.SAGE_E_INVALID),
        (L.sage_varlen_attn(pp, q, k, v, o, cq, ck, 0, 0.1, 1, None, need, None), qa.SAGE_E_WORKSPACE),
        (L.sage_varlen_attn(pp, q, k, v, o, cq, ck, 0, 0.1, 1, ws, need - 1, None), qa.SAGE_E_WORKSPACE),
        (L.sage_varlen_attn(pp, q, k, v, o, cq, ck, 0, 0.1, 1, _fake(0x50000010), need, None), qa.SAGE_E_WORKSPACE),
        (L.sage_varlen_attn(pp, q, k, v, q, cq, ck, 0, 0.1, 1, ws, need, None), qa.SAGE_E_INVALID),
    ]
    for n, (got, want) in enumerate(cases):
        assert got == want, (n, got, want, L.sage_last_error())


def test_split_choice_and_scratch_sizes():
    # the library's split choice: ranges until the query tiles fill the 512
    # FP8 (256 16-bit) workgroup slots of the 256 compute units, at least
    # four 128-key blocks per range, at most 16 ranges
    L = qa.lib()
    cases = [  # (layout, B, Hq, Hkv, Lq, Lk, D, pv) -> count
        (("NHD", 1, 32, 8, 1024, 8192, 128, 0), 2),      # 256 FP8 tiles
        (("NHD", 1, 32, 8, 1024, 8192, 128, 1), 2),      # 128 16-bit tiles
        (("HND", 2, 24, 24, 4096, 4096, 128, 0), 1),     # 1536 tiles
        (("HND", 1, 16, 16, 512, 512, 64, 0), 1),        # 4 blocks: too short to split
        (("HND", 1, 32, 8, 16, 8192, 128, 0), 16),       # decode-like: 32 tiles
        (("HND", 1, 8, 8, 100, 1000, 64, 0), 2),         # 8 blocks -> at most 2 ranges
        (("HND", 1, 1, 1, 1, 1, 64, 0), 1),
    ]
    for (lay, B, Hq, Hkv, Lq, Lk, D, pv), want in cases:
        p = qa.Problem()
        assert L.sage_problem_init(ctypes.byref(p), {"HND": 0, "NHD": 1}[lay], B, Hq, Hkv, Lq, Lk, D, 0) == 0
        p.pv = pv
        assert L.sage_split_count(ctypes.byref(p)) == want, (lay, B, Hq, Lq, Lk, pv)
        lay_ = qa.WsLayout()
        assert L.sage_workspace_layout(ctypes.byref(p), ctypes.byref(lay_)) == 0
        rows = B * Hq * lay_.Lq_pad
        for S in (2, 5, 16):
            o_bytes = -(-S * rows * lay_.Dp * 2 // 256) * 256     # normalised rows, 16-bit
            ml_bytes = -(-S * rows * 8 // 256) * 256
            assert L.sage_split_bytes(ctypes.byref(p), S) == o_bytes + ml_bytes
        assert L.sage_split_bytes(ctypes.byref(p), 1) == 0
        assert L.sage_split_bytes(ctypes.byref(p), 0) == L.sage_split_bytes(ctypes.byref(p), want)
        assert L.sage_split_bytes(ctypes.byref(p), 17) == 0
        assert L.sage_split_bytes(ctypes.byref(p), -1) == 0
    bad = qa.Problem()
    assert L.sage_split_count(ctypes.byref(bad)) == 0


def test_split_calls_refused_before_any_device_work():
    L = qa.lib()
    p = _p(Lq=64, Lk=4000)
    need = qa.workspace_bytes(p)
    pp = ctypes.byref(p)
    ws, o = _fake(0x10000000), _fake(0x20000000)
    part_need = L.sage_split_bytes(pp, 4)

    def opts(**kw):
        op = qa.AttnOpts()
        op.is_causal, op.nsplit, op.sm_scale, op.reserved = 0, 4, 0.1, 0
        op.part, op.part_bytes = 0x30000000, part_need
        for key, val in kw.items():
            setattr(op, key, val)
        return ctypes.byref(op)

    cases = [
        (L.sage_attn_quantized_ex(pp, ws, need, o, None, None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(is_causal=3), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(is_causal=-1), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(nsplit=17), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(nsplit=-2), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(reserved=1), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(sm_scale=float("nan")), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(lse=0x40000002), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(lse=0x20000000), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(part=None), None), qa.SAGE_E_WORKSPACE),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(part=0x30000010), None), qa.SAGE_E_WORKSPACE),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(part_bytes=part_need - 1), None), qa.SAGE_E_WORKSPACE),
        (L.sage_attn_quantized_ex(pp, ws, need, o, opts(part=0x10000000 + 256), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized_ex(pp, ws, need - 1, o, opts(), None), qa.SAGE_E_WORKSPACE),
        (L.sage_attn_quantized_ex(pp, ws, need, None, opts(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_quantized(pp, ws, need, o, 3, 0.1, None), qa.SAGE_E_INVALID),
    ]
    for n, (got, want) in enumerate(cases):
        assert got == want, (n, got, want, L.sage_last_error())
        assert L.sage_last_error(), n
    vp, _ = _vp()
    vpp = ctypes.byref(vp)
    vneed = qa.varlen_workspace_bytes(vp)
    q, k, v, cq, ck = (_fake(0x50000000 + 0x1000000 * i) for i in range(5))
    vpart = L.sage_varlen_split_bytes(vpp, 3)
    op = qa.AttnOpts()
    op.is_causal, op.nsplit, op.sm_scale = 2, 3, 0.1
    op.part, op.part_bytes = 0x50000000, vpart                    # overlaps q
    assert L.sage_varlen_attn_ex(vpp, q, k, v, o, cq, ck, 1, ws, vneed, ctypes.byref(op), None) == qa.SAGE_E_INVALID
    op.part, op.lse = 0x30000000, 0x51000000                      # lse overlaps k
    assert L.sage_varlen_attn_ex(vpp, q, k, v, o, cq, ck, 1, ws, vneed, ctypes.byref(op), None) == qa.SAGE_E_INVALID
    op.lse, op.is_causal = None, 5
    assert L.sage_varlen_attn_ex(vpp, q, k, v, o, cq, ck, 1, ws, vneed, ctypes.byref(op), None) == qa.SAGE_E_INVALID
    assert L.sage_varlen_attn(vpp, q, k, v, o, cq, ck, 3, 0.1, 1, ws, vneed, None) == qa.SAGE_E_INVALID
    assert L.sage_varlen_split_count(vpp) >= 1


def test_block_mask_refusals_before_any_device_work():
    L = qa.lib()
    p = _p(Lq=300, Lk=500)
    need = qa.workspace_bytes(p)
    pp = ctypes.byref(p)
    ws, o = _fake(0x10000000), _fake(0x20000000)
    assert qa.block_mask_shape(p) == (2, 4, 3, 4)

    def run(mask, nsplit=1, part=None, part_bytes=0):
        op = qa.AttnOpts()
        op.is_causal, op.nsplit, op.sm_scale = 1, nsplit, 0.1
        op.block_mask, op.part, op.part_bytes = mask, part, part_bytes
        return L.sage_attn_quantized_ex(pp, ws, need, o, ctypes.byref(op), None)

    assert run(0x10000000 + 512) == qa.SAGE_E_INVALID               # inside the workspace
    assert run(0x20000000 + 64) == qa.SAGE_E_INVALID                # inside o
    assert run(0x30000000 + 100, nsplit=2, part=0x30000000,         # inside the split scratch
               part_bytes=L.sage_split_bytes(pp, 2)) == qa.SAGE_E_INVALID
    vp, _ = _vp()
    vneed = qa.varlen_workspace_bytes(vp)
    q, k, v, cq, ck = (_fake(0x50000000 + 0x1000000 * i) for i in range(5))
    op = qa.AttnOpts()
    op.nsplit, op.sm_scale, op.block_mask = 1, 0.1, 0x40000000
    assert L.sage_varlen_attn_ex(ctypes.byref(vp), q, k, v, o, cq, ck, 1, ws, vneed, ctypes.byref(op),
                                 None) == qa.SAGE_E_UNSUPPORTED


def test_noalloc_sizes_and_refusals_before_any_device_work():
    # sage_attn_noalloc keeps the workspace and split partials in a static
    # per-GPU array; every refusal below happens before any HIP call
    L = qa.lib()
    import torch
    c3 = qa.contiguous_problem("HND", 2, 24, 24, 4096, 4096, 128, torch.float16)
    c5 = qa.contiguous_problem("NHD", 1, 40, 40, 14040, 14040, 80, torch.bfloat16)
    need3 = qa.noalloc_bytes(c3, 1)
    assert need3 == -(-qa.workspace_bytes(c3) // 256) * 256
    assert need3 <= qa.NOALLOC_SCRATCH_BYTES
    assert qa.noalloc_bytes(c3, 2) == need3 + qa.split_bytes(c3, 2)
    assert qa.noalloc_bytes(c5, 1) > qa.NOALLOC_SCRATCH_BYTES
    bad = _p()
    bad.D = 200
    assert qa.noalloc_bytes(bad, 1) == 0
    q, k, v, o = (_fake(0x10000000 * (i + 1)) for i in range(4))

    def op(nsplit=1, part=None, part_bytes=0, causal=0):
        x = qa._opts(0, 0.125, nsplit, None, None)
        x.is_causal = causal
        x.part = part
        x.part_bytes = part_bytes
        return ctypes.byref(x)

    p = _p()
    pp = ctypes.byref(p)
    cases = [
        (L.sage_attn_noalloc(pp, None, k, v, o, 1, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_noalloc(pp, q, k, v, None, 1, op(), None), qa.SAGE_E_INVALID),
        (L.sage_attn_noalloc(pp, q, k, v, o, 1, None, None), qa.SAGE_E_INVALID),
        (L.sage_attn_noalloc(pp, q, k, v, o, 1, op(causal=3), None), qa.SAGE_E_INVALID),
        (L.sage_attn_noalloc(pp, q, k, v, o, 1, op(part=0x60000000, part_bytes=1 << 20), None),
         qa.SAGE_E_INVALID),
        (L.sage_attn_noalloc(pp, q, k, v, o, 1, op(part_bytes=256), None), qa.SAGE_E_INVALID),
        (L.sage_attn_noalloc(ctypes.byref(c5), q, k, v, o, 1, op(), None), qa.SAGE_E_WORKSPACE),
        (L.sage_attn_noalloc(ctypes.byref(bad), q, k, v, o, 1, op(), None), qa.SAGE_E_UNSUPPORTED),
    ]
    for n, (got, want) in enumerate(cases):
        assert got == want, (n, got, want, L.sage_last_error())
        assert L.sage_last_error(), n
    L.sage_attn_noalloc(ctypes.byref(c5), q, k, v, o, 1, op(), None)
    assert b"more than the" in L.sage_last_error()
