"""CPU: the host-side arithmetic of bench.py — the rocprofv3 summaries it
writes into profiles/, the traffic figure it reads back, and the algorithmic
byte counts of the roofline — on small synthetic CSV files."""
import csv
import io
import os
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ATTN = "void sage::(anonymous namespace)::attn_kernel<128, __half, false, true, false, false, false>(sage::AttnArgs)"
ATTN16 = "void sage::(anonymous namespace)::attn_kernel<128, __half, false, true, true, false, false>(sage::AttnArgs)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>(int)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counters(d, values):
    """values: {(dispatch, kernel): {counter: [per-instance values]}}"""
    rows = []
    for (disp, kern), cs in values.items():
        for c, vs in cs.items():
            for v in vs:
                rows.append(dict(Dispatch_Id=disp, Kernel_Name=kern, Counter_Name=c, Counter_Value=v))
    _write(os.path.join(d, "run", "run_counter_collection.csv"), rows)


def _summary(*args):
    out = io.StringIO()
    with redirect_stdout(out):
        bench.summarize(*args)
    return out.getvalue()


def test_counter_summary_and_mfma_busy_fraction(tmp_path):
    d = str(tmp_path / "pmc")
    # two dispatches; counters reported per instance (summed per dispatch)
    _counters(d, {
        (1, ATTN): {"SQ_VALU_MFMA_BUSY_CYCLES": [100.0e6, 126.5e6], "GRBM_GUI_ACTIVE": [600000.0] * 8,
                    "SQ_INSTS_MFMA": [5111808.0]},
        (2, ATTN): {"SQ_VALU_MFMA_BUSY_CYCLES": [226.5e6], "GRBM_GUI_ACTIVE": [4800000.0],
                    "SQ_INSTS_MFMA": [5111808.0]},
    })
    text = _summary("counters", d)
    kv = dict(l.split(": ") for l in text.splitlines() if not l.startswith("#"))
    assert float(kv["attn_gpu_active_cycles_per_xcd"]) == pytest.approx(600000.0)
    assert float(kv["attn_mfma_busy_frac"]) == pytest.approx(226.5e6 / (600000.0 * 256 * 4), abs=1e-4)
    assert float(kv["attn_mfma_insts"]) == 5111808.0
    assert "(n = 2)" in text


def test_traffic_summary_and_recorded_traffic(tmp_path, monkeypatch):
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    copy_kib = bench.COPY_BYTES / 1024.0
    # the copy's FETCH_SIZE counts half of what it reads; WRITE_SIZE counts all
    _counters(fd, {(1, ATTN): {"FETCH_SIZE": [30000.0, 7000.0]}, (2, ATTN16): {"FETCH_SIZE": [50000.0]},
                   (3, NEG): {"FETCH_SIZE": [copy_kib / 2]}})
    _counters(wd, {(1, ATTN): {"WRITE_SIZE": [49152.0]}, (2, ATTN16): {"WRITE_SIZE": [49152.0]},
                   (3, NEG): {"WRITE_SIZE": [copy_kib]}})
    text = _summary("traffic", fd, wd)
    kv = dict(l.split(": ") for l in text.splitlines() if not l.startswith("#"))
    assert float(kv["attn_fetch_kib"]) == 37000.0
    assert float(kv["attn16_fetch_kib"]) == 50000.0
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert kv["kernel_source_sha256_16"] == bench.kernel_source_hash()
    tf = tmp_path / "traffic.txt"
    tf.write_text(text)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.recorded_traffic() == pytest.approx((2 * 37000.0 + 49152.0) * 1024)
    assert bench.recorded_traffic("attn16") == pytest.approx((2 * 50000.0 + 49152.0) * 1024)
    # a summary taken on another kernel source is not used
    tf.write_text(text.replace(bench.kernel_source_hash(), "0" * 16))
    assert bench.recorded_traffic() is None


def test_stats_summary_columns(tmp_path):
    d = str(tmp_path / "trace")
    _write(os.path.join(d, "run", "run_kernel_stats.csv"),
           [dict(Name=ATTN, Calls=25, AverageNs=270000.0, MinNs=260000.0, MaxNs=330000.0, Percentage=80.0)])
    # 25 dispatches: 5 slow ones first, then 20 at 265 us
    trace = [dict(Kernel_Name=ATTN, Start_Timestamp=1000000 * i, End_Timestamp=1000000 * i + (330000 if i < 5 else 265000))
             for i in range(25)]
    _write(os.path.join(d, "run", "run_kernel_trace.csv"), trace)
    line = [l for l in _summary("stats", d).splitlines() if "attn_kernel" in l][0]
    cols = line.split()
    # calls, avg, median, last20, min, max, pct
    assert cols[-7:] == ["25", "270.00", "265.00", "265.00", "260.00", "330.00", "80.00"]
    assert line.startswith("sage::attn_kernel<128, __half, false, true, false, false, false>")


def test_algorithmic_bytes_of_the_step():
    cfg = dict(B=2, Hq=24, Hkv=24, Lq=4096, Lk=4096, D=128)

    class L:
        Dp = 128
    pro, main = bench.algorithmic_bytes(cfg, L, vb=1)
    kv_codes = 2 * 24 * 4096 * 2 * 128 + 2 * 24 * (4096 // 64 + 1) * 4
    assert pro == 2 * 128 * 2 * 2 * 24 * 4096 + kv_codes            # k, v read; codes written
    assert main == 2 * (2 * 2 * 24 * 4096 * 128) + kv_codes         # q read, o written, codes read
    assert main == 151007424
    _, main16 = bench.algorithmic_bytes(cfg, L, vb=2)
    assert main16 - main == 2 * 24 * 4096 * 128                      # 16-bit V^T


def test_fp64_reference_and_accuracy_figures():
    # the bench's float64 attention (plain numpy) against the oracle's exact
    # attention, with and without a causal mask, and the accuracy figures of
    # a known perturbation: a constant offset eps on every output gives
    # max-abs eps and rel_l2 eps * sqrt(n) / ||ref|| (up to the fp32 copy the
    # accuracy routine reads the output through)
    import math
    import numpy as np
    import torch
    import oracle
    import sage_inputs as si
    cfg = dict(B=1, Hq=4, Hkv=2, Lq=200, Lk=300, D=40, dtype="fp16", layout="HND", causal=False)
    q, k, v, cfg = si.make_inputs(cfg, seed=91)
    sm = 1.0 / math.sqrt(cfg["D"])
    for causal in (False, True):
        ex = oracle.attn_exact(q, k, v, sm, causal=causal).reshape(cfg["B"], cfg["Hq"], cfg["Lq"], cfg["D"])
        got = np.stack([np.stack([bench.fp64_attention(q, k, v, sm, causal, b, h, 2, 0, cfg["Lq"])
                                  for h in range(cfg["Hq"])]) for b in range(cfg["B"])])
        assert np.abs(got - ex).max() < 1e-12
    ex = np.stack([np.stack([bench.fp64_attention(q, k, v, sm, False, 0, h, 2, 0, cfg["Lq"])
                             for h in range(cfg["Hq"])])])
    eps = 1e-3
    acc = bench.accuracy(torch.from_numpy(ex + eps), q, k, v, cfg, sm, False)
    wins = bench.strided_windows(cfg["Lq"])
    rows = np.concatenate([np.arange(a, b) for a, b in wins])
    sel = ex[:, :, rows]
    assert abs(acc["max_abs"] - eps) < 1e-6
    assert abs(acc["rel_l2"] / (eps * math.sqrt(sel.size) / np.linalg.norm(sel)) - 1.0) < 1e-3
    assert acc["cos"] > 0.999 and "4 heads" in acc["rows"]
    assert wins[-1][1] == cfg["Lq"] and all(b - a == 16 for a, b in wins)
