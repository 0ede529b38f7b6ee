"""Benchmark of the quantized-attention hot path on one MI355X.

One step = the whole path on one batch, as sage_attn_ex runs it, in its two
calls so that each can be timed: the K/V prologue (sage_quantize_kv: key
mean, smoothed INT8 K, FP8 V) followed by the attention kernel
(sage_attn_q_ex: INT8 Q codes computed in the kernel, INT8 QK^T, online
softmax, FP8 P.V, with the key split count the library picks for the shape --
1 at the default workload), enqueued through the C ABI on torch's current
stream, inputs already resident in HBM.

Workload (default): B=2 H=24 Lq=Lk=4096 D=128 fp16 HND, q, v ~ N(0,1),
k ~ N(0,1) plus a per-(head, channel) bias ~ N(0, 4), non-causal, smooth_k on.
The metric is attention TOPS = 4*B*H*Lq*Lk*D / time. ``value`` uses the whole
step; the attention kernel's own rate (the figure the pages quote, which leaves
quantization out) is reported as ``main_kernel_tops`` and in ``roofline``.

Prints one JSON line. Timings come from HIP events recorded on the launch
stream around every kernel group inside the timed region. Before the warm-up
steps, steps run untimed for --settle-s seconds: from idle the GPU needs a few
tens of milliseconds of load before its clock is at the sustained level, and
a handful of warm-up steps (~2 ms) would otherwise time the ramp.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TOPS = 5000.0      # MI355X dense int8 / fp8 matrix peak (5.0 POP/s)
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16 / bf16 matrix peak (2.5 PFLOP/s)
# The 16-bit-PV variant does half of its 4*B*H*Lq*Lk*D operations (QK^T) in
# int8 and half (P.V) in fp16/bf16: at both peaks the launch takes
# 2N/5000 + 2N/2500, so its peak in the metric's unit is 4 / (2/5000 + 2/2500).
PEAK_PV16_TOPS = 4.0 / (2.0 / PEAK_MFMA_TOPS + 2.0 / PEAK_F16_TFLOPS)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up, so the GPU clock "
                         "reaches its sustained level before anything is timed")
    ap.add_argument("--config", default="c3")
    ap.add_argument("--rotate", type=int, default=3,
                    help="input copies cycled through so the prologue reads HBM, not cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="time the default path only (same as --variants none)")
    ap.add_argument("--variants", choices=("all", "pv16", "none"), default="all",
                    help="extra timings: all (16-bit-PV variant, packed sequences, grouped-query "
                         "long-key shape), pv16 (the 16-bit-PV variant only) or none")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows per head in the CPU-oracle sample")
    ap.add_argument("--cpu-heads", type=int, default=12)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the run, launch plain device copies of known size so that "
                         "a counter run can scale FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="condense rocprofv3 CSV output into a text summary on stdout, then "
                         "exit: 'stats DIR' (kernel trace statistics), 'traffic FETCH_DIR "
                         "WRITE_DIR' (FETCH_SIZE and WRITE_SIZE runs with --copy-calibration) "
                         "or 'counters DIR' (per-kernel means of any --pmc counters)")
    return ap.parse_args()


COPY_BYTES = 256 << 20      # size of the calibration copy


def settle(fn, seconds):
    """Run fn() untimed for about `seconds` of wall time (synchronizing every
    few calls), so that what follows runs at the sustained GPU clock."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


MAIN_KERNEL = "attn_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_c3_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_kernel_c3_mfma_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_attention_sage_amd", "csrc", f)
                  for f in ("attn_kernel.h", "attn_fp8.hip", "sage_kernels.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, directory))
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "").strip()
    return name.split("(")[0]


def _name_key(name):
    """Short kernel name; torch's elementwise kernels keep their functor name."""
    short = _short(name)
    if short.startswith("at::native::"):
        for tag in ("neg", "copy", "fill"):
            if tag in name:
                return short.split("<")[0] + "[" + tag + "]"
    return short


class HipEvents:
    """HIP events recorded on a given stream (hipEventRecord on the launch stream).

    Created with hipEventDisableSystemFence: the marker then carries no
    system-scope release, so the time between two markers around a kernel is
    the kernel's own span rather than the span plus a host-visible cache
    flush. torch's runtime and this library share the one HIP runtime
    (libamdhip64.so.7), so torch's stream handle is valid here.
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, stream_handle):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream_handle)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._ok(self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE))
            self.ev.append(e)

    @staticmethod
    def _ok(st):
        if st != 0:
            raise RuntimeError("HIP event call failed with status %d" % st)

    def record(self, i):
        self._ok(self.hip.hipEventRecord(self.ev[i], self.stream))

    def elapsed_ms(self, i, j):
        ms = self.ct.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j]))
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def _per_dispatch(directory, counter):
    """Mean of one counter per dispatch, per kernel name, in dispatch order."""
    import collections
    per = collections.defaultdict(float)
    names = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
            names[int(r["Dispatch_Id"])] = _name_key(r["Kernel_Name"])
    by = collections.OrderedDict()
    for d in sorted(per):
        by.setdefault(names[d], []).append(per[d])
    return {n: (len(v), sum(v) / len(v)) for n, v in by.items()}


def summarize(kind, *dirs):
    """Text summary of rocprofv3 CSV output (kernel statistics or HBM traffic)."""
    lines = []
    if kind == "stats":
        import collections
        import statistics
        rows = _csv_rows(dirs[0], "kernel_stats.csv")
        # per-dispatch durations from the trace, for the median and the mean of
        # the last 20 dispatches of each kernel (the timed steps come last)
        dur = collections.defaultdict(list)
        for r in _csv_rows(dirs[0], "kernel_trace.csv"):
            dur[_name_key(r["Kernel_Name"])].append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        lines.append("%-66s %6s %10s %10s %10s %10s %10s %7s" % ("kernel", "calls", "avg_us", "median_us",
                                                               "last20_us", "min_us", "max_us", "pct"))
        for r in rows:
            n = _name_key(r["Name"])
            d = [x for _, x in sorted(dur.get(n, []))]
            med = statistics.median(d) if d else float("nan")
            last = sum(d[-20:]) / len(d[-20:]) if d else float("nan")
            lines.append("%-66s %6d %10.2f %10.2f %10.2f %10.2f %10.2f %7.2f" % (
                n[:66], int(r["Calls"]), float(r["AverageNs"]) / 1e3, med, last,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    elif kind == "traffic":
        fetch = _per_dispatch(dirs[0], "FETCH_SIZE")
        write = _per_dispatch(dirs[1], "WRITE_SIZE")
        # the calibration copy is torch's negation kernel launched after the run
        copy = [n for n in fetch if "neg" in n.lower()]
        lines.append("# KiB per dispatch, mean over dispatches (n); copy = plain device copy "
                     "of %d bytes" % COPY_BYTES)
        lines.append("# %-66s %4s %14s %14s" % ("kernel", "n", "FETCH_SIZE", "WRITE_SIZE"))
        for n in fetch:
            lines.append("# %-66s %4d %14.1f %14.1f" % (n[:66], fetch[n][0], fetch[n][1],
                                                         write.get(n, (0, float("nan")))[1]))
        # attention kernels <Dp, dtype, causal, vectorized output, 16-bit P.V, block-sparse,
        # normaliser channel>: the dense ones of each P.V format
        def targs(n):
            return [x.strip() for x in n.split("<", 1)[1].rstrip(">").split(",")] if "<" in n else []
        attn = [n for n in fetch if n.startswith("sage::" + MAIN_KERNEL + "<")]
        main = [n for n in attn if targs(n)[4:6] == ["false", "false"]]
        main16 = [n for n in attn if targs(n)[4:6] == ["true", "false"]]
        if main and copy:
            c = copy[-1]
            lines.append("kernel_source_sha256_16: %s" % kernel_source_hash())
            lines.append("attn_fetch_kib: %.1f" % fetch[main[0]][1])
            lines.append("attn_write_kib: %.1f" % write[main[0]][1])
            if main16:
                lines.append("attn16_fetch_kib: %.1f" % fetch[main16[0]][1])
                lines.append("attn16_write_kib: %.1f" % write[main16[0]][1])
            lines.append("copy_fetch_kib: %.1f" % fetch[c][1])
            lines.append("copy_write_kib: %.1f" % write[c][1])
            lines.append("fetch_scale: %.4f" % (COPY_BYTES / 1024.0 / fetch[c][1]))
            lines.append("write_scale: %.4f" % (COPY_BYTES / 1024.0 / write[c][1]))
    elif kind == "counters":
        import collections
        names = sorted({r["Counter_Name"] for r in _csv_rows(dirs[0], "counter_collection.csv")})
        per = {c: _per_dispatch(dirs[0], c) for c in names}
        kernels = list(collections.OrderedDict.fromkeys(k for c in names for k in per[c]))
        lines.append("# per-dispatch means over the dispatches (n) of each kernel")
        for k in kernels:
            n = max(per[c].get(k, (0, 0))[0] for c in names)
            lines.append("# %s  (n = %d)" % (k, n))
            for c in names:
                if k in per[c]:
                    lines.append("#   %-28s %18.1f" % (c, per[c][k][1]))
        # the dense FP8 attention kernel: matrix-core busy fraction, taking
        # SQ_VALU_MFMA_BUSY_CYCLES as summed over all SIMDs and GRBM_GUI_ACTIVE
        # as summed over the 8 XCDs
        main = [k for k in kernels if k.startswith("sage::" + MAIN_KERNEL + "<") and
                [x.strip() for x in k.split("<", 1)[1].rstrip(">").split(",")][4:6] == ["false", "false"]]
        if main and "SQ_VALU_MFMA_BUSY_CYCLES" in per and "GRBM_GUI_ACTIVE" in per:
            busy = per["SQ_VALU_MFMA_BUSY_CYCLES"][main[0]][1]
            act = per["GRBM_GUI_ACTIVE"][main[0]][1] / 8.0
            lines.append("kernel_source_sha256_16: %s" % kernel_source_hash())
            lines.append("attn_gpu_active_cycles_per_xcd: %.0f" % act)
            lines.append("attn_mfma_busy_frac: %.4f" % (busy / (act * 256 * 4)))
            if "SQ_INSTS_MFMA" in per:
                lines.append("attn_mfma_insts: %.0f" % per["SQ_INSTS_MFMA"][main[0]][1])
    else:
        raise SystemExit("unknown summary kind %r" % kind)
    print("\n".join(lines))


def recorded_traffic(prefix="attn"):
    """HBM bytes per attention launch from the committed counter summary, or None.

    The summary holds FETCH_SIZE and WRITE_SIZE for the attention kernel (prefix
    "attn": FP8 P.V, "attn16": 16-bit P.V) and for a plain copy of COPY_BYTES,
    and the hash of the kernel source they were taken on; a changed kernel makes
    the figure stale, and then it is not reported.
    """
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        f_k, w_k = float(kv[prefix + "_fetch_kib"]), float(kv[prefix + "_write_kib"])
        f_c, w_c = float(kv["copy_fetch_kib"]), float(kv["copy_write_kib"])
        copy_kib = COPY_BYTES / 1024.0
        return f_k * copy_kib / f_c * 1024 + w_k * copy_kib / w_c * 1024
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_bytes(cfg, L, vb=1):
    """Bytes each launch group of a step must move at least once (see the design
    notes); vb is the size of a V^T element (1 for FP8, 2 for the 16-bit
    variant). The K/V prologue reads k and v and writes their codes and
    scales; the attention kernel reads q (it makes the Q codes itself), the K
    and V codes and scales, and writes o."""
    B, Hq, Hkv, Lq, Lk, D = (cfg[x] for x in ("B", "Hq", "Hkv", "Lq", "Lk", "D"))
    Dp = L.Dp
    kv_codes = B * Hkv * Lk * (1 + vb) * Dp + B * Hkv * (Lk // 64 + 1) * 4
    pro = 2 * D * 2 * B * Hkv * Lk + kv_codes                       # k, v read once, codes written
    main = 2 * B * Hq * Lq * D + kv_codes + 2 * B * Hq * Lq * D      # q read, codes read, o written
    return pro, main


def strided_windows(Lq, n=8, w=16):
    """n windows of w query rows spread over [0, Lq), the last ending at Lq."""
    w = min(w, Lq)
    starts = sorted({min(i * (Lq // n) + (37 * i) % max(Lq // n - w, 1), Lq - w) for i in range(n - 1)}
                    | {Lq - w})
    return [(s0, s0 + w) for s0 in starts]


def fp64_attention(q, k, v, sm, causal, b, h, G, r0, r1):
    """softmax(q k^T sm) v in float64 for query rows [r0, r1) of head (b, h)
    (logical-HND float32 inputs; top-left causal mask when causal)."""
    import numpy as np
    qh = q[b, h, r0:r1].astype(np.float64)
    kh = k[b, h // G].astype(np.float64)
    vh = v[b, h // G].astype(np.float64)
    s = (qh @ kh.T) * sm
    if causal:
        s[np.arange(r0, r1)[:, None] < np.arange(kh.shape[0])[None, :]] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ vh) / p.sum(axis=1, keepdims=True)


def accuracy(o, q, k, v, cfg, sm, causal):
    """The pages' accuracy figures (cosine, relative L2, max-abs against float64
    attention) of the output o over every head, on windows of query rows
    spread over the whole range (all rows when Lq <= 128)."""
    import numpy as np
    B, Hq, Lq = cfg["B"], cfg["Hq"], cfg["Lq"]
    G = Hq // cfg["Hkv"]
    got = o.float()
    if cfg["layout"] == "NHD":
        got = got.permute(0, 2, 1, 3)
    wins = [(0, Lq)] if Lq <= 128 else strided_windows(Lq)
    g, e = [], []
    for (r0, r1) in wins:
        g.append(got[:, :, r0:r1].double().cpu().numpy())
        e.append(np.stack([np.stack([fp64_attention(q, k, v, sm, causal, b, h, G, r0, r1)
                                     for h in range(Hq)]) for b in range(B)]))
    g = np.concatenate(g, axis=2)
    e = np.concatenate(e, axis=2)
    d = g - e
    return {"cos": float((g * e).sum() / math.sqrt((g * g).sum() * (e * e).sum())),
            "rel_l2": float(math.sqrt((d * d).sum() / (e * e).sum())),
            "max_abs": float(np.abs(d).max()),
            "rows": "all %d heads x %d query rows (%d windows over [0, %d))" % (B * Hq, g.shape[2], len(wins), Lq)}


def time_step(qa, torch, np, copies, o, layout, causal, sm, pv, args, stream):
    """Settle, warm-up and timed steps of the whole path (K/V prologue, then the
    attention kernel with Q coded inside it), cycling through the input copies;
    HIP events on the launch stream around the prologue and the attention
    kernel(s) of every step."""
    p = qa.make_problem(*copies[0], o, layout, pv=pv)
    L = qa.workspace_layout(p)
    ws = qa.new_workspace(p)
    nsplit = qa.split_count(p)
    nb = qa.split_bytes(p, nsplit)
    part = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None

    def step(i, ev=None):
        qd, kd, vd = copies[i % len(copies)]
        if ev is not None:
            ev.record(3 * i)
        qa.quantize_kv(p, kd, vd, ws, smooth_k=True)
        if ev is not None:
            ev.record(3 * i + 1)
        qa.attn_q_ex(p, qd, ws, o, is_causal=causal, sm_scale=sm, nsplit=nsplit, part=part)
        if ev is not None:
            ev.record(3 * i + 2)

    settle(step, args.settle_s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = HipEvents(3 * args.steps, stream.cuda_stream)
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        step(i, events)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    pro = [events.elapsed_ms(3 * i, 3 * i + 1) for i in range(args.steps)]
    mai = [events.elapsed_ms(3 * i + 1, 3 * i + 2) for i in range(args.steps)]
    events.close()
    del ws, part
    return dict(ms_step=total_ms / args.steps, main_ms=float(np.mean(mai)), pro_ms=float(np.mean(pro)),
                nsplit=nsplit, L=L)


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def counter_clock(main_ms):
    """GPU clock during the attention kernel, from the committed counter summary
    (GRBM_GUI_ACTIVE cycles per XCD over the kernel) and this run's kernel time;
    None when the summary is missing or was taken on another kernel source."""
    try:
        kv = {}
        for line in open(COUNTERS_FILE):
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        cyc = float(kv["attn_gpu_active_cycles_per_xcd"])
        return {"ghz": cyc / (main_ms * 1e-3) / 1e9, "mfma_busy_frac": float(kv["attn_mfma_busy_frac"])}
    except (OSError, KeyError, ValueError):
        return None


def run_workload(name, qa, torch, np, si, args, stream):
    """One further workload of the pages' set, timed like the default one (its
    own inputs, prologue + attention with Q coded in the kernel), with its own
    roofline fields and accuracy."""
    q, k, v, cfg = si.make_inputs(name)
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg["dtype"]]
    layout = cfg["layout"]

    def dev(x):
        t = torch.from_numpy(x).to(dt)
        if layout == "NHD":
            t = t.permute(0, 2, 1, 3).contiguous()
        return t.cuda()

    copies = [(dev(q), dev(k), dev(v))]
    nbytes = sum(x.numel() * x.element_size() for x in copies[0])
    for _ in range(max(0, min(args.rotate, 1 + (768 << 20) // max(nbytes, 1)) - 1)):
        copies.append(tuple(x.clone() for x in copies[0]))
    o = torch.empty_like(copies[0][0])
    causal = cfg["causal"]
    sm = 1.0 / math.sqrt(cfg["D"])
    B, Hq, Lq, Lk, D = (cfg[x] for x in ("B", "Hq", "Lq", "Lk", "D"))
    r = time_step(qa, torch, np, copies, o, layout, causal, sm, "fp8", args, stream)
    Dp = r["L"].Dp
    pairs = sum(min(i + 1, Lk) for i in range(Lq)) if causal else Lq * Lk
    useful = 4.0 * B * Hq * pairs * D
    executed = 4.0 * B * Hq * pairs * Dp
    tops = useful / (r["main_ms"] * 1e-3) / 1e12
    pro_bytes, main_bytes = algorithmic_bytes(cfg, r["L"], vb=1)
    rec = {
        "workload": "%s: B=%d H=%d Lq=%d Lk=%d D=%d (padded to %d) %s %s%s" % (
            name, B, Hq, Lq, Lk, D, Dp, cfg["dtype"], layout, ", top-left causal" if causal else ""),
        "value": useful / (r["ms_step"] * 1e-3) / 1e12, "unit": "TOPS", "ms_per_step": r["ms_step"],
        "main_kernel_ms": r["main_ms"], "main_kernel_tops": tops,
        "main_kernel_tops_executed": executed / (r["main_ms"] * 1e-3) / 1e12,
        "prologue_ms": r["pro_ms"], "prologue_gbs": pro_bytes / (r["pro_ms"] * 1e-3) / 1e9,
        "nsplit": r["nsplit"], "input_copies": len(copies),
        "ops": "useful = 4 B H D x (visible query-key pairs); executed counts the padded head dim %d" % Dp,
        "roofline": {"bound": "mfma", "achieved": tops, "peak": PEAK_MFMA_TOPS, "unit": "TFLOP/s",
                     "frac": tops / PEAK_MFMA_TOPS,
                     "frac_executed": executed / (r["main_ms"] * 1e-3) / 1e12 / PEAK_MFMA_TOPS,
                     "traffic": None, "kernel": "attn_kernel", "algorithmic_ops": useful,
                     "algorithmic_bytes": main_bytes},
        "accuracy_vs_fp64": accuracy(o, q, k, v, cfg, sm, causal),
    }
    del copies, o
    torch.cuda.empty_cache()
    return rec



def main():
    args = parse()
    if args.no_variants:
        args.variants = "none"
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_attention_sage_amd as qa
    import sage_inputs as si

    name = args.config
    q, k, v, cfg = si.make_inputs(name)
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg["dtype"]]
    layout = cfg["layout"]

    def dev(x):
        t = torch.from_numpy(x).to(dt)
        if layout == "NHD":
            t = t.permute(0, 2, 1, 3).contiguous()
        return t.cuda()

    copies = [(dev(q), dev(k), dev(v))]
    for _ in range(max(0, args.rotate - 1)):
        copies.append(tuple(x.clone() for x in copies[0]))
    o = torch.empty_like(copies[0][0])
    causal = cfg["causal"]
    sm = 1.0 / math.sqrt(cfg["D"])
    stream = torch.cuda.current_stream()
    B, Hq, Lq, Lk, D = (cfg[x] for x in ("B", "Hq", "Lq", "Lk", "D"))
    ops = 4.0 * B * Hq * Lq * Lk * D
    G = cfg["Hq"] // cfg["Hkv"]

    def run(pv):
        """Warm-up and timed steps of the c3 path with the given P.V format."""
        r = time_step(qa, torch, np, copies, o, layout, causal, sm, pv, args, stream)
        r["pro_bytes"], r["main_bytes"] = algorithmic_bytes(cfg, r.pop("L"), vb=1 if pv == "fp8" else 2)
        return r

    r8 = run("fp8")
    acc8 = accuracy(o, q, k, v, cfg, sm, causal)
    ms_step, main_ms, pro_ms = r8["ms_step"], r8["main_ms"], r8["pro_ms"]
    pro_bytes, main_bytes = r8["pro_bytes"], r8["main_bytes"]
    main_tops = ops / (main_ms * 1e-3) / 1e12

    variants = None
    if args.variants != "none":
        r16 = run("fp16")
        acc16 = accuracy(o, q, k, v, cfg, sm, causal)
        t16 = ops / (r16["main_ms"] * 1e-3) / 1e12
        variants = {"qk_int8_pv_fp16": {
            "value": ops / (r16["ms_step"] * 1e-3) / 1e12, "unit": "TOPS",
            "ms_per_step": r16["ms_step"], "main_kernel_tops": t16, "main_kernel_ms": r16["main_ms"],
            "prologue_ms": r16["pro_ms"], "prologue_gbs": r16["pro_bytes"] / (r16["pro_ms"] * 1e-3) / 1e9,
            "accuracy_vs_fp64": acc16, "dtype": "int8+%s" % cfg["dtype"],
            "roofline": {"bound": "mfma", "achieved": t16, "peak": PEAK_PV16_TOPS, "unit": "TFLOP/s",
                         "frac": t16 / PEAK_PV16_TOPS,
                         "traffic": recorded_traffic("attn16") if name == "c3" else None,
                         "kernel": "attn_kernel (16-bit P.V)", "algorithmic_ops": ops,
                         "algorithmic_bytes": r16["main_bytes"]}}}

    if args.variants == "all" and name == "c3":
        # packed variable-length call on the same tokens: the 2 x 4096 tokens of
        # the workload cut into 8 sequences of mixed lengths (sum 8192), every
        # sequence attending to itself; ops counted per sequence.
        lens = [3000, 2000, 1200, 900, 500, 300, 200, 92]
        assert sum(lens) == B * Lq
        pk = lambda x: torch.from_numpy(np.ascontiguousarray(
            np.concatenate([x[b].transpose(1, 0, 2) for b in range(B)], axis=0))).to(dt).cuda()
        qp, kp, vp = pk(q), pk(k), pk(v)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32).cuda()
        vops = sum(4.0 * Hq * n * n * D for n in lens)
        ov = torch.empty_like(qp)
        for vpv in ("fp16", "fp8"):
            pvl = qa.make_varlen_problem(qp, kp, vp, ov, len(lens), max(lens), max(lens), pv=vpv)
            ws_v = torch.empty(qa.varlen_workspace_bytes(pvl), dtype=torch.uint8, device="cuda")
            call = lambda: qa.varlen_attn(pvl, qp, kp, vp, ov, cu, cu, ws_v, sm_scale=sm)
            settle(lambda i: call(), min(args.settle_s, 0.2))
            for _ in range(args.warmup):
                call()
            torch.cuda.synchronize()
            ev = HipEvents(2 * args.steps, stream.cuda_stream)
            for i in range(args.steps):
                ev.record(2 * i)
                call()
                ev.record(2 * i + 1)
            torch.cuda.synchronize()
            vms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
            ev.close()
            variants["varlen_pv_%s" % vpv] = {
                "value": vops / (vms * 1e-3) / 1e12, "unit": "TOPS", "ms_per_call": vms,
                "workload": "packed: the %d x %d tokens cut into sequences %s, H=%d D=%d %s, "
                            "prologue + attention in one call" % (B, Lq, lens, Hq, D, cfg["dtype"]),
                "algorithmic_ops": vops}
            del ws_v

    if args.variants == "all" and name == "c3":
        # the grouped-query long-key workload (B=1 Hq=32 Hkv=8 Lq=1024 Lk=8192
        # D=128 bf16 NHD): its 256 FP8 query tiles (128 16-bit ones) leave
        # workgroup slots idle, which the key splits fill. Attention only, on
        # a workspace quantized once, one pass against the library's choice.
        q4, k4, v4, c4 = si.make_inputs("c4")
        dt4 = {"fp16": torch.float16, "bf16": torch.bfloat16}[c4["dtype"]]
        d4 = lambda x: torch.from_numpy(x).to(dt4).permute(0, 2, 1, 3).contiguous().cuda()
        q4d, k4d, v4d = d4(q4), d4(k4), d4(v4)
        o4 = torch.empty_like(q4d)
        ops4 = 4.0 * c4["B"] * c4["Hq"] * c4["Lq"] * c4["Lk"] * c4["D"]
        sm4 = 1.0 / math.sqrt(c4["D"])
        for vpv in ("fp8", "fp16"):
            p4 = qa.make_problem(q4d, k4d, v4d, o4, "NHD", pv=vpv)
            ws4 = qa.new_workspace(p4)
            qa.quantize(p4, q4d, k4d, v4d, ws4)
            auto = qa.split_count(p4)
            rec = {"workload": "B=1 Hq=32 Hkv=8 Lq=1024 Lk=8192 D=128 bf16 NHD, attention kernel(s) only",
                   "unit": "TOPS", "algorithmic_ops": ops4}
            for S in (1, auto):
                nbytes = qa.split_bytes(p4, S)
                part4 = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
                # one round of workgroups: the one-call path codes Q in the
                # prologue here, so the kernel reads the workspace's Q codes
                call = lambda: qa.attn_quantized_ex(p4, ws4, o4, sm_scale=sm4, nsplit=S, part=part4)
                settle(lambda i: call(), min(args.settle_s, 0.2))
                for _ in range(args.warmup):
                    call()
                torch.cuda.synchronize()
                ev = HipEvents(2 * args.steps, stream.cuda_stream)
                for i in range(args.steps):
                    ev.record(2 * i)
                    call()
                    ev.record(2 * i + 1)
                torch.cuda.synchronize()
                ms4 = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
                ev.close()
                key = "one_pass" if S == 1 else "split_%d" % S
                rec[key] = {"ms": ms4, "tops": ops4 / (ms4 * 1e-3) / 1e12}
                del part4
            rec["value"] = rec["split_%d" % auto if auto > 1 else "one_pass"]["tops"]
            rec["nsplit"] = auto
            variants["gqa_long_keys_pv_%s" % vpv] = rec
            del ws4
        del q4d, k4d, v4d, o4

    if args.variants == "all" and name == "c3" and not causal:
        # the same workload with a causal mask (top-left, Lq = Lk): attention
        # only; ops counted over the visible (query, key) pairs,
        # 4 D B H sum_i min(i + 1, Lk), beside the unmasked count
        p_c = qa.make_problem(*copies[0], o, layout, pv="fp8")
        ws_c = qa.new_workspace(p_c)
        qa.quantize(p_c, *copies[0], ws_c)
        vis = sum(min(i + 1, Lk) for i in range(Lq))
        cops = 4.0 * D * B * Hq * vis
        call = lambda: qa.attn_q_ex(p_c, copies[0][0], ws_c, o, is_causal=True, sm_scale=sm, nsplit=1)
        settle(lambda i: call(), min(args.settle_s, 0.2))
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        ev = HipEvents(2 * args.steps, stream.cuda_stream)
        for i in range(args.steps):
            ev.record(2 * i)
            call()
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        cms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
        ev.close()
        variants["causal"] = {
            "value": cops / (cms * 1e-3) / 1e12, "unit": "TOPS", "ms": cms,
            "tops_unmasked_count": ops / (cms * 1e-3) / 1e12, "visible_pair_ops": cops,
            "workload": "same shape, FP8 P.V, top-left causal mask; attention only; ops over visible pairs"}
        del ws_c

    if args.variants == "all" and name == "c3":
        # block-sparse attention on the same workload: a seeded pattern with a
        # given fraction of the 128 x 128 blocks on, attention only. Ops are
        # counted on the computed blocks.
        p_s = qa.make_problem(*copies[0], o, layout, pv="fp8")
        ws_s = qa.new_workspace(p_s)
        qa.quantize(p_s, *copies[0], ws_s)
        shape = qa.block_mask_shape(p_s)
        for dens in (0.5, 0.25):
            rng = np.random.default_rng(11)
            mask = torch.from_numpy((rng.random(shape) < dens).astype(np.uint8)).cuda()
            frac = float(mask.float().mean())
            call = lambda: qa.attn_q_ex(p_s, copies[0][0], ws_s, o, sm_scale=sm, nsplit=1, block_mask=mask)
            settle(lambda i: call(), min(args.settle_s, 0.2))
            for _ in range(args.warmup):
                call()
            torch.cuda.synchronize()
            ev = HipEvents(2 * args.steps, stream.cuda_stream)
            for i in range(args.steps):
                ev.record(2 * i)
                call()
                ev.record(2 * i + 1)
            torch.cuda.synchronize()
            sms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
            ev.close()
            variants["block_sparse_%d" % int(round(dens * 100))] = {
                "value": frac * ops / (sms * 1e-3) / 1e12, "unit": "TOPS", "ms": sms,
                "blocks_on": frac, "speedup_vs_dense_kernel": main_ms / sms,
                "workload": "same shape, FP8 P.V, random pattern with %.0f%% of the 128x128 blocks on; "
                            "attention only; ops on computed blocks" % (100 * dens)}
        del ws_s

    if args.copy_calibration:
        # a plain elementwise copy (negation) of COPY_BYTES: reads and writes
        # COPY_BYTES once each; its kernel name carries "neg"
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    # the pages' other dense workloads, and c3's shape at head dim 64, each
    # timed on its own (prologue + attention, FP8 P.V) with its own roofline
    # fields and accuracy
    workloads = None
    if args.variants == "all" and name == "c3":
        workloads = {w: run_workload(w, qa, torch, np, si, args, stream) for w in ("c5", "c2", "c2c", "c3d64")}
    # the counter summaries were taken on the c3 workload
    clock = counter_clock(main_ms) if name == "c3" else None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        # the oracle as it stands (prologue + quantized attention) on a bounded
        # sample: cpu_heads heads of the same workload, cpu_rows query rows each
        nh = min(args.cpu_heads, Hq)
        # the box gives one GPU a share of 16 host threads, whatever the core count shows
        threads = min(16, len(os.sched_getaffinity(0)))
        qh = q[:1, :nh]
        kh = k[:1, :(nh + G - 1) // G]
        vh = v[:1, :(nh + G - 1) // G]
        t0 = time.perf_counter()
        qz = oracle.quantize(qh, kh, vh, threads=threads)
        bk, pref = qa.softmax_spec("fp8")
        oracle.attn_quantized(qz, sm, causal=causal, bk=bk, pref=pref,
                              rows=(0, args.cpu_rows), threads=threads)
        dt_cpu = time.perf_counter() - t0
        cpu_ops = 4.0 * qh.shape[1] * args.cpu_rows * Lk * D
        cpu = {"value": cpu_ops / dt_cpu / 1e12, "unit": "TOPS", "cores": threads,
               "kind": "oracle", "cpu_model": host_cpu_model(),
               "sample": "%d heads x %d query rows of the same workload (all %d keys), "
                         "prologue of those heads included; %.1f s" % (qh.shape[1], args.cpu_rows, Lk, dt_cpu)}

    out = {
        "metric": "attention TOPS (4*B*H*Lq*Lk*D/s) + %MFMA peak at B2 H24 L4096 D128; cos vs fp64",
        "value": ops / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d H=%d Hkv=%d Lq=%d Lk=%d D=%d %s %s%s" % (
            name, B, Hq, cfg["Hkv"], Lq, Lk, D, cfg["dtype"], layout, " causal" if causal else ""),
            "global_batch": B, "seq_len": Lq, "parallelism": "single-gpu", "nsplit": r8["nsplit"]},
        "main_kernel_tops": main_tops,
        "main_kernel_ms": main_ms,
        "prologue_ms": pro_ms,
        "prologue_gbs": pro_bytes / (pro_ms * 1e-3) / 1e9,
        "cos_vs_fp64": acc8["cos"],
        "accuracy_vs_fp64": acc8,
        "roofline": {"bound": "mfma", "achieved": main_tops, "peak": PEAK_MFMA_TOPS,
                     "unit": "TFLOP/s", "frac": main_tops / PEAK_MFMA_TOPS,
                     "traffic": recorded_traffic() if name == "c3" else None,
                     "kernel": "attn_kernel", "algorithmic_ops": ops,
                     "algorithmic_bytes": main_bytes, "clock": clock,
                     "frac_at_clock": (main_tops / (PEAK_MFMA_TOPS * clock["ghz"] / 2.4)) if clock else None},
        "workloads": workloads,
        "cpu_baseline": cpu,
        "variants": variants,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
