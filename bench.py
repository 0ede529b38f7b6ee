"""Benchmark of the quantized-attention hot path on one MI355X.

One step = the whole path on one batch: the quantization prologue
(sage_quantize: key mean, INT8 Q/K, FP8 V) followed by the attention kernel
(sage_attn_quantized: INT8 QK^T, online softmax, FP8 P.V), enqueued through
the C ABI on torch's current stream, inputs already resident in HBM.

Workload (default): B=2 H=24 Lq=Lk=4096 D=128 fp16 HND, q, v ~ N(0,1),
k ~ N(0,1) plus a per-(head, channel) bias ~ N(0, 4), non-causal, smooth_k on.
The metric is attention TOPS = 4*B*H*Lq*Lk*D / time. ``value`` uses the whole
step; the attention kernel's own rate (the figure the pages quote, which leaves
quantization out) is reported as ``main_kernel_tops`` and in ``roofline``.

Prints one JSON line. Timings come from HIP events recorded on the launch
stream around every kernel group inside the timed region.
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
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--rotate", type=int, default=3,
                    help="input copies cycled through so the prologue reads HBM, not cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows per head in the CPU-oracle sample")
    ap.add_argument("--cpu-heads", type=int, default=4)
    return ap.parse_args()


def algorithmic_bytes(cfg, L):
    """Bytes each kernel must move at least once (see the design notes)."""
    B, Hq, Hkv, Lq, Lk, D = (cfg[x] for x in ("B", "Hq", "Hkv", "Lq", "Lk", "D"))
    Dp = L.Dp
    inp = 2 * D * (B * Hq * Lq + 2 * B * Hkv * Lk)                 # q, k, v read once
    quant = B * Hq * Lq * (Dp + 4) + B * Hkv * Lk * (2 * Dp) + B * Hkv * (Lk // 64 + 1) * 4
    main = B * Hq * Lq * (Dp + 4) + B * Hkv * Lk * 2 * Dp + 2 * B * Hq * Lq * D
    return inp + quant, main


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
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
    p = qa.make_problem(*copies[0], o, layout)
    L = qa.workspace_layout(p)
    ws = qa.new_workspace(p)
    causal = cfg["causal"]
    sm = 1.0 / math.sqrt(cfg["D"])
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        qd, kd, vd = copies[i % len(copies)]
        if ev is not None:
            ev[0].record(stream)
        qa.quantize(p, qd, kd, vd, ws, smooth_k=True)
        if ev is not None:
            ev[1].record(stream)
        qa.attn_quantized(p, ws, o, is_causal=causal, sm_scale=sm)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        step(i, events[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    pro = [e[0].elapsed_time(e[1]) for e in events]
    mai = [e[1].elapsed_time(e[2]) for e in events]

    B, Hq, Lq, Lk, D = (cfg[x] for x in ("B", "Hq", "Lq", "Lk", "D"))
    ops = 4.0 * B * Hq * Lq * Lk * D
    ms_step = total_ms / args.steps
    main_ms = float(np.mean(mai))
    pro_ms = float(np.mean(pro))
    pro_bytes, main_bytes = algorithmic_bytes(cfg, L)
    main_tops = ops / (main_ms * 1e-3) / 1e12

    # accuracy of this run on sampled rows against exact fp64 attention
    import oracle
    heads = [(0, 0), (B - 1, Hq - 1)]
    rows = (0, 64)
    G = cfg["Hq"] // cfg["Hkv"]
    got = o.float()
    if layout == "NHD":
        got = got.permute(0, 2, 1, 3)
    got = np.stack([got[b, h, rows[0]:rows[1]].double().cpu().numpy() for b, h in heads])
    qs = np.stack([q[b, h] for b, h in heads])[:, None]
    ks = np.stack([k[b, h // G] for b, h in heads])[:, None]
    vs = np.stack([v[b, h // G] for b, h in heads])[:, None]
    ex = np.concatenate([oracle.attn_exact(qs[n:n + 1], ks[n:n + 1], vs[n:n + 1], sm, causal=causal,
                                           rows=rows) for n in range(len(heads))])
    cos = float((got * ex).sum() / math.sqrt((got * got).sum() * (ex * ex).sum()))

    cpu = None
    if not args.no_cpu_baseline:
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
        oracle.attn_quantized(qz, sm, causal=causal, bk=qa.softmax_block_keys(),
                              rows=(0, args.cpu_rows), threads=threads)
        dt_cpu = time.perf_counter() - t0
        cpu_ops = 4.0 * qh.shape[1] * args.cpu_rows * Lk * D
        cpu = {"value": cpu_ops / dt_cpu / 1e12, "unit": "TOPS", "cores": threads,
               "kind": "oracle",
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
            "global_batch": B, "seq_len": Lq, "parallelism": "single-gpu"},
        "main_kernel_tops": main_tops,
        "main_kernel_ms": main_ms,
        "prologue_ms": pro_ms,
        "prologue_gbs": pro_bytes / (pro_ms * 1e-3) / 1e9,
        "cos_vs_fp64_sampled": cos,
        "roofline": {"bound": "mfma", "achieved": main_tops, "peak": PEAK_MFMA_TOPS,
                     "unit": "TFLOP/s", "frac": main_tops / PEAK_MFMA_TOPS, "traffic": None,
                     "kernel": "attn_kernel", "algorithmic_ops": ops,
                     "algorithmic_bytes": main_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
