"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no step of the attention method: it only draws numbers.
Both the CPU oracle and the HIP path consume the tensors it returns.

Generator (counter based, so any (batch, head) slice can be regenerated on its
own):
  * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014) applied to the counter
    ``seed + (stream << 40) + 2*n`` and ``... + 2*n + 1`` for element n of the
    logical (batch, head, token, channel) tensor gives two 64-bit words;
  * their top 53 bits give uniforms u1, u2 in (0, 1];
  * Box-Muller in fp64: z = sqrt(-2 ln u1) * cos(2 pi u2);
  * value = mu + sigma * z in fp64, rounded to fp32 then to the input dtype
    (round to nearest even at each step).
Streams: q = 0, k = 1, v = 2, per-(head, channel) key bias = 3.
Element order is the logical HND order, so an NHD tensor holds the same values
as its HND counterpart, only permuted.
"""
import math

import numpy as np

M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

STREAM_Q, STREAM_K, STREAM_V, STREAM_KBIAS = 0, 1, 2, 3


def splitmix64(x):
    """SplitMix64 output function on a uint64 numpy array (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = x + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        return z ^ (z >> np.uint64(31))


def normal(seed, stream, start, count):
    """count standard normals for flat element indices [start, start+count)."""
    n = np.arange(start, start + count, dtype=np.uint64)
    base = np.uint64(seed) + (np.uint64(stream) << np.uint64(40))
    with np.errstate(over="ignore"):
        c = base + np.uint64(2) * n
        w1 = splitmix64(c)
        w2 = splitmix64(c + np.uint64(1))
    u1 = ((w1 >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = ((w2 >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def round_to_dtype(x64, dtype):
    """fp64 -> fp32 -> dtype, returned as float32 values exactly representable in dtype."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        bits = x32.view(np.uint32).astype(np.uint64)
        # round to nearest even on the low 16 bits (finite inputs only)
        lsb = (bits >> np.uint64(16)) & np.uint64(1)
        bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
        return bits.astype(np.uint32).view(np.float32)
    if dtype == "fp32":
        return x32
    raise ValueError(dtype)


# Workloads. Distributions: N(mean, variance); "kbias_var" adds a key bias
# bias[h, d] ~ N(0, kbias_var) shared by every batch and token.
CONFIGS = {
    "c1": dict(B=1, Hq=2, Hkv=2, Lq=128, Lk=128, D=64, dtype="fp16", layout="HND",
               causal=False, kbias_var=0.0),
    "c2": dict(B=1, Hq=16, Hkv=16, Lq=512, Lk=512, D=64, dtype="fp16", layout="HND",
               causal=False, kbias_var=0.0),
    "c2c": dict(B=1, Hq=16, Hkv=16, Lq=512, Lk=512, D=64, dtype="fp16", layout="HND",
                causal=True, kbias_var=0.0),
    "c3": dict(B=2, Hq=24, Hkv=24, Lq=4096, Lk=4096, D=128, dtype="fp16", layout="HND",
               causal=False, kbias_var=4.0),
    "c4": dict(B=1, Hq=32, Hkv=8, Lq=1024, Lk=8192, D=128, dtype="bf16", layout="NHD",
               causal=False, kbias_var=0.0),
    "c5": dict(B=1, Hq=40, Hkv=40, Lq=14040, Lk=14040, D=80, dtype="bf16", layout="NHD",
               causal=False, kbias_var=2.0),
    # c3's shape at head dim 64 (the pages' small workloads use D = 64): a
    # long-sequence figure for the Dp = 64 tile
    "c3d64": dict(B=2, Hq=24, Hkv=24, Lq=4096, Lk=4096, D=64, dtype="fp16", layout="HND",
                  causal=False, kbias_var=4.0),
}
SEEDS = {"c1": 0x5A6E0001, "c2": 0x5A6E0002, "c2c": 0x5A6E0002, "c3": 0x5A6E0003,
         "c4": 0x5A6E0004, "c5": 0x5A6E0005, "c3d64": 0x5A6E0006}


def gen_tensor(seed, stream, B, H, L, D, dtype, mean=0.0, std=1.0, heads=None, bias=None):
    """Logical-HND float32 tensor [B, len(heads) or H, L, D] of dtype-representable values.

    heads: optional list of head indices to generate (each regenerated from its
    own counters). bias: optional [H, D] fp64 array added before rounding.
    """
    hs = list(range(H)) if heads is None else list(heads)
    out = np.empty((B, len(hs), L, D), np.float32)
    per_head = L * D
    for b in range(B):
        for n, h in enumerate(hs):
            start = (b * H + h) * per_head
            x = mean + std * normal(seed, stream, start, per_head).reshape(L, D)
            if bias is not None:
                x = x + bias[h][None, :]
            out[b, n] = round_to_dtype(x, dtype)
    return out


def key_bias(seed, H, D, var):
    if var == 0.0:
        return None
    return (math.sqrt(var) * normal(seed, STREAM_KBIAS, 0, H * D)).reshape(H, D)


def make_inputs(name_or_cfg, seed=None, heads=None, kv_heads=None):
    """(q, k, v, cfg) as logical-HND float32 numpy arrays for a named workload.

    heads / kv_heads optionally restrict which q / kv heads are generated.
    """
    if isinstance(name_or_cfg, str):
        cfg = dict(CONFIGS[name_or_cfg])
        seed = SEEDS[name_or_cfg] if seed is None else seed
    else:
        cfg = dict(name_or_cfg)
        seed = 0x5A6E0000 if seed is None else seed
    B, Hq, Hkv, Lq, Lk, D, dt = (cfg[x] for x in ("B", "Hq", "Hkv", "Lq", "Lk", "D", "dtype"))
    bias = key_bias(seed, Hkv, D, cfg.get("kbias_var", 0.0))
    q = gen_tensor(seed, STREAM_Q, B, Hq, Lq, D, dt, heads=heads)
    k = gen_tensor(seed, STREAM_K, B, Hkv, Lk, D, dt, heads=kv_heads, bias=bias)
    v = gen_tensor(seed, STREAM_V, B, Hkv, Lk, D, dt, heads=kv_heads)
    return q, k, v, cfg
