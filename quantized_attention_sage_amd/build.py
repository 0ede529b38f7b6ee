"""Compile the gfx950 HIP sources into quantized_attention_sage_amd/libsage_attn.so.

Run as ``python -m quantized_attention_sage_amd.build`` or through the repository's
``__graft_entry__.build()``. Sources are compiled in parallel, then linked.

Flags:
  --offload-arch=gfx950           MI355X only.
  -ffp-contract=off               no implicit fused multiply-adds: the prologue's fp32
                                  quantization steps round after every operation (the
                                  attention kernel uses explicit fmaf where it wants one).
  -target-feature -packed-fp32-ops  keep the compiler from emitting packed fp32 ops.
  -amdgpu-mfma-vgpr-form=1         matrix-core results in ordinary VGPRs: the softmax
                                  reads the logits with VALU instructions, so keeping
                                  them out of the accumulation registers saves a copy
                                  per element.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsage_attn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "prologue.hip", "attn.hip", "attn_fp8.hip", "attn_pv16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in x)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    if out.strip() and verbose:
        print(out)


def build(verbose=False, extra_flags=()):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC] + FLAGS + list(extra_flags) + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
