"""Build libfp4kv.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m fp4_kv_cache_amd.build`` or ``fp4_kv_cache_amd.build.build()``.
Objects go to ``fp4_kv_cache_amd/_build/``; the library to ``fp4_kv_cache_amd/libfp4kv.so``.
The same sources compiled with -DFP4KV_ABLATION give ``libfp4kv_ablate.so``, the study
build whose technique switches (fp4kv_ablation_set) turn parts of the method off; the product
library has none of that code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp4kv.so")
LIB_ABLATION = os.path.join(HERE, "libfp4kv_ablate.so")
SOURCES = ["api.hip", "append.hip", "decode_gqa.hip", "decode_mla.hip", "decode_bf16.hip", "stream.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # every quantization decision is a single rounded fp32 operation: no contraction
    "-ffp-contract=off",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), err))
    return err


def build(verbose=False):
    """Compile every source for gfx950 and link libfp4kv.so and the ablation-study build
    libfp4kv_ablate.so (always rebuilds both)."""
    os.makedirs(OUT, exist_ok=True)
    os.makedirs(os.path.join(OUT, "ablation"), exist_ok=True)

    def compile_one(job):
        src, abl = job
        obj = os.path.join(OUT, "ablation" if abl else "", src + ".o")
        extra = ["-DFP4KV_ABLATION"] if abl else []
        err = _run([HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(compile_one, jobs))
    for lib, group in ((LIB, objs[:len(SOURCES)]), (LIB_ABLATION, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + group)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
