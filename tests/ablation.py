"""Per-technique ablation of the method's accuracy, computed by the oracle.

Each technique of the method ("BitDecoding-FP4 : décodage natif du KV cache FP4", Analyse
approfondie; "FP4 KV Cache Done Right", What is actually new in BitDecoding-FP4?) is
switched off in turn -- dual-residual query, static smoothing, Hadamard rotation, key scale
search, underflow-aware probability scaling -- on the five synthetic workloads, and three
numbers are reported per setting:

* logit error  ||s - s_ref||_F / ||s_ref||_F over the sampled rows, s_ref = the exact
  (unquantized, fp64) base-2 logit,
* output error  mean over rows of ||o - o_ref||_2 / ||o_ref||_2 against unquantized fp64
  attention (and the max over rows of the same),
* the share of probability blocks that quantized to all zeros.

The GPU kernels implement the full method only; the switches change accuracy, not the data
flow that the kernels time, so this study runs on the CPU.

Usage: python tests/ablation.py [--quick] [--md]
"""
import argparse
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from fp4_kv_cache_amd import workloads as W  # noqa: E402
from oracle import attention as A  # noqa: E402
from oracle import kvquant as KQ  # noqa: E402

SETTINGS = [
    ("full method", {}),
    ("single-pass query (no dual residual)", {"dual": False}),
    ("no smoothing", {"smooth": False}),
    ("no Hadamard rotation", {"rotate": False}),
    ("no key scale search", {"search": False}),
    ("normalized P, tensor scale 1 (no underflow-aware scaling)", {"p_mode": "vanilla"}),
    ("unquantized P (reference for the P codec)", {"p_mode": "exact"}),
]

# (workload, sampled units, context cap) -- units are (sequence, KV head) for GQA, sequences for MLA
PLAN = {
    "tiny": ([(0, 0), (0, 1)], None),
    "qwen3_4b": ([(0, 0), (3, 5), (9, 2)], None),
    "qwen3_30b_a3b": ([(0, 0), (5, 3), (17, 1)], None),
    "long_underflow": ([(0, 0), (2, 6)], None),
    "mla": ([0, 5], 8192),
}
QUICK = {
    "tiny": ([(0, 0)], 2048),
    "qwen3_4b": ([(0, 0)], 4096),
    "qwen3_30b_a3b": ([(0, 0)], 4096),
    "long_underflow": ([(0, 0)], 16384),
    "mla": ([0], 1024),
}
LOG2E = 1.0 / math.log(2.0)


def _p_blocks(L, rows, fmt):
    B = 16 if fmt == 0 else 32
    return rows * -(-L // B)


def gqa_unit(w, b, h, L, calib, opts):
    ksi, qs, gk, gv = calib
    g = w["hq"] // w["hkv"]
    q = W.queries(w, b)[h * g:(h + 1) * g]
    K = W.keys(w, b, h, L)
    V = W.values(w, b, h, L)
    sc = W.softmax_scale(w)
    res = A.gqa_head(q, K, V, ksi[h], qs[h], gk[h], gv[h], w["fmt"], sc, L=L, opts=opts)
    s_ref = LOG2E * sc * (np.asarray(q, np.float64) @ np.asarray(K, np.float64).T)
    o_ref = A.reference_attention(q, K, V, sc)
    return res, s_ref, o_ref, _p_blocks(L, g, w["fmt"])


def mla_unit(w, b, L, calib, opts):
    ksi, qs, gk, gv = calib
    D = w["d"]
    q = W.queries(w, b)[:, :D]
    qr = W.rope_queries(w, b)
    K = W.keys(w, b, 0, L)
    kr = W.rope_keys(w, b, L)
    sc = W.softmax_scale(w)
    res = A.mla_seq(q, qr, K, kr, ksi[0], qs[0], gk[0], w["fmt"], sc, L=L, opts=opts)
    s_ref = LOG2E * sc * (np.asarray(q, np.float64) @ np.asarray(K, np.float64).T +
                          np.asarray(qr, np.float64) @ np.asarray(kr, np.float64).T)
    o_ref = A.reference_attention(q, K, K, sc, q_rope=qr, k_rope=kr)
    return res, s_ref, o_ref, _p_blocks(L, w["hq"], w["fmt"])


def run_setting(name, plan, opts):
    """Errors of one setting on one workload: (logit err, mean output err, max output err, zero share)."""
    w = W.workload(name)
    units, cap = plan
    calib = W.calibration(w)
    lens = W.seq_lens(w)
    ds, ns, rel, zero, blocks = 0.0, 0.0, [], 0, 0
    for u in units:
        b = u if w["attn"] == 1 else u[0]
        L = int(lens[b]) if cap is None else min(int(lens[b]), cap)
        if w["attn"] == 1:
            res, s_ref, o_ref, nb = mla_unit(w, b, L, calib, opts)
        else:
            res, s_ref, o_ref, nb = gqa_unit(w, b, u[1], L, calib, opts)
        s = np.asarray(res["s"], np.float64)[:, :L]
        ds += float(np.sum((s - s_ref) ** 2))
        ns += float(np.sum(s_ref ** 2))
        o = np.asarray(res["out"], np.float64)
        rel.extend((np.linalg.norm(o - o_ref, axis=-1) / np.linalg.norm(o_ref, axis=-1)).tolist())
        zero += int(res["zero_blocks"])
        blocks += nb
    return math.sqrt(ds / ns), float(np.mean(rel)), float(np.max(rel)), zero / max(blocks, 1)


def key_sse(name, L, search):
    """Key reconstruction error sum((k_hat - x)^2) of one (sequence, KV head), x the transformed key."""
    w = W.workload(name)
    ksi, qs, gk, gv = W.calibration(w)
    K = W.keys(w, 0, 0, L)
    kc, ks = KQ.quantize_keys(K, ksi[0], gk[0], w["fmt"], search, True)
    khat = A.key_dequant_exact(kc, ks, w["fmt"]) * (gk[0] if w["fmt"] == 0 else 1.0)
    x = KQ.rotate_keys(K, ksi[0], True)
    return float(np.sum((khat.astype(np.float64) - x.astype(np.float64)) ** 2))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--quick", action="store_true", help="one short unit per workload")
    ap.add_argument("--md", action="store_true", help="print a markdown table")
    args = ap.parse_args()
    plan = QUICK if args.quick else PLAN
    rows = []
    for name in plan:
        t0 = time.time()
        for label, opts in SETTINGS:
            r = run_setting(name, plan[name], opts)
            rows.append((name, label) + r)
            if not args.md:
                print("%-15s %-58s logit %.3e  out mean %.3e max %.3e  zero blocks %.4f" % ((name, label) + r),
                      flush=True)
        if not args.md:
            print("  (%s: %.1f s)" % (name, time.time() - t0), flush=True)
    if args.md:
        print("| workload | setting | logit error | output error (mean) | output error (max) | all-zero P blocks |")
        print("|---|---|---|---|---|---|")
        for r in rows:
            print("| %s | %s | %.2e | %.2e | %.2e | %.1f%% |" % (r[0], r[1], r[2], r[3], r[4], 100 * r[5]))


if __name__ == "__main__":
    main()
