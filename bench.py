#!/usr/bin/env python3
"""Benchmark of the FP4 paged-KV decode hot path on one MI355X.

One step = the whole hot path for one decode token of every sequence: the
KV-append quantizer on the new token (kv_quant_append) and paged FP4 decode
attention over the full context (fp4_decode_attention: fused dual-residual
query prologue, FP4 QK^T, transposed softmax with fused P quantization, FP4
P.V, split-K merge).  Default workload: the Qwen3-4B-shaped batch
(16 sequences x 32768 tokens, 32 query / 8 KV heads, head_dim 128, page 64,
shuffled page table, NVFP4), inputs synthetic and resident in HBM.

Prints one JSON line on stdout.  `value` is KV-cache bytes read per step
divided by the step time (GB/s); `roofline` is the decode-attention kernel's
algorithmic KV bytes over its own average duration (HIP events on the stream
it runs on) against the 8 TB/s HBM peak; `cpu_baseline` is the CPU oracle
timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP4_MFMA_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 matrix peak
METRIC = "FP4 paged decode attention: µs/step + KV HBM GB/s (% of 8 TB/s peak)"
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_token_head(w):
    """Packed codes + scales one decode step must read per (token, KV head)."""
    d = w["d"]
    B = 16 if w["fmt"] == 0 else 32
    if w["attn"] == 0:
        return 2 * (d // 2 + d // B)
    return d // 2 + (d // B) / B + 2 * w["rope"]


def decode_kernel(w):
    """Name of the decode-partials kernel that serves workload w."""
    return "mla" if w["attn"] == 1 else "gqa"


def decode_kernel_hash(kernel="gqa"):
    """Hash of the sources that define the decode-partials kernel and its launch."""
    h = hashlib.sha256()
    for f in ("decode_%s.hip" % kernel, "decode_common.h", "fp4kv_device.h", "fp4kv_internal.h", "api.hip"):
        h.update(open(os.path.join(ROOT, "fp4_kv_cache_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(w, workload):
    """HBM traffic per decode launch from the committed counter summary, if it matches this kernel."""
    kernel = decode_kernel(w)
    path = os.path.join(PROFILES, "decode_%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_hash") != decode_kernel_hash(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def mla_flops_per_token(w):
    """Algorithmic flops per cached token of an MLA decode step: Q.K^T for the Q1 and Q2 rows of
    every query head over the latent channels, the rope part once per head (it is not
    quantized, so the dual query does not apply to it), P.V over the latent channels."""
    hq, d, r = w["hq"], w["d"], w["rope"]
    return 2 * (2 * hq) * d + 2 * hq * r + 2 * hq * d


def cpu_baseline(w, n_units, budget_s):
    """The oracle's decode step (query prep, logits, FP4 softmax, P.V, merge) on a sample of
    (sequence, KV head) units at full context, repeated over the sample until `budget_s`
    seconds of timed work; cache quantization is done once beforehand, untimed."""
    from threadpoolctl import threadpool_limits
    from fp4_kv_cache_amd import workloads as W
    from oracle import attention as A
    from oracle import kvquant as KQ
    from oracle.query import quantize_query
    cores = len(os.sched_getaffinity(0))
    ksi, qs, gk, gv = W.calibration(w)
    g = w["hq"] // w["hkv"]
    lens = W.seq_lens(w)
    units = [(b, h) for b in range(w["batch"]) for h in range(w["hkv"])][:n_units]
    done_bytes, t_total, steps = 0.0, 0.0, 0
    if w["attn"] == 1:
        return _cpu_baseline_mla(w, n_units, budget_s, cores)
    with threadpool_limits(limits=cores):
        prepared = []
        for b, h in units:
            L = int(lens[b])
            kc, ks = KQ.quantize_keys(W.keys(w, b, h, L), ksi[h], gk[h], w["fmt"])
            vc, vs = KQ.quantize_values(W.values(w, b, h, L), gv[h], w["fmt"])
            prepared.append((b, h, L, kc, ks, vc, vs, W.queries(w, b)[h * g:(h + 1) * g]))
        while t_total < budget_s:
            for b, h, L, kc, ks, vc, vs, q in prepared:
                t0 = time.perf_counter()
                qq = quantize_query(q, qs[h], w["fmt"])
                s = A.logits(qq, A.key_dequant_exact(kc, ks, w["fmt"]), gk[h],
                             A.logit_coeff(W.softmax_scale(w), w["d"]), w["fmt"])
                A.attend(s, A.value_dequant_exact(vc, vs, w["fmt"], gv[h] if w["fmt"] == 0 else 1.0), L,
                         w["fmt"])
                t_total += time.perf_counter() - t0
                done_bytes += L * kv_bytes_per_token_head(w)
                steps += 1
    # the same steps with one BLAS thread (the oracle's elementwise work is single-threaded anyway)
    one_bytes, t_one = 0.0, 0.0
    with threadpool_limits(limits=1):
        while t_one < budget_s / 3:
            for b, h, L, kc, ks, vc, vs, q in prepared[:2]:
                t0 = time.perf_counter()
                qq = quantize_query(q, qs[h], w["fmt"])
                s = A.logits(qq, A.key_dequant_exact(kc, ks, w["fmt"]), gk[h],
                             A.logit_coeff(W.softmax_scale(w), w["d"]), w["fmt"])
                A.attend(s, A.value_dequant_exact(vc, vs, w["fmt"], gv[h] if w["fmt"] == 0 else 1.0), L,
                         w["fmt"])
                t_one += time.perf_counter() - t0
                one_bytes += L * kv_bytes_per_token_head(w)
    return {"value": round(done_bytes / t_total / 1e9, 5), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "value_1_thread": round(one_bytes / t_one / 1e9, 5),
            "sample": "%d (sequence, KV head) decode steps over %d of the workload's %d units, at full "
                      "context (%d tokens each); cache quantized once beforehand, untimed; %.1f s of "
                      "timed CPU work with %d BLAS threads, %.1f s with one" % (
                          steps, len(prepared), w["batch"] * w["hkv"], int(lens[0]), t_total, cores, t_one)}


def _cpu_baseline_mla(w, n_units, budget_s, cores):
    """MLA: the oracle's decode step (query prep, latent + rope logits, FP4 softmax, P.V with
    the latent, merge, un-rotation) per sequence; latent quantization done beforehand, untimed."""
    from threadpoolctl import threadpool_limits
    from fp4_kv_cache_amd import workloads as W
    from oracle import attention as A
    from oracle import kvquant as KQ
    from oracle.query import quantize_query
    ksi, qs, gk, gv = W.calibration(w)
    lens = W.seq_lens(w)
    D = w["d"]
    sc = W.softmax_scale(w)
    done_bytes, t_total, steps = 0.0, 0.0, 0
    with threadpool_limits(limits=cores):
        prepared = []
        for b in range(min(n_units, w["batch"], 2)):
            L = int(lens[b])
            lc, ls, _ = KQ.quantize_latent(W.keys(w, b, 0, L), ksi[0], gk[0], w["fmt"])
            lat = A.latent_dequant_exact(lc, ls, w["fmt"], 1.0)
            prepared.append((L, lat, W.rope_keys(w, b, L), W.queries(w, b), W.rope_queries(w, b)))
        while t_total < budget_s:
            for L, lat, kr, q, qr in prepared:
                t0 = time.perf_counter()
                qq = quantize_query(q, qs[0], w["fmt"])
                s = A.logits(qq, lat[:L], gk[0], A.logit_coeff(sc, D), w["fmt"],
                             rope=(qr, kr, A.logit_coeff(sc, 1)))
                out = A.attend(s, lat * gk[0], L, w["fmt"])["out"]
                _ = A.fwht_f64(out) / D * qs[0].astype(np.float64)[None, :]
                t_total += time.perf_counter() - t0
                done_bytes += L * kv_bytes_per_token_head(w)
                steps += 1
    one_bytes, t_one = 0.0, 0.0
    with threadpool_limits(limits=1):
        while t_one < budget_s / 3:
            L, lat, kr, q, qr = prepared[0]
            t0 = time.perf_counter()
            qq = quantize_query(q, qs[0], w["fmt"])
            s = A.logits(qq, lat[:L], gk[0], A.logit_coeff(sc, D), w["fmt"], rope=(qr, kr, A.logit_coeff(sc, 1)))
            out = A.attend(s, lat * gk[0], L, w["fmt"])["out"]
            _ = A.fwht_f64(out) / D * qs[0].astype(np.float64)[None, :]
            t_one += time.perf_counter() - t0
            one_bytes += L * kv_bytes_per_token_head(w)
    return {"value": round(done_bytes / t_total / 1e9, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "value_1_thread": round(one_bytes / t_one / 1e9, 5),
            "sample": "%d sequence decode steps (all %d query heads) over %d of the workload's %d sequences, "
                      "full context (%d tokens each); latent quantized once beforehand, untimed; %.1f s of "
                      "timed CPU work with %d BLAS threads, %.1f s with one" % (
                          steps, w["hq"], len(prepared), w["batch"], int(lens[0]), t_total, cores, t_one)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_4b")
    ap.add_argument("--copies", type=int, default=3, help="cache copies rotated between steps")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence per step (GQA; >1: causal multi-token decode, e.g. "
                         "speculative verification; the step appends that many tokens)")
    ap.add_argument("--cpu-units", type=int, default=8)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the BF16-KV comparison decode (GQA workloads)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="profiling mode: after setup, launch the decode kernel --steps times and one "
                         "1 GiB stream copy (the known-size reference for traffic counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from fp4_kv_cache_amd import workloads as W
    from fp4_kv_cache_amd import harness
    from fp4_kv_cache_amd import lib as L
    L.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.workload(args.workload)
    mla = w["attn"] == 1
    QN = args.q_len
    if QN > 1 and mla:
        print("--q-len > 1 is a GQA mode", file=sys.stderr)
        sys.exit(2)
    lens = W.seq_lens(w)
    B, hq, hkv, d, P = w["batch"], w["hq"], w["hkv"], w["d"], w["page"]
    log("workload", args.workload, "batch", B, "ctx", int(lens.max()), "fmt", "NVFP4" if w["fmt"] == 0 else "MXFP4")

    # prefill all but the last QN tokens of every sequence; each step appends them
    t0 = time.time()
    built = harness.build(w, lens=lens, stop=lens - QN, device=dev, workers=16)
    copies = [built.cache]
    for _ in range(1, args.copies):
        c2 = L.PagedFP4Cache(w["fmt"], w["attn"], built.cache.desc.num_pages, P, hkv, d, B, *built.calib[:2],
                             built.calib[2] if w["fmt"] == 0 else None,
                             built.calib[3] if (w["fmt"] == 0 and not mla) else None, rope_dim=w["rope"],
                             device=dev)
        for name in ("k_codes", "k_scales", "v_codes", "v_scales", "stage", "k_rope"):
            if getattr(built.cache, name, None) is not None:
                getattr(c2, name).copy_(getattr(built.cache, name))
        copies.append(c2)
    torch.cuda.synchronize()
    log("prefill + %d cache copies: %.1f s" % (len(copies), time.time() - t0))

    # the step's inputs: the last token of every sequence and the decode query
    last = (lens - 1).astype(np.int32)
    tdt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    kr_new = None
    if mla:   # the latent (as the key) and the bf16 rope key of each sequence's last token
        k_new = torch.from_numpy(np.stack([W.keys(w, b, 0, int(lens[b]))[-1:] for b in range(B)]))
        kr_new = torch.from_numpy(np.stack([W.bf16_bits(W.rope_keys(w, b, int(lens[b]))[-1])
                                            for b in range(B)]).view(np.int16)).to(dev)
        k_new, v_new = k_new.to(tdt).to(dev).contiguous(), None
    else:
        k_new = torch.from_numpy(np.concatenate([built.tail[b][0][:QN] for b in range(B)]))
        v_new = torch.from_numpy(np.concatenate([built.tail[b][1][:QN] for b in range(B)]))
        k_new, v_new = k_new.to(tdt).to(dev).contiguous(), v_new.to(tdt).to(dev).contiguous()
    newpos = np.concatenate([np.arange(int(lens[b]) - QN, int(lens[b])) for b in range(B)]).astype(np.int32)
    slots = torch.from_numpy(np.concatenate([harness.slots_for(built.bt_np[b], np.arange(int(lens[b]) - QN,
                                                                                         int(lens[b])), P)
                                             for b in range(B)]).astype(np.int32)).to(dev)
    seq_ids = torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), QN)).to(dev)
    pos = torch.from_numpy(newpos).to(dev)
    q1 = built.queries()
    q = built.queries_multi(QN) if QN > 1 else q1
    scale = W.softmax_scale(w)
    maxp = built.bt.shape[1]
    ws_bytes = L.fp4_decode_multi_workspace_bytes(copies[0].desc, B, QN, hq, maxp * P)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, QN, hq, d) if QN > 1 else (B, hq, d), dtype=torch.float32, device=dev)
    qdt = L.BF16 if q.dtype == torch.bfloat16 else L.F32
    stream = torch.cuda.current_stream().cuda_stream

    def cur_stream():
        return torch.cuda.current_stream().cuda_stream

    def decode_multi(i):
        c = copies[i % len(copies)]
        L.check(L.fp4_decode_attention_multi(c.desc, q.data_ptr(), qdt, B, QN, hq, built.bt.data_ptr(), maxp,
                                             built.seq_lens.data_ptr(), scale, out.data_ptr(), ws.data_ptr(),
                                             ws_bytes, None, cur_stream()), "fp4_decode_attention_multi")

    def step(i):
        c = copies[i % len(copies)]
        c.append(k_new, v_new, slots, seq_ids, pos, kr_new)
        if QN > 1:
            decode_multi(i)
            return
        L.check(L.fp4_decode_attention(c.desc, q.data_ptr(), qdt, B, hq, built.bt.data_ptr(), maxp,
                                       built.seq_lens.data_ptr(), scale, out.data_ptr(), ws.data_ptr(),
                                       ws_bytes, None, cur_stream()), "fp4_decode_attention")

    def partials(i):   # one query token (the newest): the single-token decode kernel
        c = copies[i % len(copies)]
        L.check(L.fp4_decode_partials(c.desc, q1.data_ptr(), qdt, B, hq, built.bt.data_ptr(), maxp,
                                      built.seq_lens.data_ptr(), scale, ws.data_ptr(), ws_bytes, None,
                                      cur_stream()), "fp4_decode_partials")

    out1 = out if QN == 1 else torch.empty((B, hq, d), dtype=torch.float32, device=dev)

    def merge(i):
        c = copies[i % len(copies)]
        L.check(L.fp4_decode_merge(c.desc, B, hq, maxp, built.seq_lens.data_ptr(), out1.data_ptr(),
                                   ws.data_ptr(), ws_bytes, cur_stream()), "fp4_decode_merge")

    def append(i):
        copies[i % len(copies)].append(k_new, v_new, slots, seq_ids, pos, kr_new)

    if args.kernel_only:
        stream = cur_stream()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        L.check(L.fp4kv_stream_copy(src.data_ptr(), dst.data_ptr(), 1 << 30, stream), "stream_copy")
        for i in range(args.steps):
            partials(i)
        torch.cuda.synchronize()
        log("kernel-only run done: %d decode launches, kv bytes per launch %d" % (args.steps,
            int(np.sum(lens.astype(np.float64)) * hkv * kv_bytes_per_token_head(w))))
        return

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # eager: every launch issued from Python
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_step_eager = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out).all().item(), "non-finite decode output"
    out_eager = out.clone()

    # The same work replayed from a HIP graph that holds exactly `steps` launch sequences
    # (rotating over the cache copies), which removes the host's launch overhead: the step time,
    # and each kernel alone back to back -- the kernel's average duration as a profiler's kernel
    # trace reports it.
    nc = len(copies)

    def graph_time(fn, n=None):
        n = args.steps if n is None else n
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        # untimed warm-up replays, at least ~30 ms of device time: the first milliseconds of
        # work after the host-side capture run at ramping clocks (the same graph timed first
        # measured ~10% slower than timed again later)
        t_w = time.time()
        while True:
            g.replay()
            torch.cuda.synchronize()
            if time.time() - t_w > 0.03:
                break
        t0, t1 = ev(), ev()
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n * 1e3, g

    step_us, g_step = graph_time(step)
    # every replay recomputes the same steps (appending the same token is idempotent): it must
    # reproduce the eager output bit for bit
    out.zero_()
    g_step.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, out_eager), "graph replay differs from the eager step"
    del g_step
    ms_step = step_us * 1e-3
    kv_bytes = float(np.sum(lens.astype(np.float64)) * hkv * kv_bytes_per_token_head(w))
    k_us, _ = graph_time(partials)
    m_us, _ = graph_time(merge)
    a_us, _ = graph_time(append)

    def decode(i):   # fp4_decode_attention alone: partials + merge
        c = copies[i % len(copies)]
        L.check(L.fp4_decode_attention(c.desc, q1.data_ptr(), qdt, B, hq, built.bt.data_ptr(), maxp,
                                       built.seq_lens.data_ptr(), scale, out1.data_ptr(), ws.data_ptr(),
                                       ws_bytes, None, cur_stream()), "fp4_decode_attention")
    d_us, _ = graph_time(decode)
    mq_us = graph_time(decode_multi)[0] if QN > 1 else None

    # measured streaming-read ceiling of this device (2 GiB, 16-byte non-temporal loads)
    stream = cur_stream()
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    for _ in range(2):
        L.check(L.fp4kv_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream), "stream_read")
    s0, s1 = ev(), ev()
    s0.record()
    for _ in range(10):
        L.check(L.fp4kv_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream), "stream_read")
    s1.record()
    torch.cuda.synchronize()
    stream_gbps = nbytes * 10 / (s0.elapsed_time(s1) * 1e-3) / 1e9
    del buf

    # the decode kernel's own reads without its arithmetic (same partition, pages and loads)
    pattern_gbps = None
    if not mla:
        nsink = L.fp4kv_cache_read_sink_words(copies[0].desc, B, hq, maxp * P)
        csink = torch.empty(max(nsink, 1), dtype=torch.int32, device=dev)

        def cache_read(i):
            c = copies[i % len(copies)]
            L.check(L.fp4kv_cache_read(c.desc, B, hq, built.bt.data_ptr(), maxp, built.seq_lens.data_ptr(),
                                       csink.data_ptr(), nsink, cur_stream()), "cache_read")
        r_us, _ = graph_time(cache_read)
        pattern_gbps = kv_bytes / (r_us * 1e-6) / 1e9

    # the same decode over a BF16 KV cache of the same workload (the pages' comparison system):
    # one cache copy suffices, its 512 B per token-head dwarf the 256 MB Infinity Cache
    bf16_cmp = None
    if not mla and QN == 1 and not args.no_bf16:
        t0 = time.time()
        del copies[1:]
        torch.cuda.empty_cache()
        b16 = harness.build_bf16(w, lens=lens, device=dev, workers=16)
        ws16_bytes = L.bf16_decode_workspace_bytes(b16.cache.desc, B, hq, maxp * P)
        ws16 = torch.empty(ws16_bytes, dtype=torch.uint8, device=dev)
        out16 = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
        log("bf16 cache: %.1f s" % (time.time() - t0))

        def decode_bf16(i):
            L.check(L.bf16_decode_attention(b16.cache.desc, q1.data_ptr(), qdt, B, hq, b16.bt.data_ptr(), maxp,
                                            b16.seq_lens.data_ptr(), scale, out16.data_ptr(), ws16.data_ptr(),
                                            ws16_bytes, cur_stream()), "bf16_decode_attention")
        b_us, _ = graph_time(decode_bf16)
        assert torch.isfinite(out16).all().item(), "non-finite bf16 decode output"
        bf16_bytes = float(np.sum(lens.astype(np.float64))) * hkv * 2 * d * 2
        bf16_cmp = {"decode_attention_us": round(b_us, 2), "kv_bytes_per_step": int(bf16_bytes),
                    "kv_GBps": round(bf16_bytes / (b_us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(bf16_bytes / (b_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "fp4_decode_speedup": round(b_us / d_us, 3)}
        del b16, ws16, out16

    traffic = read_traffic(w, args.workload)
    if mla:   # matrix-core bound: algorithmic flops against the dense FP4 matrix peak
        flops = float(np.sum(lens.astype(np.float64))) * mla_flops_per_token(w)
        achieved = flops / (k_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP4_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP4_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                    "flops_per_launch": flops,
                    "kv_GBps": round(kv_bytes / (k_us * 1e-6) / 1e9, 1),
                    "kv_frac_of_hbm_peak": round(kv_bytes / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    else:
        # one query token: the partial kernel; several: the whole multi-token decode (partials and
        # merge, no separate entry point for its partials)
        achieved = kv_bytes / ((k_us if QN == 1 else mq_us) * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic if QN == 1 else None}
    res = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "us_per_step_eager_launches": round(ms_step_eager * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(e2m1) x fp4 -> f32",
        "data": "synthetic",
        "config": {"workload": ("%s: batch %d, %d query heads on one latent head (latent %d FP4 + rope %d bf16), "
                                "context %s, page %d, %s, shuffled page table, 1 new token per sequence per step"
                                % (args.workload, B, hq, d, w["rope"],
                                   int(lens.max()) if lens.min() == lens.max() else
                                   "%d-%d (ragged)" % (lens.min(), lens.max()), P,
                                   "NVFP4" if w["fmt"] == 0 else "MXFP4")) if mla else
                               ("%s: batch %d, %d query / %d KV heads, head_dim %d, context %s, page %d, %s K/V, "
                                "shuffled page table, %s"
                                % (args.workload, B, hq, hkv, d,
                                   int(lens.max()) if lens.min() == lens.max() else
                                   "%d-%d (ragged)" % (lens.min(), lens.max()), P,
                                   "NVFP4" if w["fmt"] == 0 else "MXFP4",
                                   "1 new token per sequence per step" if QN == 1 else
                                   "%d new tokens per sequence per step, all %d decoded (causal)" % (QN, QN))),
                   "global_batch": B, "seq_len": int(lens.max()), "kv_bytes_per_step": int(kv_bytes),
                   "cache_copies_rotated": nc},
        "roofline": roofline,
        "breakdown_us": {"decode_partials_kernel": round(k_us, 2), "split_merge_kernel": round(m_us, 2),
                         "kv_append_1_token": round(a_us, 2)},
        # fp4_decode_attention alone (partials + merge, one launch after the other)
        "decode_attention": {"us": round(d_us, 2), "kv_GBps": round(kv_bytes / (d_us * 1e-6) / 1e9, 1),
                             "frac_of_hbm_peak": round(kv_bytes / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
        "stream_read_ceiling_GBps": round(stream_gbps, 1),
        **({"bf16_kv_comparison": bf16_cmp} if bf16_cmp else {}),
        **({"multi_token": {"q_len": QN, "decode_us": round(mq_us, 2),
                            "single_token_decode_us": round(k_us + m_us, 2),
                            "query_tokens_per_s": round(B * QN / (mq_us * 1e-6), 1),
                            "vs_separate_single_token_decodes": round(QN * (k_us + m_us) / mq_us, 3)}}
           if QN > 1 else {}),
        "pattern_read_ceiling_GBps": round(pattern_gbps, 1) if pattern_gbps else None,
        "decode_kernel_hash": decode_kernel_hash(decode_kernel(w)),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_units, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
