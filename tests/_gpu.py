"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare."""
import sys

import numpy as np

from fp4_kv_cache_amd import workloads as W
from fp4_kv_cache_amd import harness
from oracle import attention as A
from oracle import kvquant as KQ
from oracle import layout as LY


# Loose bound on the GPU output's error against unquantized fp64 attention, taken over all
# compared rows together: ||O - O_ref||_F / ||O_ref||_F.  The method itself sits at 0.08-0.17
# (NVFP4) and 0.21-0.25 (MXFP4, lognormal magnitudes) on these workloads; a mistake shared by
# the kernel and the oracle (a lost smoothing factor, a wrong un-rotation, a value scale
# applied twice) lands near or far above 1.  Single rows are not bounded: a short context with
# near-tied logits can legitimately pick other tokens after quantization.
REF_BOUND = {W.NVFP4: 0.35, W.MXFP4: 0.5}


class _RefErr:
    """Accumulates ||O - O_ref||_F^2 and ||O_ref||_F^2 over the compared rows."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, ref):
        d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
        self.num += float(np.sum(d * d))
        self.den += float(np.sum(np.asarray(ref, np.float64) ** 2))

    def check(self, fmt, tag, bound=None):
        if self.den == 0.0:
            return 0.0
        bound = REF_BOUND[fmt] if bound is None else bound
        agg = (self.num / self.den) ** 0.5
        say("%s: error against fp64 attention over all rows %.3g (bound %.2g)" % (tag, agg, bound))
        assert agg <= bound, "%s: error %.3g against fp64 attention" % (tag, agg)
        return agg


# A row whose GPU output is off the oracle's by more than this has a quantization decision
# (a query or probability code) taken differently; fp32 summation order alone stays below.
FLIP_EPS = 1e-6


def _flip_report(tag, errs):
    errs = np.asarray(errs, np.float64).ravel()
    if errs.size:
        say("%s: %d of %d rows beyond %.0e of the oracle (code flips), max %.3g"
            % (tag, int(np.sum(errs > FLIP_EPS)), errs.size, FLIP_EPS, float(errs.max())))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cache_np(built):
    return {k: v.cpu().numpy() for k, v in built.cache.views().items()}


def check_gqa_cache(built, seqs=None, pairs=None, opts=None):
    """Cache bytes of the given sequences (or (sequence, KV head) pairs) == the oracle's
    one-shot quantization (bit exact); ``opts`` carries the oracle's search / rotate switches."""
    search = (opts or {}).get("search", True)
    rotate = (opts or {}).get("rotate", True)
    w = built.w
    ksi, qs, gk, gv = built.calib
    views = cache_np(built)
    if pairs is None:
        seqs = range(w["batch"]) if seqs is None else seqs
        pairs = [(b, h) for b in seqs for h in range(w["hkv"])]
    for b, h in pairs:
        L = int(built.lens[b])
        kc, ks, vc, vs = LY.gather_gqa(views, h, built.bt_np[b], L, w["fmt"])
        okc, oks = KQ.quantize_keys(W.keys(w, b, h, L), ksi[h], gk[h], w["fmt"], search, rotate)
        ovc, ovs = KQ.quantize_values(W.values(w, b, h, L), gv[h], w["fmt"])
        for name, got, exp in (("k_codes", kc, okc), ("k_scales", ks, oks),
                               ("v_codes", vc, ovc), ("v_scales", vs, ovs)):
            if not np.array_equal(got, exp):
                bad = np.argwhere(got != exp)
                raise AssertionError("seq %d head %d %s: %d mismatches, first at %s (got %s want %s)"
                                     % (b, h, name, len(bad), bad[0].tolist(), got[tuple(bad[0])],
                                        exp[tuple(bad[0])]))


def check_mla_cache(built, seqs=None, opts=None):
    """Latent codes, tile scales and rope bytes of the given sequences == the oracle's one-shot
    quantization (bit exact); ``opts`` carries the oracle's search / rotate switches."""
    search = (opts or {}).get("search", True)
    rotate = (opts or {}).get("rotate", True)
    w = built.w
    ksi, qs, gk, gv = built.calib
    views = cache_np(built)
    seqs = range(w["batch"]) if seqs is None else seqs
    for b in seqs:
        L = int(built.lens[b])
        lc, ls, kr = LY.gather_mla(views, built.bt_np[b], L, w["fmt"])
        olc, ols, _ = KQ.quantize_latent(W.keys(w, b, 0, L), ksi[0], gk[0], w["fmt"], search, rotate)
        okr = W.bf16_bits(W.rope_keys(w, b, L))
        for name, got, exp in (("latent codes", lc, olc), ("tile scales", ls, ols),
                               ("rope", kr.view(np.uint16), okr)):
            if not np.array_equal(got, exp):
                bad = np.argwhere(got != exp)
                raise AssertionError("seq %d %s: %d mismatches, first at %s" % (b, name, len(bad),
                                                                               bad[0].tolist()))


def gqa_oracle(built, b, kvh, qn, opts=None):
    w = built.w
    ksi, qs, gk, gv = built.calib
    g = w["hq"] // w["hkv"]
    L = int(built.lens[b])
    rows = qn[b, kvh * g:(kvh + 1) * g]
    K = W.keys(w, b, kvh, L)
    V = W.values(w, b, kvh, L)
    res = A.gqa_head(rows, K, V, ksi[kvh], qs[kvh], gk[kvh], gv[kvh], w["fmt"], W.softmax_scale(w),
                     L=L, opts=opts)
    res["ref"] = A.reference_attention(rows, K, V, W.softmax_scale(w)) if L else np.zeros_like(res["out"])
    return res


def run_decode(built, zero=True):
    import torch
    q = built.queries()
    zc = torch.zeros(1, dtype=torch.int32, device=built.device) if zero else None
    out = built.cache.decode(q, built.bt, built.seq_lens, W.softmax_scale(built.w), zero_block_count=zc)
    torch.cuda.synchronize()
    return q.float().cpu().numpy(), out.cpu().numpy(), (int(zc.item()) if zero else None)


def compare_gqa(built, pairs=None, tol=1e-3, opts=None, ref_bound=None):
    """GPU decode vs oracle on (seq, kv-head) pairs; returns (max err, max err vs fp64, zero counts).
    ``opts``: the oracle's technique switches; ``ref_bound`` overrides the aggregate bound
    against fp64 attention."""
    w = built.w
    g = w["hq"] // w["hkv"]
    qn, out, zgpu = run_decode(built)
    pairs = [(b, h) for b in range(w["batch"]) for h in range(w["hkv"])] if pairs is None else pairs
    worst, worst_ref, zor = 0.0, 0.0, 0
    rows = []
    agg = _RefErr()
    for b, h in pairs:
        res = gqa_oracle(built, b, h, qn, opts)
        got = out[b, h * g:(h + 1) * g]
        er_rows = A.row_rel_err(got, res["out"]) if built.lens[b] else np.abs(got).max(-1)
        rows.append(er_rows)
        e = float(np.max(er_rows))
        er = float(np.max(A.row_rel_err(got, res["ref"]))) if built.lens[b] else 0.0
        worst, worst_ref = max(worst, e), max(worst_ref, er)
        zor += res["zero_blocks"]
        assert np.all(np.isfinite(got)), (b, h)
        assert e <= tol, "seq %d kv head %d: max row error %.3g > %.1g" % (b, h, e, tol)
        if built.lens[b]:
            agg.add(got, res["ref"])
    _flip_report("gqa", np.concatenate(rows) if rows else [])
    compare_gqa.last_agg = agg.check(w["fmt"], "gqa", ref_bound)
    return worst, worst_ref, zgpu, zor


def compare_mla(built, seqs=None, tol=1e-3, ref_bound=None, opts=None):
    """GPU MLA decode vs oracle on the given sequences; returns (max err, max err vs fp64 attention).
    ``ref_bound`` overrides the aggregate bound against fp64 attention; ``opts``: the oracle's
    technique switches."""
    w = built.w
    ksi, qs, gk, gv = built.calib
    qn, out, zgpu = run_decode(built)
    seqs = range(w["batch"]) if seqs is None else seqs
    worst, worst_ref = 0.0, 0.0
    sc = W.softmax_scale(w)
    D = w["d"]
    rows = []
    agg = _RefErr()
    compare_mla.last_zero_oracle = 0
    for b in seqs:
        L = int(built.lens[b])
        got = out[b]
        assert np.all(np.isfinite(got)), b
        if L == 0:
            worst = max(worst, float(np.abs(got).max()))
            continue
        K = W.keys(w, b, 0, L)
        kr = W.rope_keys(w, b, L)
        res = A.mla_seq(qn[b, :, :D], qn[b, :, D:], K, kr, ksi[0], qs[0], gk[0], w["fmt"], sc, L=L, opts=opts)
        compare_mla.last_zero_oracle += res["zero_blocks"]
        ref = A.reference_attention(qn[b, :, :D], K, K, sc, q_rope=qn[b, :, D:], k_rope=kr)
        er_rows = A.row_rel_err(got, res["out"])
        rows.append(er_rows)
        e = float(np.max(er_rows))
        er = float(np.max(A.row_rel_err(got, ref)))
        worst, worst_ref = max(worst, e), max(worst_ref, er)
        assert e <= tol, "seq %d: max row error %.3g > %.1g" % (b, e, tol)
        agg.add(got, ref)
    _flip_report("mla", np.concatenate(rows) if rows else [])
    compare_mla.last_agg = agg.check(w["fmt"], "mla", ref_bound)
    return worst, worst_ref, zgpu


def compare_gqa_multi(built, n, pairs=None, tol=1e-3):
    """Multi-token decode (n newest tokens per sequence, causal) vs the oracle's stacked-row
    pipeline on (sequence, KV head) pairs; returns (max err, max err vs fp64 attention)."""
    import torch
    w = built.w
    g = w["hq"] // w["hkv"]
    ksi, qs, gk, gv = built.calib
    q = built.queries_multi(n)
    zc = torch.zeros(1, dtype=torch.int32, device=built.device)
    out = built.cache.decode_multi(q, built.bt, built.seq_lens, W.softmax_scale(w), zero_block_count=zc)
    torch.cuda.synchronize()
    qn, out = q.float().cpu().numpy(), out.cpu().numpy()
    pairs = [(b, h) for b in range(w["batch"]) for h in range(w["hkv"])] if pairs is None else pairs
    worst, worst_ref, zor = 0.0, 0.0, 0
    sc = W.softmax_scale(w)
    rows = []
    agg = _RefErr()
    for b, h in pairs:
        L = int(built.lens[b])
        got = out[b, :, h * g:(h + 1) * g]
        assert np.all(np.isfinite(got)), (b, h)
        if L == 0:
            worst = max(worst, float(np.abs(got).max()))
            continue
        K = W.keys(w, b, h, L)
        V = W.values(w, b, h, L)
        qrows = qn[b, :, h * g:(h + 1) * g]
        res = A.gqa_head_multi(qrows, K, V, ksi[h], qs[h], gk[h], gv[h], w["fmt"], sc, L=L)
        zor += res["zero_blocks"]
        for j in range(n):
            er_rows = A.row_rel_err(got[j], res["out"][j])
            rows.append(er_rows)
            e = float(np.max(er_rows))
            ref = A.reference_attention(qrows[j], K[:L - n + 1 + j], V[:L - n + 1 + j], sc)
            er = float(np.max(A.row_rel_err(got[j], ref)))
            worst = max(worst, e)
            worst_ref = max(worst_ref, er)
            assert e <= tol, "seq %d kv head %d token %d: max row error %.3g > %.1g" % (b, h, j, e, tol)
            agg.add(got[j], ref)
    _flip_report("gqa multi-token", np.concatenate(rows) if rows else [])
    agg.check(w["fmt"], "gqa multi-token")
    return worst, worst_ref, int(zc.item()), zor

