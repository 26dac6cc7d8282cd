"""Seeded synthetic decode workloads (inputs only).

This module is shared by the product-side benchmark and by the tests that
drive the CPU oracle, so it holds random draws, shapes, page tables and the
static calibration statistics only -- none of the quantization, rotation or
attention arithmetic.  It needs numpy, not torch.

Every tensor chunk is drawn from its own counter-based stream,
``Philox(SeedSequence([workload id, tensor id, seq, head]))``, so any
(sequence, head) slice can be regenerated on its own, in any order, and the
first n tokens of a sequence do not depend on how many tokens are drawn.

Workloads (shapes of Qwen3-4B, Qwen3-30B-A3B and an MLA model; the pages'
serving runs used those models, and their evaluation data is not available,
so these synthetic batches stand in for them):

  tiny            B=1,  Hq=8,   Hkv=2, d=128, L=4096,          page 16, NVFP4, fp32
                  K channels 3,17,64,100 scaled x12
  qwen3_4b        B=16, Hq=32,  Hkv=8, d=128, L=32768,         page 64, NVFP4, bf16,
                  shuffled page table, 3 seeded key channels per head x10
  qwen3_30b_a3b   B=64, Hq=32,  Hkv=4, d=128, L~U[1024,65536], page 64, MXFP4, bf16,
                  K, V ~ N(0,1) * lognormal(0, 0.5) per (token, head)
  long_underflow  B=4,  Hq=32,  Hkv=8, d=128, L=131072,        page 64, NVFP4, bf16,
                  K ~ N(0, 0.05^2): nearly flat logits, probabilities ~1e-5
  mla             B=32, Hq=128, one latent head, D=512 + rope 64, L=16384, page 64,
                  NVFP4, bf16, 10 seeded latent channels x8
  mla_ragged      as mla with L ~ U[1024, 32768]
  mla_mxfp4       as mla with an MXFP4 latent
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

NVFP4 = 0
MXFP4 = 1
GQA = 0
MLA = 1

WORKLOADS = {
    "tiny": dict(id=1, attn=GQA, batch=1, hq=8, hkv=2, d=128, rope=0, ctx=4096, page=16,
                 fmt=NVFP4, dtype="f32", shuffle=False, outlier_channels=(3, 17, 64, 100),
                 outlier_scale=12.0, n_outliers=0, k_std=1.0, lognormal=0.0),
    "qwen3_4b": dict(id=2, attn=GQA, batch=16, hq=32, hkv=8, d=128, rope=0, ctx=32768, page=64,
                     fmt=NVFP4, dtype="bf16", shuffle=True, outlier_channels=None,
                     outlier_scale=10.0, n_outliers=3, k_std=1.0, lognormal=0.0),
    "qwen3_30b_a3b": dict(id=3, attn=GQA, batch=64, hq=32, hkv=4, d=128, rope=0,
                          ctx=(1024, 65536), page=64, fmt=MXFP4, dtype="bf16", shuffle=True,
                          outlier_channels=None, outlier_scale=1.0, n_outliers=0, k_std=1.0,
                          lognormal=0.5),
    "long_underflow": dict(id=4, attn=GQA, batch=4, hq=32, hkv=8, d=128, rope=0, ctx=131072,
                           page=64, fmt=NVFP4, dtype="bf16", shuffle=True, outlier_channels=None,
                           outlier_scale=1.0, n_outliers=0, k_std=0.05, lognormal=0.0),
    "mla": dict(id=5, attn=MLA, batch=32, hq=128, hkv=1, d=512, rope=64, ctx=16384, page=64,
                fmt=NVFP4, dtype="bf16", shuffle=True, outlier_channels=None, outlier_scale=8.0,
                n_outliers=10, k_std=1.0, lognormal=0.0),
    # the MLA shape with ragged contexts (uniform in [1024, 32768], mean close to the uniform
    # batch's 16384): the balanced partition's per-token rate against the uniform batch's
    "mla_ragged": dict(id=7, attn=MLA, batch=32, hq=128, hkv=1, d=512, rope=64, ctx=(1024, 32768), page=64,
                       fmt=NVFP4, dtype="bf16", shuffle=True, outlier_channels=None, outlier_scale=8.0,
                       n_outliers=10, k_std=1.0, lognormal=0.0),
    # the MLA shape with an MXFP4 latent (32 x 32 E8M0 tiles); not one of the five headline
    # configurations -- it exercises the natively block-scaled MLA path
    "mla_mxfp4": dict(id=6, attn=MLA, batch=32, hq=128, hkv=1, d=512, rope=64, ctx=16384, page=64,
                      fmt=MXFP4, dtype="bf16", shuffle=True, outlier_channels=None, outlier_scale=8.0,
                      n_outliers=10, k_std=1.0, lognormal=0.0),
}

T_Q, T_K, T_V, T_KROPE, T_QROPE, T_LEN, T_PAGES, T_OUTL, T_KMAG, T_VMAG = range(1, 11)


def workload(name, **over):
    """A copy of a named workload's parameters with overrides (e.g. batch=2, ctx=300)."""
    w = dict(WORKLOADS[name])
    w.update(over)
    w["name"] = name
    return w


def _rng(w, tensor, *idx):
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([w["id"], tensor, *idx])))


def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x):
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _cast(w, x):
    return bf16_round(x) if w["dtype"] == "bf16" else np.asarray(x, np.float32)


def seq_lens(w):
    ctx = w["ctx"]
    if isinstance(ctx, tuple):
        return _rng(w, T_LEN).integers(ctx[0], ctx[1] + 1, size=w["batch"]).astype(np.int32)
    return np.full(w["batch"], ctx, dtype=np.int32)


def page_table(w, lens=None, copy=0):
    """(block_table int32 [B, max_pages], num_pages).  Pages are shuffled when the workload says so.

    ``copy`` selects an independent permutation (used to build rotating cache copies).
    Unused entries hold 0, a valid page id.
    """
    lens = seq_lens(w) if lens is None else lens
    P = w["page"]
    npg = [-(-int(L) // P) for L in lens]
    total = int(sum(npg))
    ids = np.arange(total, dtype=np.int32)
    if w["shuffle"]:
        ids = _rng(w, T_PAGES, copy).permutation(total).astype(np.int32)
    maxp = max(npg) if npg else 0
    bt = np.zeros((len(lens), max(maxp, 1)), dtype=np.int32)
    o = 0
    for b, n in enumerate(npg):
        bt[b, :n] = ids[o:o + n]
        o += n
    return bt, total


def outlier_channels(w, h):
    if w["outlier_channels"] is not None:
        return np.array(w["outlier_channels"], dtype=np.int64)
    if w["n_outliers"] == 0:
        return np.zeros(0, dtype=np.int64)
    return _rng(w, T_OUTL, h).choice(w["d"], size=w["n_outliers"], replace=False)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def special_rows(w, x, b):
    """With w["degenerate"], token rows of special values replace drawn rows of x [L, d], by
    token index t % 8: 0 zeros, 1 negative zeros, 2 the constant 0.75, 3 E2M1 grid values
    times powers of two 2^-2 .. 2^2 with mixed signs, 4 a drawn row with one element set to
    1000; other rows stay as drawn.  Deterministic in (t, channel), so a slice of a sequence
    regenerates on its own.  w["seq_scales"] (optional, one power of two per sequence)
    multiplies sequence b's rows, e.g. far beyond the calibration statistics of sequence 0."""
    sc = w.get("seq_scales")
    if sc is not None:
        x = x * np.float32(sc[b])
    if not w.get("degenerate"):
        return x
    x = np.array(x, dtype=np.float32, copy=True)
    L, d = x.shape
    t = np.arange(L)
    c = np.arange(d)
    r = t % 8
    x[r == 0] = 0.0
    x[r == 1] = -0.0
    x[r == 2] = 0.75
    t3 = t[r == 3][:, None]
    sign = np.where((t3 + c[None, :]) % 3 == 0, -1.0, 1.0).astype(np.float32)
    x[r == 3] = E2M1_GRID[(t3 + c[None, :]) % 8] * np.exp2((c % 5) - 2).astype(np.float32)[None, :] * sign
    t4 = t[r == 4]
    x[t4, (7 * t4) % d] = 1000.0
    return x


def keys(w, b, h, L):
    """K[b, :L, h, :] as float32 (bf16-rounded for bf16 workloads).  For MLA: the latent."""
    k = _rng(w, T_K, b, h).standard_normal((L, w["d"]), dtype=np.float32) * np.float32(w["k_std"])
    if w["lognormal"]:
        k *= np.exp(_rng(w, T_KMAG, b, h).normal(0.0, w["lognormal"], size=(L, 1))).astype(np.float32)
    ch = outlier_channels(w, h)
    if len(ch):
        k[:, ch] *= np.float32(w["outlier_scale"])
    return _cast(w, special_rows(w, k, b))


def values(w, b, h, L):
    v = _rng(w, T_V, b, h).standard_normal((L, w["d"]), dtype=np.float32)
    if w["lognormal"]:
        v *= np.exp(_rng(w, T_VMAG, b, h).normal(0.0, w["lognormal"], size=(L, 1))).astype(np.float32)
    return _cast(w, special_rows(w, v, b))


def queries(w, b):
    """Q[b] as float32 [Hq, d] (MLA: the latent query [Hq, 512])."""
    return _cast(w, _rng(w, T_Q, b).standard_normal((w["hq"], w["d"]), dtype=np.float32))


def queries_multi(w, b, n):
    """Queries of the n newest tokens of sequence b, float32 [n, Hq, d] (token n - 1 is the
    one ``queries`` draws)."""
    rows = [_cast(w, _rng(w, T_Q, b, 1 + j).standard_normal((w["hq"], w["d"]), dtype=np.float32))
            for j in range(n - 1)]
    return np.stack(rows + [queries(w, b)])


def rope_keys(w, b, L):
    return bf16_round(_rng(w, T_KROPE, b).standard_normal((L, w["rope"]), dtype=np.float32))


def rope_queries(w, b):
    return bf16_round(_rng(w, T_QROPE, b).standard_normal((w["hq"], w["rope"]), dtype=np.float32))


def softmax_scale(w):
    return 1.0 / math.sqrt(w["d"] + w["rope"])


def calibration(w, n_cal=1024):
    """Static per-KV-head calibration: (k_smooth_inv [Hkv, d], q_smooth [Hkv, d], G_K [Hkv], G_V [Hkv]).

    Smoothing: lambda_c = 2^round(0.5 * log2(amax_c(K) / amax_c(Q))) over the
    first ``n_cal`` tokens of sequence 0 and its query (powers of two, so
    q_smooth * k_smooth_inv == 1 exactly).  Tensor scales (NVFP4 only, 1.0
    for MXFP4) come from second moments, with no transform applied: the
    rotated key element is a +-1 sum over channels, so its standard deviation
    is sqrt(sum_c var(K_c / lambda_c)); G_K = 8 * that / 2688 and
    G_V = 8 * max_c rms(V_c) / 2688, which keeps every block scale inside the
    E4M3 range for 8-sigma blocks.
    """
    hkv, d = w["hkv"], w["d"]
    L = min(n_cal, seq_lens(w)[0])
    ksi = np.ones((hkv, d), np.float32)
    qs = np.ones((hkv, d), np.float32)
    gk = np.ones(hkv, np.float32)
    gv = np.ones(hkv, np.float32)
    q = queries(w, 0)
    g = w["hq"] // hkv
    for h in range(hkv):
        k = keys(w, 0, h, L).astype(np.float64)
        qa = np.abs(q[h * g:(h + 1) * g]).max(0).astype(np.float64)
        ka = np.abs(k).max(0)
        lam = np.exp2(np.round(0.5 * np.log2(np.maximum(ka, 1e-30) / np.maximum(qa, 1e-30))))
        lam = np.clip(lam, 2.0 ** -20, 2.0 ** 20)
        ksi[h] = (1.0 / lam).astype(np.float32)
        qs[h] = lam.astype(np.float32)
        if w["fmt"] == NVFP4:
            sd = math.sqrt(float(np.sum(np.mean(k * k, axis=0) / (lam * lam))))
            gk[h] = np.float32(8.0 * sd / 2688.0)
            if w["attn"] == GQA:
                v = values(w, 0, h, L).astype(np.float64)
                gv[h] = np.float32(8.0 * float(np.sqrt(np.mean(v * v, axis=0)).max()) / 2688.0)
    return ksi, qs, gk, gv


def parallel_map(fn, items, workers=8):
    """Run fn over items in a thread pool (numpy's generators release the GIL)."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))
