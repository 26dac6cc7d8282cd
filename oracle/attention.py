"""Decode-attention emulation over the FP4 cache, split-K merge, and the unquantized reference.

Test infrastructure only (see ``oracle/__init__``).

What the pages fix ([Abstract]; [Blog/New]; [Explainer/Analyse]; the
system-level paragraph of [Explainer/Analyse] after the three algorithmic
parts): attention runs natively in FP4 on a paged cache; the query is the
dual-residual pair; the softmax is computed transposed with the probability
quantization fused into it (no trip to memory); stacked query rows share one
K/V tile load; probabilities are scaled so that E4M3 block scales do not
round long-context probabilities to zero (Underflow-Aware Probability
Scaling).  The split-K merge is standard flash-decoding arithmetic that the
pages do not spell out.

Readings:
* R1/R2  Probabilities are quantized tile-relative: per query row and per
         tile of 128 tokens aligned at token 0, m = max s over the tile,
         p~ = 2^(s - m) (so the tile maximum is exactly 1) and P = p~ is
         quantized with tensor scale G_P = 2^-10 and power-of-two E4M3 block
         scales of 16 tokens (NVFP4, ceil rule R-P2), or with MX E8M0 scales
         of 32 tokens (MXFP4).  Mapping the tile maximum near the top of the
         E4M3 range is the underflow-aware scaling: a block only loses its
         scale when all its p~ are below 2^-19 of the tile maximum.
* R3     The softmax denominator sums the unquantized fp32 p~.
* R11    Logits work in base 2: s = fl32(fl32(a1*raw1) + fl32(a2*raw2)) with
         a_k = fl32(fl32(G_Qk * G_K) * c) and raw_k = fl32(<q^_k, k^>): the dot
         of the exact block-scaled values (codes times block scales, no tensor
         scale) rounded once to fp32, for both formats.  It is formed in
         float64; every product is exact there and the float64 sum's own
         rounding (relative 2^-53 per add) lies far below the fp32 rounding
         that follows, so raw is the correctly rounded fp32 dot except where
         the exact dot sits within ~2^-45 of an fp32 rounding midpoint.
         c = fl32(softmax_scale * fl32(log2(e) / n)), n = head_dim when the
         rotation is on (1 otherwise).  MLA adds fl32(c_r * raw_rope) with
         c_r = fl32(softmax_scale * fl32(log2 e)).
* Decision precision: s, the tile maximum and p~ are fp32 values, as in the
         kernel; p~ = fl32(2^fl32(s - m)) is taken correctly rounded here.
         The kernel's hardware exp2 may differ in the last bit, so a P code
         can differ where p~ sits within an ulp of an E2M1 rounding boundary.
         The pages fix no precision for p~, so it takes the kernel's: an fp32
         value in the normal range, a result below 2^-126 being 0 (the
         hardware exp2 returns no subnormals).  Only MXFP4 P codes can tell
         (NVFP4's power-of-two P block scales stop at 2^-19, below which every
         p~ quantizes to 0 anyway): a block whose largest p~ lies in
         (2^-129, 2^-126) keeps nonzero E8M0-scaled codes with subnormal p~ and
         none without; its weight in the output is below 2^-126 of the tile
         maximum's.
* Merge  M = max_tau m_tau, out = sum 2^(m_tau - M) o_tau / sum 2^(m_tau - M) l_tau
         (float64 here).

Pins (tests/test_oracle_attention.py): with an identity codec the emulation
equals textbook softmax attention; any split of the tiles merged with
``merge_partials`` equals the one-shot result; tiny contexts (1, 2, 15, 16,
17, 127, 128, 129, 300) match an explicit per-token loop; on the
long-context flat-logit workload the tile-relative P has no all-zero block
while vanilla normalised P with G = 1 loses every block (closed form:
1/L / 6 < 2^-10).
"""
import numpy as np

from .codecs import e2m1_decode, e4m3_decode, e8m0_decode, mx_shared_exp
from .blockfmt import (NV_BLOCK, MX_BLOCK, p2_block_exp, p2_encode, p2_dequant_exact,
                       mx_encode, mx_dequant_exact, nvfp4_default_scale, nvfp4_encode,
                       nvfp4_dequant_exact)
from .kvquant import NVFP4, block_size, quantize_keys, quantize_values, quantize_latent
from .query import quantize_query
from .transforms import fwht_f32

F32 = np.float32
LOG2E = 1.4426950408889634
P_TILE = 128
GP_EXP = -10
GP = F32(2.0 ** GP_EXP)


def logit_coeff(softmax_scale, n):
    """c = fl32(softmax_scale * fl32(log2(e) / n))  (R11)."""
    return F32(F32(softmax_scale) * F32(LOG2E / n))


def key_dequant_exact(codes, scales, fmt):
    """Block-scaled key values without G (float64): dec(code) * S[token, block]."""
    L, d = codes.shape
    B = block_size(fmt)
    S = e4m3_decode(scales) if fmt == NVFP4 else e8m0_decode(scales)
    return (e2m1_decode(codes).reshape(L, d // B, B) * S[..., None]).reshape(L, d)


def value_dequant_exact(codes_tm, scales, fmt, G=1.0):
    """Token-major value codes [Lpad, d] with channel-wise token-block scales [d, Lpad/B] -> float64."""
    Lp, d = codes_tm.shape
    B = block_size(fmt)
    S = e4m3_decode(scales) if fmt == NVFP4 else e8m0_decode(scales)     # [d, nblk]
    dec = e2m1_decode(codes_tm).reshape(Lp // B, B, d)                   # [nblk, B, d]
    return (dec * S.T[:, None, :]).reshape(Lp, d) * float(G)


def latent_dequant_exact(codes_tm, tile_scales, fmt, G=1.0):
    """MLA latent codes [Lpad, D] with 2-D tile scales [Lpad/B, D/B] -> float64 (with G)."""
    Lp, D = codes_tm.shape
    B = block_size(fmt)
    S = e4m3_decode(tile_scales) if fmt == NVFP4 else e8m0_decode(tile_scales)
    dec = e2m1_decode(codes_tm).reshape(Lp // B, B, D // B, B)
    return (dec * S[:, None, :, None]).reshape(Lp, D) * float(G)


def logits(qq, khat, G_K, cs, fmt, rope=None):
    """Base-2 logits s [R, L] (fp32) from a QuantQuery and exact block-scaled keys (R11).

    ``rope`` = (q_rope [R, r], k_rope [L, r], c_r) adds the unquantized MLA rope term.
    """
    gk = F32(G_K) if fmt == NVFP4 else F32(1.0)
    raw1 = raw_dot(qq.dequant_exact(1), khat)
    raw2 = raw_dot(qq.dequant_exact(2), khat)
    a1 = ((qq.G1.astype(F32) * gk).astype(F32) * cs).astype(F32)
    a2 = ((qq.G2.astype(F32) * gk).astype(F32) * cs).astype(F32)
    s = ((a1[:, None] * raw1).astype(F32) + (a2[:, None] * raw2).astype(F32)).astype(F32)
    if rope is not None:
        qr, kr, cr = rope
        rawr = (np.asarray(qr, np.float64) @ np.asarray(kr, np.float64).T).astype(F32)
        s = (s + (F32(cr) * rawr).astype(F32)).astype(F32)
    return s


def raw_dot(qhat, khat):
    """raw [R, L] = fl32(<qhat_r, khat_t>): exact block-scaled values (float64) dotted and
    rounded once to fp32 (R11)."""
    return (np.asarray(qhat, np.float64) @ np.asarray(khat, np.float64).T).astype(F32)


def quantize_probs(pt, fmt, mode="tile"):
    """Quantize probabilities pt [R, Ltot] per (row, token block).

    Returns (Phat float64 [R, Ltot], codes [R, nblk, B]).
    mode 'tile': R1 (power-of-two NVFP4 with G_P = 2^-10, or MX).
    mode 'vanilla': default-scale NVFP4 with G = 1 (general E4M3), or MX.
    """
    R, Lt = pt.shape
    B = NV_BLOCK if fmt == NVFP4 else MX_BLOCK
    pb = pt.reshape(R, Lt // B, B)
    amax = np.max(pb, axis=-1)
    if fmt == NVFP4 and mode == "tile":
        e, valid = p2_block_exp(amax, GP)
        codes, _ = p2_encode(pb, e, valid, GP)
        ph = p2_dequant_exact(codes, e, valid) * float(GP)
    elif fmt == NVFP4:
        c = nvfp4_default_scale(amax, F32(1.0))
        codes = nvfp4_encode(pb, c, F32(1.0))
        ph = nvfp4_dequant_exact(codes, c)
    else:
        e = mx_shared_exp(amax)
        codes = mx_encode(pb, e)
        ph = mx_dequant_exact(codes, e)
    return ph.reshape(R, Lt), codes


def p_tilde_fp32(x):
    """p~ = 2^x (x <= 0, or -inf) as fp32 in the normal range: correctly rounded, and 0 where
    the result lies below 2^-126 (decision precision reading in the module header)."""
    p = np.exp2(np.asarray(x, np.float64)).astype(F32)
    return np.where(p < F32(2.0 ** -126), F32(0.0), p).astype(F32)


def attend(s, vhat, L, fmt, tile=P_TILE, p_mode="tile", partials=False, row_len=None):
    """Tile-wise FP4 softmax.V emulation for rows s [R, L] (fp32 base-2 logits).

    vhat: float64 [>=L, d] dequantized values (with G_V).  ``row_len`` (optional, [R],
    each in 1..L) limits row r to tokens < row_len[r] (causal multi-token decode); a
    tile with no valid token for a row contributes nothing to it.  Returns a dict with
    'out' [R, d] (float64), 'zero_blocks' (count of P blocks that hold at least
    one valid token and quantize to all zeros) and, if ``partials``, the
    per-tile (o, m, l).
    """
    s = np.asarray(s, F32)
    R = s.shape[0]
    d = vhat.shape[1]
    B = NV_BLOCK if fmt == NVFP4 else MX_BLOCK
    if L == 0:
        return {"out": np.zeros((R, d)), "zero_blocks": 0}
    T = -(-L // tile)
    Lt = T * tile
    sp = np.full((R, Lt), -np.inf, dtype=F32)
    sp[:, :L] = s[:, :L]
    rl = np.full(R, L, dtype=np.int64) if row_len is None else np.asarray(row_len, np.int64)
    for r in range(R):
        sp[r, rl[r]:] = -np.inf
    vp = np.zeros((Lt, d))
    vp[:L] = vhat[:L]
    nvalid_blk = -(-rl // B)                  # [R]: blocks holding a valid token of the row
    blk_valid = np.arange(Lt // B)[None, :] < nvalid_blk[:, None]
    if p_mode == "vanilla":
        M = np.max(sp, axis=-1).astype(np.float64)
        p = np.exp2(sp.astype(np.float64) - M[:, None])
        p = (p / p.sum(-1, keepdims=True)).astype(F32)
        ph, codes = quantize_probs(p, fmt, "vanilla")
        zero = int(np.sum(np.all((codes & 7) == 0, axis=-1) & blk_valid))
        return {"out": ph @ vp, "zero_blocks": zero}
    m = np.max(sp.reshape(R, T, tile), axis=-1)                          # fp32 [R, T]
    live = np.isfinite(m)                     # the tile holds a valid token of the row
    diff = np.where(live[..., None], sp.reshape(R, T, tile) - np.where(live, m, 0)[..., None],
                    -np.inf).astype(F32)
    pt = p_tilde_fp32(diff).reshape(R, Lt)
    if p_mode == "exact":                     # identity codec on P (ablation / skeleton check)
        ph, codes, zero = pt.astype(np.float64), None, 0
    else:
        ph, codes = quantize_probs(pt, fmt, "tile")
        zero = int(np.sum(np.all((codes & 7) == 0, axis=-1) & blk_valid))
    o_t = np.einsum("rtk,tkd->rtd", ph.reshape(R, T, tile), vp.reshape(T, tile, d))
    l_t = pt.reshape(R, T, tile).astype(np.float64).sum(-1)
    out = merge_partials(o_t, m.astype(np.float64), l_t)
    res = {"out": out, "zero_blocks": zero}
    if partials:
        res.update(o_tiles=o_t, m_tiles=m, l_tiles=l_t, p_codes=codes, p_tilde=pt)
    return res


def merge_partials(o, m, l):
    """Split-K merge over axis 1: o [R, S, d], m [R, S] (base-2), l [R, S] -> [R, d].

    M = max m_s, w_s = 2^(m_s - M); out = sum w_s o_s / sum w_s l_s.  Splits
    with m = -inf (no tokens) get weight 0.  Rows with no tokens give 0.
    """
    o = np.asarray(o, np.float64)
    m = np.asarray(m, np.float64)
    l = np.asarray(l, np.float64)
    M = np.max(m, axis=1)
    Ms = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(m), np.exp2(m - Ms[:, None]), 0.0)
    num = np.einsum("rs,rsd->rd", w, o)
    den = np.sum(w * l, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)
    return out


def fwht_f64(u):
    """Unnormalised Walsh-Hadamard transform in float64 (used to un-rotate MLA outputs)."""
    u = np.array(u, dtype=np.float64, copy=True)
    n = u.shape[-1]
    h = 1
    while h < n:
        v = u.reshape(u.shape[:-1] + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return u


# ------------------------------------------------------------------ pipelines

DEFAULT_OPTS = dict(dual=True, smooth=True, rotate=True, search=True, p_mode="tile")


def gqa_head(q_rows, K, V, k_smooth_inv, q_smooth, G_K, G_V, fmt, softmax_scale,
             L=None, opts=None, partials=False, row_len=None):
    """One (sequence, KV head): the g query rows against L tokens, whole pipeline.

    q_rows [g, d], K/V [>=L, d] as float32 (bf16 inputs converted exactly); ``row_len``
    (optional) limits each row to its own prefix (see ``attend``).
    Returns the ``attend`` dict plus the cache contents and the QuantQuery.
    """
    o = dict(DEFAULT_OPTS, **(opts or {}))
    K = np.asarray(K, F32)
    L = K.shape[0] if L is None else L
    d = K.shape[1]
    ones = np.ones(d, F32)
    ksi = k_smooth_inv if o["smooth"] else ones
    qs = q_smooth if o["smooth"] else ones
    kc, ks = quantize_keys(K[:L], ksi, G_K, fmt, o["search"], o["rotate"])
    vc, vs = quantize_values(np.asarray(V, F32)[:L], G_V, fmt)
    qq = quantize_query(q_rows, qs, fmt, o["dual"], o["rotate"])
    cs = logit_coeff(softmax_scale, d if o["rotate"] else 1)
    s = logits(qq, key_dequant_exact(kc, ks, fmt), G_K, cs, fmt)
    gv = G_V if fmt == NVFP4 else 1.0
    res = attend(s, value_dequant_exact(vc, vs, fmt, gv), L, fmt, p_mode=o["p_mode"],
                 partials=partials, row_len=row_len)
    res.update(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, qq=qq, s=s)
    return res


def gqa_head_multi(q, K, V, k_smooth_inv, q_smooth, G_K, G_V, fmt, softmax_scale, L=None, opts=None):
    """Multi-token decode of one (sequence, KV head): q [n, g, d] holds n consecutive query
    tokens (positions L - n .. L - 1, all already in the cache) of the g query heads; query j
    attends to tokens 0 .. L - n + j.  The n*g rows (row j*g + h) go through ``gqa_head``
    together -- one quantization of the cache, each row masked to its own prefix -- which
    is the stacked-query reading of several query tokens per sequence.
    Returns the ``gqa_head`` dict with 'out' reshaped to [n, g, d].
    """
    q = np.asarray(q, F32)
    n, g, d = q.shape
    K = np.asarray(K, F32)
    L = K.shape[0] if L is None else L
    row_len = np.repeat(L - n + 1 + np.arange(n), g)
    res = gqa_head(q.reshape(n * g, d), K, V, k_smooth_inv, q_smooth, G_K, G_V, fmt, softmax_scale,
                   L=L, opts=opts, row_len=row_len)
    res["out"] = res["out"].reshape(n, g, d)
    return res


def mla_seq(q_lat, q_rope, K_lat, k_rope, k_smooth_inv, q_smooth, G_K, fmt, softmax_scale,
            L=None, opts=None, partials=False):
    """One MLA sequence: R query heads against the shared latent (as key and value) plus rope.

    q_lat [R, D], q_rope [R, r] (bf16 values), K_lat [>=L, D], k_rope [>=L, r].
    The output is un-rotated and un-smoothed: out = (o'' H / D) * q_smooth.
    """
    o = dict(DEFAULT_OPTS, **(opts or {}))
    K_lat = np.asarray(K_lat, F32)
    L = K_lat.shape[0] if L is None else L
    D = K_lat.shape[1]
    ones = np.ones(D, F32)
    ksi = k_smooth_inv if o["smooth"] else ones
    qs = q_smooth if o["smooth"] else ones
    lc, ls, _ = quantize_latent(K_lat[:L], ksi, G_K, fmt, o["search"], o["rotate"])
    qq = quantize_query(q_lat, qs, fmt, o["dual"], o["rotate"])
    cs = logit_coeff(softmax_scale, D if o["rotate"] else 1)
    cr = logit_coeff(softmax_scale, 1)
    gk = G_K if fmt == NVFP4 else 1.0
    lat = latent_dequant_exact(lc, ls, fmt, 1.0)          # [Lpad, D]; rows >= L are padding
    s = logits(qq, lat[:L], G_K, cs, fmt, rope=(q_rope, np.asarray(k_rope, F32)[:L], cr))
    res = attend(s, lat * gk, L, fmt, p_mode=o["p_mode"], partials=partials)
    out = res["out"]
    if o["rotate"]:
        out = fwht_f64(out) / D
    res["out"] = out * np.asarray(qs, np.float64)[None, :]
    res.update(l_codes=lc, l_scales=ls, qq=qq, s=s)
    return res


def reference_attention(q, k, v, softmax_scale, q_rope=None, k_rope=None):
    """Unquantized softmax attention in float64 from the original inputs (the error yardstick)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    s = q @ k.T
    if q_rope is not None:
        s = s + np.asarray(q_rope, np.float64) @ np.asarray(k_rope, np.float64).T
    s = s * float(softmax_scale)
    s = s - s.max(-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(-1, keepdims=True)
    return p @ np.asarray(v, np.float64)


def row_rel_err(a, b):
    """max_c |a - b| / ||b||_2 per row (the output tolerance measure)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nrm = np.linalg.norm(b, axis=-1)
    return np.max(np.abs(a - b), axis=-1) / np.where(nrm > 0, nrm, 1.0)
