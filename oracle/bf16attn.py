"""Decode attention over a BF16 KV cache: the comparison system of the FP4 path.

Test infrastructure only (see ``oracle/__init__``).

The pages measure the FP4 KV cache against a BF16 KV cache ("FP4 KV Cache Done Right",
section "How good are the results, really?": the peak serving throughput gain over a BF16
KV cache; "BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System Co-Design",
Article Summary).  They do not describe the BF16 baseline's kernel; this is plain softmax
attention with the cache, the query and the probabilities held in bfloat16 and every sum in
fp32 or wider.

Readings (none of them is the method's; they fix the comparison kernel's arithmetic):
* B1  Keys, values and the query are rounded to bfloat16 (round to nearest, ties to even)
      once, on append and on load.
* B2  Logits in base 2: s = fl32(c * raw) with raw = fl32(<q, k>) (the exact dot of the
      bf16 values rounded once) and c = fl32(softmax_scale * fl32(log2 e)).
* B3  Softmax over tiles of 64 tokens aligned at token 0: m = max s over the tile,
      p~ = fl32(2^fl32(s - m)); the probabilities that multiply the values are
      bf16(p~); the denominator sums the fp32 p~ (as the FP4 path's R3).
* B4  Tiles merged as in ``attention.merge_partials``.

Pins (tests/test_oracle_bf16attn.py): the bf16 rounding equals torch's bfloat16 cast
(library routine) on random values and on exact ties; with the probabilities kept in
fp32 the result equals textbook softmax attention over the bf16 inputs; the bf16
probabilities move the output by at most 2^-8 of the largest |value| (closed-form bound);
tiny contexts match an explicit per-token loop.
"""
import numpy as np

from .attention import merge_partials

F32 = np.float32
LOG2E = 1.4426950408889634
TILE = 64


def bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(F32).reshape(x.shape)


def bf16_attention(q, K, V, softmax_scale, L=None, tile=TILE, p_mode="bf16"):
    """q [R, d], K/V [>=L, d] (any float) -> out [R, d] float64, per B1-B4.

    p_mode 'bf16' (the kernel's arithmetic) or 'exact' (probabilities kept in fp32).
    """
    K = np.asarray(K, F32)
    L = K.shape[0] if L is None else L
    qb = bf16(np.asarray(q, F32)).astype(np.float64)
    Kb = bf16(K[:L]).astype(np.float64)
    Vb = bf16(np.asarray(V, F32)[:L]).astype(np.float64)
    R, d = qb.shape
    if L == 0:
        return np.zeros((R, d))
    c = F32(F32(softmax_scale) * F32(LOG2E))
    raw = (qb @ Kb.T).astype(F32)
    s = (c * raw).astype(F32)
    T = -(-L // tile)
    o_t = np.zeros((R, T, d))
    m_t = np.zeros((R, T))
    l_t = np.zeros((R, T))
    for t in range(T):
        a, e = t * tile, min(L, t * tile + tile)
        st = s[:, a:e]
        m = np.max(st, axis=1)
        pt = np.exp2((st - m[:, None]).astype(F32).astype(np.float64)).astype(F32)
        pm = bf16(pt) if p_mode == "bf16" else pt
        o_t[:, t] = pm.astype(np.float64) @ Vb[a:e]
        m_t[:, t] = m
        l_t[:, t] = pt.astype(np.float64).sum(axis=1)
    return merge_partials(o_t, m_t, l_t)
