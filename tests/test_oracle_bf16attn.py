"""Pins of oracle/bf16attn.py (the BF16-KV comparison path)."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import bf16attn as BA

F32 = np.float32


def test_bf16_rounding_is_the_library_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(50)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-20, 20, 100000))).astype(F32)
    # exact ties: a bf16 value plus half an ulp of bf16 (bit 15 set, lower bits clear)
    base = BA.bf16(rng.standard_normal(1000).astype(F32))
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(F32)
    for v in (x, ties, np.array([0.0, -0.0, 1.0, -1.5, 3.0e38], F32)):
        want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(BA.bf16(v), want)


def test_exact_probabilities_are_textbook_attention():
    rng = np.random.default_rng(51)
    for L in (1, 63, 64, 65, 300):
        q = rng.standard_normal((4, 128)).astype(F32)
        K = rng.standard_normal((L, 128)).astype(F32)
        V = rng.standard_normal((L, 128)).astype(F32)
        got = BA.bf16_attention(q, K, V, 1 / math.sqrt(128), p_mode="exact")
        ref = A.reference_attention(BA.bf16(q), BA.bf16(K), BA.bf16(V), 1 / math.sqrt(128))
        # fp32 logits and fp32 probabilities: relative error of order 1e-6
        assert np.max(A.row_rel_err(got, ref)) < 2e-6, L


def test_bf16_probabilities_within_the_rounding_bound():
    """Each weight p~ changes by at most 2^-9 of itself when rounded to bf16, so the output moves
    by at most 2^-9 * sum p~ |v| / sum p~ <= 2^-9 * max |v| (per channel)."""
    rng = np.random.default_rng(52)
    L = 1000
    q = rng.standard_normal((3, 128)).astype(F32)
    K = rng.standard_normal((L, 128)).astype(F32)
    V = rng.standard_normal((L, 128)).astype(F32)
    a = BA.bf16_attention(q, K, V, 0.2)
    b = BA.bf16_attention(q, K, V, 0.2, p_mode="exact")
    bound = 2.0 ** -9 * np.max(np.abs(BA.bf16(V)))
    assert np.max(np.abs(a - b)) <= bound
    assert np.max(np.abs(a - b)) > 0      # the rounding is applied


def test_tiny_contexts_match_a_per_token_loop():
    rng = np.random.default_rng(53)
    for L in (1, 2, 64, 65, 130):
        q = rng.standard_normal((2, 16)).astype(F32)
        K = rng.standard_normal((L, 16)).astype(F32)
        V = rng.standard_normal((L, 16)).astype(F32)
        got = BA.bf16_attention(q, K, V, 0.5)
        c = F32(F32(0.5) * F32(math.log2(math.e)))
        qb, Kb, Vb = BA.bf16(q), BA.bf16(K), BA.bf16(V)
        for r in range(2):
            ms, os_, ls = [], [], []
            for t0 in range(0, L, 64):
                toks = range(t0, min(L, t0 + 64))
                s = {t: F32(c * F32(sum(float(x) * float(y) for x, y in zip(qb[r], Kb[t])))) for t in toks}
                m = max(s.values())
                p = {t: F32(2.0 ** float(F32(s[t] - m))) for t in toks}
                o = sum(float(BA.bf16(np.array([p[t]], F32))[0]) * Vb[t].astype(np.float64) for t in toks)
                ms.append(float(m)); os_.append(o); ls.append(sum(float(p[t]) for t in toks))
            M = max(ms)
            w = [2.0 ** (x - M) for x in ms]
            ref = sum(wi * oi for wi, oi in zip(w, os_)) / sum(wi * li for wi, li in zip(w, ls))
            assert np.allclose(got[r], ref, rtol=1e-12, atol=1e-13), (L, r)
