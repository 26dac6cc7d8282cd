"""Pins of oracle/blockfmt.py: hand-worked examples, closed-form bounds, exactness."""
import os

import numpy as np

from oracle import blockfmt as BF
from oracle import codecs as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _examples():
    ex = {}
    for line in open(os.path.join(GOLD, "block_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        kv = dict(p.split("=") for p in parts[1:])
        ex[parts[0]] = kv
    return ex


def test_nvfp4_hand_example():
    ex = _examples()["N1"]
    x = np.array([3, -1.5, 0.75, 0.125, 2.25, -3, 0, 1.25, 0.5, -0.25, 1.75, 2.5, 0.375, -0.625, 1, 2],
                 F32)
    G = F32(ex["G"])
    c0 = BF.nvfp4_default_scale(np.max(np.abs(x)), G)
    assert int(c0) == int(ex["scale"], 16)
    codes = BF.nvfp4_encode(x[None], np.array([c0]), G)[0]
    assert codes.tolist() == [int(c) for c in ex["codes"].split(",")]


def test_mxfp4_hand_examples():
    ex = _examples()
    for name, x in (("M1", [7.5, 1.0, -2.0] + [0.0] * 29), ("M2", [0.1875, -0.09375] + [0.0] * 30)):
        x = np.array(x, F32)
        e = C.mx_shared_exp(np.max(np.abs(x)))
        assert int(BF.mx_scale_code(e)) == int(ex[name]["scale"])
        codes = BF.mx_encode(x[None], np.array([e]))[0]
        assert codes.tolist() == [int(c) for c in ex[name]["codes"].split(",")]


def _half_step(y):
    """Half the E2M1 grid gap around |y| (the rounding error bound for |y| <= 6)."""
    a = np.abs(y)
    return np.where(a <= 2.0, 0.25, np.where(a <= 4.0, 0.5, 1.0))


def test_nvfp4_default_scale_bounds():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((20000, 16)) * np.exp(rng.normal(0, 2, (20000, 1)))).astype(F32)
    G = F32(0.01)
    amax = np.max(np.abs(x), -1)
    c0 = BF.nvfp4_default_scale(amax, G)
    codes = BF.nvfp4_encode(x, c0, G)
    S = C.e4m3_decode(c0)
    y = x.astype(np.float64) / (S * float(G))[:, None]
    deq = C.e2m1_decode(codes)
    ok = (c0 > 8) & (c0 < 0x7E)          # scale neither saturated nor subnormal
    assert ok.mean() > 0.5
    inr = np.abs(y) <= 6.0
    m = ok[:, None] & inr
    assert np.all(np.abs(y - deq)[m] <= _half_step(y)[m] * (1 + 1e-6) + 1e-12)
    # the block maximum lands on or near the top of the grid (E4M3 rounding of the scale
    # moves it by at most 1/16 relative)
    top = np.max(np.abs(y), -1)[ok]
    assert np.all((top > 6 * (1 - 1 / 15)) & (top < 6 * (1 + 1 / 15)))


def test_p2_ceil_rule_no_clipping():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((20000, 16)) * np.exp(rng.normal(0, 1.5, (20000, 1)))).astype(F32)
    G = (np.max(np.abs(x)) / F32(1536)).astype(F32)
    amax = np.max(np.abs(x), -1)
    e, valid = BF.p2_block_exp(amax, G)
    codes, sc = BF.p2_encode(x, e, valid, G)
    y = x.astype(np.float64) / (np.exp2(e.astype(np.float64)) * float(G))[:, None]
    inr = (e > BF.P2_EMIN)
    assert np.all(np.abs(y[inr]) <= 6.0 * (1 + 1e-6))                    # never clips
    top = np.max(np.abs(y), -1)[inr]
    assert np.all(top > 3.0 * (1 - 1e-6))                                # uses the upper octave
    assert np.all(C.e4m3_decode(sc[valid]) == np.exp2(e[valid]))         # the stored code is 2^e
    deq = BF.p2_dequant_exact(codes, e, valid) * float(G)
    assert np.all(np.abs(deq - x) <= _half_step(y) * np.exp2(e)[:, None] * float(G) * (1 + 1e-6))


def test_p2_invalid_and_extremes():
    e, v = BF.p2_block_exp(np.array([0.0, 1.0, 1e-30, 1e30], F32), F32(2.0 ** -10))
    assert v.tolist() == [False, True, True, True]
    assert e[1] == 8 and e[2] == -9 and e[3] == 8
    e, v = BF.p2_block_exp(np.array([1.0], F32), F32(0.0))
    assert not v[0]


def test_mx_rule_and_dequant_exact():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((5000, 32)) * np.exp(rng.normal(0, 3, (5000, 1)))).astype(F32)
    e = C.mx_shared_exp(np.max(np.abs(x), -1))
    codes = BF.mx_encode(x, e)
    deq32 = BF.mx_dequant_f32(codes, e)
    deq64 = BF.mx_dequant_exact(codes, e)
    assert np.array_equal(deq32.astype(np.float64), deq64)
    y = x.astype(np.float64) / np.exp2(e.astype(np.float64))[:, None]
    sat = np.abs(y) > 6
    assert np.all(np.abs(C.e2m1_decode(codes))[sat] == 6.0)
    ins = ~sat
    assert np.all(np.abs(y - C.e2m1_decode(codes))[ins] <= _half_step(y)[ins] + 1e-12)


def test_nvfp4_dequant_f32_is_rounded_exact():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, (1000, 16)).astype(np.uint8)
    sc = rng.integers(1, 0x7F, 1000).astype(np.uint8)
    G = F32(0.0371)
    d32 = BF.nvfp4_dequant_f32(codes, sc, G)
    exact = BF.nvfp4_dequant_exact(codes, sc) * float(G)
    assert np.array_equal(d32, exact.astype(F32))
