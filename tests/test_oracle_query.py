"""Pins of oracle/query.py: residual bound, dual vs single logit error, exact rows."""
import numpy as np

from oracle import codecs as C
from oracle import kvquant as KQ
from oracle.query import quantize_query
from oracle.attention import key_dequant_exact

F32 = np.float32


def _keys(rng, L, d, outl=True):
    K = rng.standard_normal((L, d)).astype(F32)
    if outl:
        K[:, [3, 17, 64, 100]] *= 12
    return K


def test_residual_is_within_q2_half_step():
    rng = np.random.default_rng(20)
    for fmt in (KQ.NVFP4, KQ.MXFP4):
        Q = (rng.standard_normal((64, 128)) * np.exp(rng.normal(0, 1, (64, 1)))).astype(F32)
        qq = quantize_query(Q, np.ones(128, F32), fmt)
        approx = qq.approx()
        y = qq.y.astype(np.float64)
        B = 16 if fmt == KQ.NVFP4 else 32
        step = np.exp2(qq.e2.astype(np.float64)) * qq.G2[:, None].astype(np.float64)   # [R, nblk]
        err = np.abs(approx - y).reshape(64, -1, B)
        # |R - Q2| <= half the top grid gap (1.0 in code units) plus the fp32 rounding of y - Q1;
        # the MX floor rule may also clip values in (6, 8) to 6, so its bound is 2 code units
        units = 1.0 if fmt == KQ.NVFP4 else 2.0
        bound = step[..., None] * units + np.abs(y).reshape(64, -1, B) * 2.0 ** -22
        assert np.all(err <= bound)


def test_dual_cuts_logit_error_tenfold():
    rng = np.random.default_rng(21)
    d, L = 128, 512
    for fmt in (KQ.NVFP4, KQ.MXFP4):
        K = _keys(rng, L, d)
        ksi = np.ones(d, F32)
        kc, ks = KQ.quantize_keys(K, ksi, F32(0.05), fmt)
        khat = key_dequant_exact(kc, ks, fmt)
        Q = rng.standard_normal((32, d)).astype(F32)
        qd = quantize_query(Q, ksi, fmt, dual=True)
        qs = quantize_query(Q, ksi, fmt, dual=False)
        exact = qd.y.astype(np.float64) @ khat.T
        e_dual = np.linalg.norm(qd.approx() @ khat.T - exact) / np.linalg.norm(exact)
        e_single = np.linalg.norm(qs.approx() @ khat.T - exact) / np.linalg.norm(exact)
        # NVFP4 (per-row G, ceil rule) gains >10x; the MX floor rule drops the residual's
        # exponent by only ~2 octaves, so MXFP4 gains >5x
        limit = 0.1 if fmt == KQ.NVFP4 else 0.2
        assert e_dual <= limit * e_single, (fmt, e_dual, e_single)


def test_exactly_representable_row_has_zero_residual():
    # a row whose rotated values sit on the FP4 grid of one power-of-two scale
    d = 128
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 16, d).astype(np.uint8)
    codes[0] = 7                                           # make +6 the row maximum
    y = C.e2m1_decode(codes).astype(F32)
    # rotate^-1 so that the oracle's rotation lands exactly on y (H H = d I)
    from oracle.transforms import fwht_f32
    q = (fwht_f32(y[None]) / F32(d)).astype(F32)
    qq = quantize_query(q, np.ones(d, F32), KQ.NVFP4)
    assert np.array_equal(qq.y[0], y)
    assert np.all((qq.c2 & 7) == 0) or qq.G2[0] == 0


def test_nvfp4_row_max_encodes_as_six():
    rng = np.random.default_rng(23)
    Q = rng.standard_normal((50, 128)).astype(F32)
    qq = quantize_query(Q, np.ones(128, F32), KQ.NVFP4)
    i = np.argmax(np.abs(qq.y), axis=1)
    top = qq.c1[np.arange(50), i] & 7
    assert np.all(top == 7)
