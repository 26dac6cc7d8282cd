"""Dual-Residual Query Quantization.

Test infrastructure only (see ``oracle/__init__``).

The pages: a native FP4 product needs the query in FP4 as well, and one FP4
pass leaves a large logit error, so the query is split into two FP4 tensors
where the second encodes the residual the first leaves, and their sum
approximates the query ([Abstract]; [Blog/New]; [Explainer/Analyse];
[Editorial/Three]).  The pages report the query-logit error falling from 60 %
to 1 % on their models; that figure is context only here (different data).

Readings:
* R10  Q1 and Q2 use the cache's format.  NVFP4: 16-element blocks with
       power-of-two E4M3 block scales and an fp32 per-row tensor scale
       (reading R-P2 of ``blockfmt``), G = fl32(amax(row) / 1536) where
       1536 = 6 * 256 maps the row maximum onto the largest power-of-two E4M3
       scale.  MXFP4: the MX rule per 32 elements, no tensor scale.
* C6   y = FWHT(fl32(q * q_smooth)); Q1 = enc(y); R = fl32(y - deq32(Q1));
       Q2 = enc(R), where deq32 is fl32(fl32(dec * 2^e) * G) (NVFP4) or
       ldexp(dec, e) (MXFP4).
* MLA  The 512-d latent query goes through the same path over 512 channels;
       its 64-d rope part stays in bf16 and is not quantized.

Pins (tests/test_oracle_query.py): Q1 + Q2 reconstructs y within Q2's
half-step bound; the dual logit error is at most a tenth of the single-pass
error on random and outlier-heavy keys; with an exactly representable row
(Q1 exact) Q2 is all zero; the NVFP4 row maximum encodes as +-6.
"""
import numpy as np

from .codecs import e2m1_decode, mx_shared_exp
from .blockfmt import (NV_BLOCK, MX_BLOCK, blocks, amax_blocks, p2_block_exp, p2_encode,
                       mx_encode, mx_dequant_f32)
from .transforms import rotate_queries
from .kvquant import NVFP4

F32 = np.float32
Q_ROW_DIV = F32(1536.0)


class QuantQuery:
    """Per-row quantized query: codes [R, d], block exponents [R, d/B], validity, G [R]."""

    def __init__(self, fmt, y, c1, e1, v1, G1, c2, e2, v2, G2):
        self.fmt = fmt
        self.y = y
        self.c1, self.e1, self.v1, self.G1 = c1, e1, v1, G1
        self.c2, self.e2, self.v2, self.G2 = c2, e2, v2, G2

    def dequant_exact(self, which):
        """dec(code) * 2^e in float64 without G, shape [R, d]."""
        c, e, v = (self.c1, self.e1, self.v1) if which == 1 else (self.c2, self.e2, self.v2)
        B = NV_BLOCK if self.fmt == NVFP4 else MX_BLOCK
        R, d = c.shape
        val = e2m1_decode(c).reshape(R, d // B, B) * np.exp2(e.astype(np.float64))[..., None]
        val = np.where(v[..., None], val, 0.0)
        return val.reshape(R, d)

    def approx(self, which=(1, 2)):
        """Dequantized query including G (float64)."""
        out = 0.0
        if 1 in which:
            out = out + self.dequant_exact(1) * self.G1.astype(np.float64)[:, None]
        if 2 in which:
            out = out + self.dequant_exact(2) * self.G2.astype(np.float64)[:, None]
        return out


def _nv_pass(x):
    R, d = x.shape
    G = (np.max(np.abs(x), axis=-1) / Q_ROW_DIV).astype(F32)
    xb = blocks(x, NV_BLOCK)
    e, valid = p2_block_exp(amax_blocks(x, NV_BLOCK), G[:, None])
    codes, _ = p2_encode(xb, e, valid, G[:, None])
    deq = (e2m1_decode(codes).astype(F32) * np.exp2(e.astype(np.float64)).astype(F32)[..., None]).astype(F32)
    deq = (deq * G[:, None, None]).astype(F32)
    return codes.reshape(R, d), e, valid, G, deq.reshape(R, d)


def _mx_pass(x):
    R, d = x.shape
    xb = blocks(x, MX_BLOCK)
    e = mx_shared_exp(amax_blocks(x, MX_BLOCK))
    codes = mx_encode(xb, e)
    deq = mx_dequant_f32(codes, e)
    valid = np.ones(e.shape, dtype=bool)
    return codes.reshape(R, d), e, valid, np.ones(R, F32), deq.reshape(R, d).astype(F32)


def quantize_query(Q, q_smooth, fmt, dual=True, rotate=True):
    """Rows Q float32 [R, d] (one KV head's query heads, or MLA latent rows) -> QuantQuery."""
    Q = np.asarray(Q, F32)
    y = rotate_queries(Q, q_smooth, rotate)
    one = _nv_pass if fmt == NVFP4 else _mx_pass
    c1, e1, v1, G1, deq1 = one(y)
    if dual:
        Rres = (y - deq1).astype(F32)
        c2, e2, v2, G2, _ = one(Rres)
    else:
        c2 = np.zeros_like(c1)
        e2 = np.zeros_like(e1)
        v2 = np.zeros_like(v1)
        G2 = np.zeros_like(G1)
    return QuantQuery(fmt, y, c1, e1, v1, G1, c2, e2, v2, G2)
