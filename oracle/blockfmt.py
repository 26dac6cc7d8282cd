"""Block encoders: NVFP4 (16-element blocks, E4M3 scale, fp32 tensor scale G) and
MXFP4 (32-element blocks, E8M0 scale), plus the power-of-two NVFP4 encoder
used for the query and probability operands.

Test infrastructure only (see ``oracle/__init__``).

Arithmetic convention: ``fl32`` means one IEEE binary32 operation rounded to
nearest-even; numpy float32 arrays give exactly that, and no step here is
fused.  Block dimension is always the last axis.

Formats: [NVFP4] and [OCP-MX]; the pages name NVFP4/MXFP4 as the cache
formats ([Abstract]) and E4M3 as the scale type whose underflow the method
guards against ([Blog/New]).

Readings (where the pages are silent):
* R-NV1  NVFP4 encode with scale code c: S = E4M3(c), r = fl32(1 / fl32(S*G))
         (r = 0 when S*G == 0), code_i = E2M1(fl32(x_i * r)); the default
         scale is c0 = E4M3_sat(fl32(amax / fl32(6*G))).
* R-P2   Query and probability blocks are NVFP4 with the E4M3 block scale
         restricted to powers of two (mantissa field zero, a valid E4M3 value)
         and the mantissa freedom carried by the fp32 tensor scale G:
         e = clamp(ceil(log2 t), -9, 8), t = fl32(amax * fl32(1 / fl32(6*G))).
         The ceiling keeps every element within +-6 (no clipping).  A power of
         two scale is what the E8M0-scaled FP4 matrix cores accept exactly.
* R-MX   MXFP4 uses the MX rule e = floor(log2 amax) - 2 (elements above 6
         saturate), codes E2M1(x * 2^-e) -- exact scaling.

Pins (tests/test_oracle_blockfmt.py): reconstruction bound |x - xhat| <= half
an E2M1 step * scale unless clipped; default-scale maps the block maximum to
code magnitude 6 (or saturates); ceil rule keeps the maximum in (3, 6];
MX rule keeps amax / 2^e in [4, 8); brute force over every scale code on tiny
blocks for the search objective (in test_oracle_kvquant.py).
"""
import numpy as np

from .codecs import (e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode_sat,
                     e4m3_code_of_pow2, ceil_log2, mx_shared_exp)

F32 = np.float32
NV_BLOCK = 16
MX_BLOCK = 32
P2_EMIN = -9     # smallest power of two an E4M3 code holds (subnormal 0x01)
P2_EMAX = 8      # largest power of two below the E4M3 maximum 448


def _f32(x):
    return np.asarray(x, dtype=F32)


def _recip_or_zero(v):
    v = _f32(v)
    out = np.zeros(v.shape, dtype=F32)
    np.divide(F32(1.0), v, out=out, where=(v != 0))
    return out


# ---------------------------------------------------------------- NVFP4 (E4M3 scales)

def nvfp4_default_scale(amax, G):
    """c0 = E4M3_sat(fl32(amax / fl32(6*G))); 0 when G == 0.  Reading R-NV1."""
    amax = _f32(amax)
    G = _f32(G)
    sixg = _f32(F32(6.0) * G)
    t = np.zeros(np.broadcast(amax, sixg).shape, dtype=F32)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        np.divide(amax, sixg, out=t, where=(sixg != 0))
    c = e4m3_encode_sat(np.where(np.isfinite(t), t, F32(np.inf)))
    return np.where(np.broadcast_to(G, t.shape) == 0, 0, c).astype(np.uint8)


def nvfp4_encode(x, scale_code, G):
    """E2M1 codes of blocks x[..., n] under scale codes [...] and tensor scale G.  R-NV1."""
    x = _f32(x)
    S = e4m3_decode(scale_code).astype(F32)
    sg = _f32(S * _f32(G))
    r = _recip_or_zero(sg)
    y = _f32(x * r[..., None])
    return e2m1_encode(y)


def nvfp4_dequant_f32(codes, scale_code, G):
    """fl32(fl32(dec(code) * S) * G); the first product is exact (<= 6 significant bits)."""
    d = e2m1_decode(codes).astype(F32)
    S = e4m3_decode(scale_code).astype(F32)
    ds = _f32(d * S[..., None])
    Gb = _f32(G)
    if Gb.ndim:
        Gb = Gb[..., None]
    return _f32(ds * Gb)


def nvfp4_dequant_exact(codes, scale_code):
    """dec(code) * S in float64, without the tensor scale (exact)."""
    return e2m1_decode(codes) * e4m3_decode(scale_code)[..., None]


# ---------------------------------------------------------------- NVFP4, power-of-two block scales

def p2_block_exp(amax, G):
    """Power-of-two block exponent of reading R-P2.

    Returns (e, valid): e = clamp(ceil(log2 t), -9, 8) with
    t = fl32(amax * fl32(1/fl32(6*G))); valid is False where amax == 0 or
    G == 0 (the block is stored with scale code 0 and all-zero codes).
    t == 0 (underflow) gives -9, t == inf gives 8.
    """
    amax = _f32(amax)
    G = _f32(G)
    inv6g = _recip_or_zero(_f32(F32(6.0) * G))
    with np.errstate(over="ignore"):
        t = _f32(amax * inv6g)
    valid = (amax > 0) & (np.broadcast_to(G, amax.shape) > 0)
    tc = np.minimum(t.astype(np.float64), 2.0 ** 9)
    e = np.where(tc > 0, ceil_log2(np.where(tc > 0, tc, 1.0)), P2_EMIN)
    e = np.clip(e, P2_EMIN, P2_EMAX)
    return e.astype(np.int64), valid


def p2_encode(x, e, valid, G):
    """Codes of blocks x[..., n] with power-of-two block scales 2^e and tensor scale G.

    r = fl32(1 / fl32(2^e * G)) (0 for invalid blocks), code = E2M1(fl32(x * r)).
    Returns (codes, scale_codes) with the scale code 0 for invalid blocks.
    """
    x = _f32(x)
    S = np.exp2(e.astype(np.float64)).astype(F32)
    sg = _f32(S * _f32(G))
    r = np.where(valid, _recip_or_zero(sg), F32(0.0)).astype(F32)
    codes = e2m1_encode(_f32(x * r[..., None]))
    sc = np.where(valid, e4m3_code_of_pow2(e), 0).astype(np.uint8)
    return codes, sc


def p2_dequant_exact(codes, e, valid):
    """dec(code) * 2^e in float64 (without G); zero for invalid blocks."""
    v = e2m1_decode(codes) * np.exp2(e.astype(np.float64))[..., None]
    return np.where(valid[..., None], v, 0.0)


# ---------------------------------------------------------------- MXFP4 (E8M0 scales)

def mx_encode(x, e):
    """E2M1 codes of blocks x[..., n] scaled by 2^-e (exact scaling).  Reading R-MX."""
    x = _f32(x)
    y = np.ldexp(x, -np.asarray(e, dtype=np.int64)[..., None]).astype(F32)
    return e2m1_encode(y)


def mx_dequant_f32(codes, e):
    """ldexp(dec(code), e) as float32 (exact for e in [-127, 125])."""
    d = e2m1_decode(codes).astype(F32)
    return np.ldexp(d, np.asarray(e, dtype=np.int64)[..., None]).astype(F32)


def mx_dequant_exact(codes, e):
    return e2m1_decode(codes) * np.exp2(np.asarray(e, dtype=np.float64))[..., None]


def mx_scale_code(e):
    """E8M0 byte of 2^e."""
    return (np.asarray(e, dtype=np.int64) + 127).astype(np.uint8)


def blocks(x, n):
    """View the last axis of x as (..., last/n, n)."""
    x = np.asarray(x)
    assert x.shape[-1] % n == 0
    return x.reshape(x.shape[:-1] + (x.shape[-1] // n, n))


def amax_blocks(x, n):
    return np.max(np.abs(blocks(x, n)), axis=-1)
