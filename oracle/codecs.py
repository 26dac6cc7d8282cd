"""Scalar codecs: E2M1 (FP4 element), E4M3 (NVFP4 block scale), E8M0 (MX scale).

Test infrastructure only (see ``oracle/__init__``).

The pages name the formats (NVFP4 and MXFP4 in [Abstract]; E4M3 scales in
[Blog/New]) but print no bit layouts, so the layouts follow the public specs
[OCP-MX] and [OCP-FP8].  Every function takes and returns numpy arrays and
works elementwise.

Pins (tests/test_oracle_codecs.py):
* e2m1_encode   -- brute-force nearest point of the printed grid
                   {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}, ties to the
                   even code, over every float32 in [2^-4, 2^4) and edge sets.
* e4m3_decode   -- torch.float8_e4m3fn decode of all 256 bytes.
* e4m3_encode_sat -- brute-force nearest of the 127 finite non-negative codes.
* e8m0_decode   -- torch.float8_e8m0fnu decode of all 256 bytes.
* mx_shared_exp -- closed form amax / 2^e in [4, 8) (the MX rule).
"""
import numpy as np

# Magnitudes of the 3-bit E2M1 field (exponent 2 bits, mantissa 1 bit, bias 1):
# code 0 -> 0, 1 -> 0.5 (subnormal), 2.. -> (1 + m/2) * 2^(e-1).  [OCP-MX]
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e2m1_decode(codes):
    """4-bit code (bit 3 = sign, bits 2..0 = magnitude index) -> float64.

    The sign bit of a zero magnitude gives -0.0.  [OCP-MX] E2M1.
    """
    c = np.asarray(codes).astype(np.uint8) & np.uint8(0xF)
    mag = E2M1_MAGNITUDES[(c & 7).astype(np.intp)]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_encode(y):
    """float32 -> 4-bit code, round to nearest, ties to the even code, saturating at 6.

    The magnitude index is the number of decision thresholds |y| has passed.
    A tie sits exactly on a threshold; it goes to the neighbour whose code is
    even, which is what the choice of ``>`` (tie goes down) or ``>=`` (tie
    goes up) at each threshold encodes:

        0.25 -> 0 (code 0)   0.75 -> 1.0 (code 2)   1.25 -> 1.0 (code 2)
        1.75 -> 2.0 (code 4) 2.5  -> 2.0 (code 4)   3.5  -> 4.0 (code 6)
        5.0  -> 4.0 (code 6)

    Values above 6 (and +-inf) saturate to +-6.  The sign is the float's sign
    bit, so -0.0 and small negatives that round to zero give code 8.
    NaN is a caller error (reading R12).  [OCP-MX] E2M1 conversion.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y)
    idx = ((a > 0.25).astype(np.uint8)
           + (a >= 0.75)
           + (a > 1.25)
           + (a >= 1.75)
           + (a > 2.5)
           + (a >= 3.5)
           + (a > 5.0))
    sign = np.signbit(y).astype(np.uint8) << 3
    return (idx.astype(np.uint8) | sign).astype(np.uint8)


def pack_nibbles(codes):
    """Pack 4-bit codes along the last axis: byte j = code[2j] | code[2j+1] << 4."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of :func:`pack_nibbles`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def e4m3_decode(codes):
    """E4M3 ("FN": no infinities, 0x7F/0xFF are NaN) byte -> float64.  [OCP-FP8]

    exponent field e = bits 6..3 (bias 7), mantissa m = bits 2..0:
    e == 0 -> m * 2^-9 (subnormal), else (1 + m/8) * 2^(e-7).  Max 448 (0x7E).
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(s == 1, -val, val)


def e4m3_encode_sat(t):
    """Non-negative float32 -> E4M3 byte, round to nearest (ties to even code), saturate at 448.

    Values at or above 448 give 0x7E (the largest finite code), so the NaN
    pattern is never produced.  Inputs at or below 2^-10 round to code 0.
    Negative inputs are a caller error.  [OCP-FP8] with saturation.
    """
    t = np.asarray(t, dtype=np.float32).astype(np.float64)
    assert not np.any(t < 0), "e4m3_encode_sat takes non-negative values"
    out = np.zeros(t.shape, dtype=np.int64)
    sat = t >= E4M3_MAX
    sub = t < 2.0 ** -6
    # subnormal range: multiples of 2^-9; integer 8 is exactly the first normal (code 0x08)
    q_sub = np.rint(np.where(sub, t, 0.0) * 2.0 ** 9).astype(np.int64)
    # normal range: t = q * 2^(e-3) with q in [8, 16)
    frac, k = np.frexp(np.where(sub | sat, 1.0, t))
    e = k - 1
    q = np.rint(np.ldexp(np.where(sub | sat, 1.0, t), -(e - 3))).astype(np.int64)
    carry = q == 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    code_norm = ((e + 7) << 3) | (q - 8)
    out = np.where(sub, q_sub, code_norm)
    out = np.where(sat, E4M3_MAX_CODE, out)
    out = np.minimum(out, E4M3_MAX_CODE)
    return out.astype(np.uint8)


def e4m3_code_of_pow2(e):
    """E4M3 byte of the power of two 2^e, for integer e in [-9, 8]."""
    e = np.asarray(e, dtype=np.int64)
    assert np.all((e >= -9) & (e <= 8))
    return np.where(e >= -6, (e + 7) << 3, 1 << (e + 9)).astype(np.uint8)


def e8m0_decode(codes):
    """E8M0 byte u -> 2^(u-127); 0xFF is NaN.  [OCP-MX]"""
    u = np.asarray(codes).astype(np.int64) & 0xFF
    val = np.exp2((u - 127).astype(np.float64))
    return np.where(u == 255, np.nan, val)


def floor_log2(x):
    """Exact floor(log2 x) of positive finite floats (via frexp)."""
    _, k = np.frexp(np.asarray(x, dtype=np.float64))
    return (k - 1).astype(np.int64)


def ceil_log2(x):
    """Exact ceil(log2 x) of positive finite floats (via frexp)."""
    m, k = np.frexp(np.asarray(x, dtype=np.float64))
    return np.where(m == 0.5, k - 1, k).astype(np.int64)


def mx_shared_exp(amax):
    """MX shared exponent of a block: floor(log2 amax) - 2, clamped to [-127, 127].

    2 is the largest exponent of an E2M1 element (6 = 1.5 * 2^2), so the
    block maximum lands in [4, 8) after scaling and elements above 6
    saturate, as the MX conversion rule prescribes.  amax == 0 gives -127.
    [OCP-MX] section on converting to MX formats.
    """
    a = np.asarray(amax, dtype=np.float64)
    safe = np.where(a > 0, a, 1.0)
    e = floor_log2(safe) - 2
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)
