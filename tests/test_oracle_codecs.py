"""Pins of oracle/codecs.py against the formats' definitions and independent routines."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = line.split()
        rows.append((a, b))
    return rows


def test_e2m1_grid_matches_printed_table():
    rows = _read_pairs("e2m1_grid.txt")
    codes = np.array([int(a) for a, _ in rows])
    vals = np.array([float(b) for _, b in rows])
    got = C.e2m1_decode(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))
    # the grid of the format: {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}
    assert sorted(set(np.abs(got).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute_e2m1(y):
    """Nearest grid magnitude by exhaustive distance, ties to the even code; sign from signbit."""
    y = np.asarray(y, np.float32)
    a = np.abs(y).astype(np.float64)
    mags = C.E2M1_MAGNITUDES
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates choose the even index (the tie partners are adjacent codes)
    ar = np.arange(8)[None, :]
    even = np.where(cand & (ar % 2 == 0), ar, 99).min(1)
    first = np.where(cand, ar, 99).min(1)
    ntied = cand.sum(1)
    code = np.where(ntied > 1, even, first)
    code = np.where(a > 6.0, 7, code)
    return (code | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_encode_exhaustive_core_range():
    """Every positive float32 in [2^-4, 2^4) plus its negative, against brute force."""
    lo = np.float32(2.0 ** -4).view(np.uint32)
    hi = np.float32(2.0 ** 4).view(np.uint32)
    step = 1 << 21
    for start in range(int(lo), int(hi), step):
        bits = np.arange(start, min(start + step, int(hi)), dtype=np.uint32)
        y = bits.view(np.float32)
        assert np.array_equal(C.e2m1_encode(y), _brute_e2m1(y))
        yn = -y[::97]
        assert np.array_equal(C.e2m1_encode(yn), _brute_e2m1(yn))


def test_e2m1_encode_edges():
    th = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    near = np.concatenate([th, np.nextafter(th, np.float32(0)), np.nextafter(th, np.float32(10))])
    extra = np.array([0.0, -0.0, 1e-30, -1e-30, 6.5, 7.0, 1e30, np.inf, -np.inf,
                      np.float32(2.0 ** -149)], np.float32)
    y = np.concatenate([near, -near, extra]).astype(np.float32)
    assert np.array_equal(C.e2m1_encode(y), _brute_e2m1(y))
    assert C.e2m1_encode(np.float32(-0.0)) == 8
    assert C.e2m1_encode(np.float32(100.0)) == 7


def test_pack_nibble_order():
    codes = np.array([1, 2, 3, 4, 0xF, 0], np.uint8)
    packed = C.pack_nibbles(codes)
    assert packed.tolist() == [0x21, 0x43, 0x0F]
    assert np.array_equal(C.unpack_nibbles(packed), codes)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = C.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_golden_points():
    for hx, v in _read_pairs("e4m3_points.txt"):
        got = float(C.e4m3_decode(np.array([int(hx, 16)]))[0])
        if v == "nan":
            assert np.isnan(got)
        else:
            assert got == float(v)


def _brute_e4m3(t):
    codes = np.arange(0, 0x7F)
    vals = C.e4m3_decode(codes)
    t = np.asarray(t, np.float32).astype(np.float64)
    dist = np.abs(t[:, None] - vals[None, :])
    best = dist.min(1, keepdims=True)
    cand = dist == best
    even = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 999).min(1)
    first = np.where(cand, codes[None, :], 999).min(1)
    code = np.where(cand.sum(1) > 1, even, first)
    return np.where(t >= 448.0, 0x7E, code).astype(np.uint8)


def test_e4m3_encode_sat_brute_force():
    rng = np.random.default_rng(0)
    vals = C.e4m3_decode(np.arange(0, 0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    rnd = np.exp2(rng.uniform(-14, 10, 200000)).astype(np.float32)
    t = np.concatenate([near, rnd, np.array([0, 2.0 ** -10, 447.9, 448, 460, 464, 470, 1e30, np.inf],
                                             np.float32)])
    t = t[t >= 0]
    assert np.array_equal(C.e4m3_encode_sat(t), _brute_e4m3(t))


def test_e4m3_encode_agrees_with_torch_in_range():
    rng = np.random.default_rng(1)
    t = np.exp2(rng.uniform(-12, np.log2(447.0), 100000)).astype(np.float32)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(C.e4m3_encode_sat(t), ref)


def test_e4m3_pow2_codes():
    for e in range(-9, 9):
        assert C.e4m3_decode(C.e4m3_code_of_pow2(np.array([e])))[0] == 2.0 ** e


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = C.e8m0_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_mx_shared_exp_closed_form():
    rng = np.random.default_rng(2)
    a = np.exp2(rng.uniform(-100, 100, 100000))
    e = C.mx_shared_exp(a)
    r = a / np.exp2(e.astype(np.float64))
    assert np.all((r >= 4.0) & (r < 8.0))
    assert C.mx_shared_exp(np.array([0.0]))[0] == -127
    assert C.mx_shared_exp(np.array([4.0]))[0] == 0
    assert C.mx_shared_exp(np.array([np.nextafter(4.0, 0)]))[0] == -1


def test_ceil_floor_log2():
    x = np.array([1.0, 2.0, 3.0, 0.75, 2.0 ** -30, 1000.0])
    assert C.floor_log2(x).tolist() == [0, 1, 1, -1, -30, 9]
    assert C.ceil_log2(x).tolist() == [0, 1, 2, 0, -30, 10]
