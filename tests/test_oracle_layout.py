"""Pins of oracle/layout.py: byte positions from the layout definition, and round trips."""
import numpy as np

from oracle import layout as LY
from oracle import kvquant as KQ


def _cache(num_pages, hkv, P, d, B):
    return dict(k_codes=np.zeros((num_pages, hkv, P, d // 2), np.uint8),
                k_scales=np.zeros((num_pages, hkv, P * d // B), np.uint8),
                v_codes=np.zeros((num_pages, hkv, d, P // 2), np.uint8),
                v_scales=np.zeros((num_pages, hkv, d * P // B), np.uint8))


def test_gqa_byte_positions_and_round_trip():
    rng = np.random.default_rng(40)
    P, d, hkv, B = 32, 128, 2, 16
    L = 75
    bt = np.array([5, 2, 7], np.int32)
    kc = rng.integers(0, 16, (L, d)).astype(np.uint8)
    ks = rng.integers(0, 127, (L, d // B)).astype(np.uint8)
    nblk = -(-L // B)
    vc = rng.integers(0, 16, (nblk * B, d)).astype(np.uint8)
    vc[L:] = 0
    vs = rng.integers(0, 127, (d, nblk)).astype(np.uint8)
    cache = _cache(8, hkv, P, d, B)
    LY.scatter_gqa(cache, 1, bt, L, kc, ks, vc, vs, KQ.NVFP4)
    # token 40 -> logical page 1 -> physical page 2, slot 8; channels 6, 7 share byte 3
    assert cache["k_codes"][2, 1, 8, 3] == (kc[40, 6] | (kc[40, 7] << 4))
    assert cache["k_scales"][2, 1, 8 * 8 + 2] == ks[40, 2]
    # value of token 70 (page 7, slot 6) channel 9: byte 3 of channel 9's row, low nibble
    assert cache["v_codes"][7, 1, 9, 3] & 0xF == vc[70, 9]
    # its value block 4 is page 7's block 0; channel 9 -> (0 * 16 + 9) * 8 * 2 + 0 * 2 + 0
    assert cache["v_scales"][7, 1, 144] == vs[9, 4]
    g = LY.gather_gqa(cache, 1, bt, L, KQ.NVFP4)
    for a, b in zip(g, (kc, ks, vc, vs)):
        assert np.array_equal(a, b)
    assert not cache["k_codes"][:, 0].any()


def test_gqa_mxfp4_scale_positions_and_round_trip():
    """MXFP4, page 64: the key scales one decode lane reads (tokens t, t+4, ..., t+28 of a
    32-token span, one channel block) are 8 consecutive bytes; value scales of channels
    c, c+16, ..., c+112 over one span likewise."""
    rng = np.random.default_rng(42)
    P, d, hkv, B = 64, 128, 1, 32
    L = 150
    bt = np.array([1, 3, 0], np.int32)
    kc = rng.integers(0, 16, (L, d)).astype(np.uint8)
    ks = rng.integers(0, 255, (L, d // B)).astype(np.uint8)
    nblk = -(-L // B)
    vc = rng.integers(0, 16, (nblk * B, d)).astype(np.uint8)
    vc[L:] = 0
    vs = rng.integers(0, 255, (d, nblk)).astype(np.uint8)
    cache = _cache(4, hkv, P, d, B)
    LY.scatter_gqa(cache, 0, bt, L, kc, ks, vc, vs, KQ.MXFP4)
    # token 64 + 37 = 101 -> page 3, t = 37: span 1, row 1, step 1; block 3
    assert cache["k_scales"][3, 0, ((1 * 4 + 1) * 4 + 3) * 8 + 1] == ks[101, 3]
    run = cache["k_scales"][3, 0, ((1 * 4 + 1) * 4 + 3) * 8:][:8]
    assert np.array_equal(run, ks[64 + 33:64 + 64:4, 3])
    # value block 3 (tokens 96..127) = page 3's block 1; channel 100 = 16 * 6 + 4
    assert cache["v_scales"][3, 0, (1 * 16 + 4) * 8 + 6] == vs[100, 3]
    assert np.array_equal(cache["v_scales"][3, 0, (1 * 16 + 4) * 8:][:8], vs[4::16, 3])
    g = LY.gather_gqa(cache, 0, bt, L, KQ.MXFP4)
    for a, b in zip(g, (kc, ks, vc, vs)):
        assert np.array_equal(a, b)


def test_mla_round_trip():
    rng = np.random.default_rng(41)
    P, D, r, B = 64, 512, 64, 16
    L = 100
    bt = np.array([3, 0], np.int32)
    nblk = -(-L // B)
    lc = rng.integers(0, 16, (nblk * B, D)).astype(np.uint8)
    ls = rng.integers(0, 127, (nblk, D // B)).astype(np.uint8)
    kr = rng.integers(0, 65535, (L, r)).astype(np.uint16)
    cache = dict(k_codes=np.zeros((4, 1, P, D // 2), np.uint8),
                 k_scales=np.zeros((4, 1, P // B, D // B), np.uint8),
                 k_rope=np.zeros((4, 1, P, r), np.uint16))
    LY.scatter_mla(cache, bt, L, lc, ls, kr, KQ.NVFP4)
    assert cache["k_scales"][0, 0, 1, 7] == ls[5, 7]          # token block 5 = page 1, block 1
    # token 70 = page 0 (physical), slot 6; channel 300: byte 150 of the token row, low nibble
    assert cache["k_codes"][0, 0, 6, 150] & 0xF == lc[70, 300]
    assert cache["k_codes"][0, 0, 6, 150] >> 4 == lc[70, 301]
    g = LY.gather_mla(cache, bt, L, KQ.NVFP4)
    for a, b in zip(g, (lc, ls, kr)):
        assert np.array_equal(a, b)
