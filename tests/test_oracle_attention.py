"""Pins of oracle/attention.py: textbook special case, split invariance, per-token loops,
underflow closed form, and the logit formula."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import codecs as C
from oracle import kvquant as KQ
from oracle.query import quantize_query

F32 = np.float32


def _rand_case(rng, L, d=128, fmt=KQ.NVFP4, g=4):
    K = rng.standard_normal((L, d)).astype(F32)
    V = rng.standard_normal((L, d)).astype(F32)
    Q = rng.standard_normal((g, d)).astype(F32)
    return Q, K, V


def test_identity_codec_is_textbook_softmax():
    rng = np.random.default_rng(30)
    for L in (1, 100, 128, 1000):
        s = (rng.standard_normal((3, L)) * 3).astype(F32)
        v = rng.standard_normal((L, 64))
        got = A.attend(s, v, L, KQ.NVFP4, p_mode="exact")["out"]
        z = s.astype(np.float64) * math.log(2.0)
        p = np.exp(z - z.max(-1, keepdims=True))
        ref = (p / p.sum(-1, keepdims=True)) @ v
        # p~ is rounded to fp32 (as in the kernel): relative error per weight <= 2^-24
        assert np.all(A.row_rel_err(got, ref) < 1e-6)


def _online_split(o_t, m_t, l_t, bounds):
    """Running-max accumulation of tiles inside each split, then the split merge."""
    R, T, d = o_t.shape
    os_, ms, ls = [], [], []
    for a, b in bounds:
        m = np.full(R, -np.inf)
        o = np.zeros((R, d))
        l = np.zeros(R)
        for t in range(a, b):
            mn = np.maximum(m, m_t[:, t])
            al = np.where(np.isfinite(m), np.exp2(m - mn), 0.0)
            be = np.exp2(m_t[:, t] - mn)
            o = o * al[:, None] + o_t[:, t] * be[:, None]
            l = l * al + l_t[:, t] * be
            m = mn
        os_.append(o)
        ms.append(m)
        ls.append(l)
    return A.merge_partials(np.stack(os_, 1), np.stack(ms, 1), np.stack(ls, 1))


def test_split_merge_invariance():
    rng = np.random.default_rng(31)
    L = 1500
    s = (rng.standard_normal((4, L)) * 4).astype(F32)
    v = rng.standard_normal((L, 32))
    res = A.attend(s, v, L, KQ.NVFP4, partials=True)
    T = res["m_tiles"].shape[1]
    for bounds in ([(0, T)], [(0, 3), (3, 7), (7, T)], [(i, i + 1) for i in range(T)],
                   [(0, 5), (5, 5), (5, T)]):
        got = _online_split(res["o_tiles"], res["m_tiles"].astype(np.float64), res["l_tiles"], bounds)
        assert np.allclose(got, res["out"], rtol=1e-12, atol=1e-14)


def _loop_reference(s, vhat, L, fmt):
    """Per-token, per-block loops written from the definitions (no vectorised helpers)."""
    R = s.shape[0]
    d = vhat.shape[1]
    B = 16 if fmt == KQ.NVFP4 else 32
    out = np.zeros((R, d))
    for r in range(R):
        ms, os_, ls = [], [], []
        for t0 in range(0, L, 128):
            toks = range(t0, min(L, t0 + 128))
            m = max(F32(s[r, t]) for t in toks)
            p = {t: F32(2.0 ** float(F32(F32(s[r, t]) - m))) for t in toks}
            o = np.zeros(d)
            l = 0.0
            for b0 in range(t0, min(L, t0 + 128), B):
                bt = [t for t in range(b0, b0 + B) if t < L]
                amax = max(p[t] for t in bt)
                if fmt == KQ.NVFP4:
                    tq = F32(amax * F32(F32(1.0) / F32(F32(6.0) * F32(2.0 ** -10))))
                    e = int(math.ceil(math.log2(float(tq)))) if tq > 0 else -9
                    if tq > 0 and 2.0 ** (e - 1) >= float(tq):     # guard log2 rounding
                        e -= 1
                    e = min(8, max(-9, e))
                    r_ = F32(F32(1.0) / F32(F32(2.0 ** e) * F32(2.0 ** -10)))
                    scale = 2.0 ** (e - 10)
                else:
                    e = max(-127, math.frexp(float(amax))[1] - 1 - 2) if amax > 0 else -127
                    r_ = F32(2.0 ** -e)
                    scale = 2.0 ** e
                for t in bt:
                    code = C.e2m1_encode(np.array([F32(p[t] * r_)], F32))[0]
                    ph = float(C.e2m1_decode(np.array([code]))[0]) * scale
                    o += ph * vhat[t]
                for t in bt:
                    l += float(p[t])
            ms.append(float(m))
            os_.append(o)
            ls.append(l)
        M = max(ms)
        w = [2.0 ** (x - M) for x in ms]
        out[r] = sum(wi * oi for wi, oi in zip(w, os_)) / sum(wi * li for wi, li in zip(w, ls))
    return out


@pytest.mark.parametrize("fmt", [KQ.NVFP4, KQ.MXFP4])
def test_tiny_contexts_match_explicit_loops(fmt):
    rng = np.random.default_rng(32)
    for L in (1, 2, 15, 16, 17, 127, 128, 129, 300):
        s = (rng.standard_normal((2, L)) * 3).astype(F32)
        v = rng.standard_normal((L, 16))
        got = A.attend(s, v, L, fmt)["out"]
        ref = _loop_reference(s, v, L, fmt)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-13), L


def test_underflow_closed_form():
    """Flat logits at long context: tile-relative P keeps every block, vanilla P loses all.

    Closed form: vanilla p ~ 1/L, its E4M3 scale amax/6 <= 2^-10 once L > 6*2^10/e^{max gap}.
    The tile-relative p~ >= 2^(-gap) with gap << 19, so no block falls to zero.
    """
    rng = np.random.default_rng(33)
    L, d = 16384, 128
    Q = rng.standard_normal((4, d)).astype(F32)
    K = (rng.standard_normal((L, d)) * 0.05).astype(F32)
    V = rng.standard_normal((L, d)).astype(F32)
    ones = np.ones(d, F32)
    args = (Q, K, V, ones, ones, F32(0.05 * 8 * math.sqrt(d) / 2688), F32(8 / 2688), KQ.NVFP4,
            1 / math.sqrt(d))
    tile = A.gqa_head(*args)
    van = A.gqa_head(*args, opts=dict(p_mode="vanilla"))
    nblk = 4 * (L // 16)
    assert tile["zero_blocks"] == 0
    assert van["zero_blocks"] == nblk
    smax = np.max(np.abs(tile["s"]))
    assert smax < 2.0                       # the logits are indeed nearly flat (base 2)


def test_logit_formula_closed_form():
    rng = np.random.default_rng(34)
    L, d = 50, 128
    Q, K, V = _rand_case(rng, L)
    ones = np.ones(d, F32)
    G_K = F32(0.02)
    kc, ks = KQ.quantize_keys(K, ones, G_K, KQ.NVFP4)
    qq = quantize_query(Q, ones, KQ.NVFP4)
    cs = A.logit_coeff(0.125, d)
    s = A.logits(qq, A.key_dequant_exact(kc, ks, KQ.NVFP4), G_K, cs, KQ.NVFP4)
    q_full = qq.approx()                                       # (Q1 + Q2) with G, float64
    k_full = A.key_dequant_exact(kc, ks, KQ.NVFP4) * float(G_K)
    ref = (q_full @ k_full.T) * 0.125 * math.log2(math.e) / d
    assert np.allclose(s, ref, rtol=3e-6, atol=1e-6 * np.abs(ref).max())


def test_mla_exact_codecs_is_textbook_attention():
    """MLA emulation with every codec exact (grid-valued latent with power-of-two tile
    scales, grid-valued query blocks, unquantized P; rotation and smoothing off) equals
    textbook softmax attention with the latent as key and value plus the rope term, for a
    context that is not a multiple of the 16-token tile."""
    rng = np.random.default_rng(7)
    D, r, L, R = 512, 64, 37, 3
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def grid_blocks(shape, exps):
        v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v[..., 0] = 6.0                                     # every block holds its maximum
        return v * exps

    # latent: 16 x 16 tiles, tile (token block, channel block) scaled by 2^e
    tile_e = rng.integers(-3, 3, size=(-(-L // 16), D // 16)).astype(np.float64)
    K = np.zeros((L, D))
    for tb in range(tile_e.shape[0]):
        for cb in range(D // 16):
            rows = slice(16 * tb, min(L, 16 * tb + 16))
            n = rows.stop - rows.start
            blk = grid_blocks((n, 16), 2.0 ** tile_e[tb, cb])
            blk[1:, 0] = blk[1:, 0] * rng.choice([-1.0, 1.0], size=n - 1)
            K[rows, 16 * cb:16 * cb + 16] = blk
    # query rows: 16-channel blocks scaled by 2^-j, j in 0..3; each row holds +-6 in block 0
    q = np.zeros((R, D))
    for i in range(R):
        for cb in range(D // 16):
            q[i, 16 * cb:16 * cb + 16] = grid_blocks(16, 2.0 ** (-int(rng.integers(0, 4)) if cb else 0))
    qr = W_bf16(rng.standard_normal((R, r)))
    kr = W_bf16(rng.standard_normal((L, r)))
    sc = 1.0 / np.sqrt(D + r)
    ones = np.ones(D, np.float32)
    res = A.mla_seq(q.astype(np.float32), qr, K.astype(np.float32), kr, ones, ones, 1.0, KQ.NVFP4, sc, L=L,
                    opts=dict(rotate=False, smooth=False, p_mode="exact"))
    ref = A.reference_attention(q, K, K, sc, q_rope=qr, k_rope=kr)
    assert np.max(A.row_rel_err(res["out"], ref)) < 1e-5
    # the latent codes reproduce K exactly (no search improvement possible over zero error)
    assert np.array_equal(A.latent_dequant_exact(res["l_codes"], res["l_scales"], KQ.NVFP4, 1.0)[:L], K)


def W_bf16(x):
    from fp4_kv_cache_amd.workloads import bf16_round
    return bf16_round(np.asarray(x, np.float32))


def test_multi_token_exact_codecs_is_causal_attention():
    """Multi-token decode with every codec exact (MXFP4 grid-valued keys, values and query
    blocks, unquantized P; rotation and smoothing off) equals textbook causal attention:
    query j of n sees tokens 0 .. L - n + j.  L = 130 with n = 4 leaves the second 128-token
    tile empty for the first two queries (such a tile must contribute nothing)."""
    rng = np.random.default_rng(11)
    d, L, n, g = 128, 130, 4, 2
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def grid_vals(shape):
        return rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)

    # keys: each token's 32-channel blocks hold a +-6 and are scaled by 2^e
    K = grid_vals((L, d))
    K[:, ::32] = 6.0 * rng.choice([-1.0, 1.0], size=(L, d // 32))
    K = K * np.repeat(2.0 ** rng.integers(-2, 3, size=(L, d // 32)), 32, axis=1)
    # values: each channel's 32-token blocks hold a +-6 (tail block: within the tokens present)
    V = grid_vals((L, d))
    for t0 in range(0, L, 32):
        V[t0, :] = 6.0 * rng.choice([-1.0, 1.0], size=d)
        V[t0:t0 + 32] *= 2.0 ** rng.integers(-2, 3, size=(1, d))
    q = grid_vals((n, g, d))
    q[..., ::32] = 6.0
    q = q * np.repeat(2.0 ** rng.integers(-2, 1, size=(n, g, d // 32)), 32, axis=-1)
    sc = 1.0 / np.sqrt(d)
    ones = np.ones(d, np.float32)
    res = A.gqa_head_multi(q.astype(np.float32), K.astype(np.float32), V.astype(np.float32), ones, ones,
                           1.0, 1.0, KQ.MXFP4, sc, L=L, opts=dict(rotate=False, smooth=False, p_mode="exact"))
    for j in range(n):
        Lj = L - n + 1 + j
        ref = A.reference_attention(q[j], K[:Lj], V[:Lj], sc)
        assert np.max(A.row_rel_err(res["out"][j], ref)) < 1e-6, j


def test_multi_token_single_query_is_gqa_head():
    """n = 1 is the ordinary decode: same rows, same output bit for bit."""
    rng = np.random.default_rng(12)
    L, d, g = 300, 128, 4
    Q, K, V = _rand_case(rng, L)
    q = rng.standard_normal((1, g, d)).astype(np.float32)
    ones = np.ones(d, np.float32)
    a = A.gqa_head(q[0], K, V, ones, ones, np.float32(0.01), np.float32(0.01), KQ.NVFP4, 0.08, L=L)
    b = A.gqa_head_multi(q, K, V, ones, ones, np.float32(0.01), np.float32(0.01), KQ.NVFP4, 0.08, L=L)
    assert np.array_equal(a["out"], b["out"][0])


def _nearest_f32(x):
    """The fp32 values nearest to the exact rational x (one, or two on a tie)."""
    from fractions import Fraction
    c = np.float32(float(x))
    best = []
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        best.append((abs(Fraction(float(cand)) - x), cand))
    dmin = min(d for d, _ in best)
    return [v for d, v in best if d == dmin]


@pytest.mark.parametrize("fmt", [KQ.NVFP4, KQ.MXFP4])
def test_raw_dot_is_exact_dot_rounded_once(fmt):
    """raw = fl32(<q^, k^>): the exact rational dot of the block-scaled values (brute force
    with fractions) rounded once to the nearest fp32, for random codes and scales whose
    products span the whole E4M3 / power-of-two range (R11)."""
    from fractions import Fraction
    rng = np.random.default_rng(35)
    d, R, L = 128, 3, 6
    Q = (rng.standard_normal((R, d)) * np.exp2(rng.integers(-6, 6, size=(R, d)))).astype(F32)
    K = (rng.standard_normal((L, d)) * np.exp2(rng.integers(-6, 6, size=(L, d)))).astype(F32)
    ones = np.ones(d, F32)
    kc, ks = KQ.quantize_keys(K, ones, F32(0.01) if fmt == KQ.NVFP4 else 1.0, fmt)
    khat = A.key_dequant_exact(kc, ks, fmt)
    qq = quantize_query(Q, ones, fmt)
    for which in (1, 2):
        qhat = qq.dequant_exact(which)
        raw = A.raw_dot(qhat, khat)
        for r in range(R):
            for t in range(L):
                exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qhat[r], khat[t])),
                            Fraction(0))
                assert raw[r, t] in _nearest_f32(exact), (which, r, t)


def _hadamard_preimage(x, factors):
    """z with FWHT(fl32(z * factors)) == x exactly: z = (x H / n) / factors, for x on a
    grid fine enough that every Walsh-Hadamard stage stays exact in fp32."""
    import scipy.linalg
    n = x.shape[-1]
    return ((np.asarray(x, np.float64) @ scipy.linalg.hadamard(n) / n) / factors).astype(F32)


def test_mla_rotated_smoothed_exact_codecs_is_textbook_attention():
    """The MLA pipeline with smoothing and rotation ON and exact codecs equals textbook
    attention over the original latent (as key and value) plus the rope term.

    The inputs are chosen so that the transformed latent x = FWHT(K * k_smooth_inv) and the
    transformed query y = FWHT(q * q_smooth) are grid-valued with power-of-two scales (every
    codec exact, Q2 = 0).  Logit invariance <yH, xH>/512 = <q, k> and the output un-rotation
    o = (o'' H / 512) * q_smooth must then give softmax(q K^T + q_r k_r^T) K.  Taking
    k_smooth_inv for q_smooth in the un-rotation, dropping the / 512, or a wrong smoothing
    direction each moves the output by a large factor."""
    rng = np.random.default_rng(36)
    D, r, L, R = 512, 64, 45, 3
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    # smoothing: powers of two, q_smooth * k_smooth_inv == 1
    lam = np.exp2(rng.integers(-2, 3, size=D)).astype(F32)
    ksi, qs = (1.0 / lam).astype(F32), lam
    # transformed latent: 16 x 16 tiles of grid values, each tile holding a +-6, scaled 2^e
    x = rng.choice(grid, size=(L, D)) * rng.choice([-1.0, 1.0], size=(L, D))
    tile_e = rng.integers(-3, 3, size=(-(-L // 16), D // 16))
    for tb in range(tile_e.shape[0]):
        for cb in range(D // 16):
            x[16 * tb, 16 * cb] = 6.0
            x[16 * tb:16 * tb + 16, 16 * cb:16 * cb + 16] *= 2.0 ** tile_e[tb, cb]
    # transformed query rows: 16-channel blocks scaled by 2^-j, a +-6 in block 0 (so Q1 is exact)
    y = rng.choice(grid, size=(R, D)) * rng.choice([-1.0, 1.0], size=(R, D))
    y[:, ::16] = 6.0
    ex = rng.integers(0, 4, size=(R, D // 16))
    ex[:, 0] = 0
    y = y * np.repeat(2.0 ** -ex, 16, axis=1)
    K = _hadamard_preimage(x, ksi)
    q = _hadamard_preimage(y, qs)
    qr = W_bf16(rng.standard_normal((R, r)))
    kr = W_bf16(rng.standard_normal((L, r)))
    sc = 1.0 / np.sqrt(D + r)
    res = A.mla_seq(q, qr, K, kr, ksi, qs, 1.0, KQ.NVFP4, sc, L=L, opts=dict(p_mode="exact"))
    # the transforms really were exact: codes reproduce x, the query residual is zero
    assert np.array_equal(A.latent_dequant_exact(res["l_codes"], res["l_scales"], KQ.NVFP4, 1.0)[:L], x)
    assert np.all(res["qq"].c2 & 7 == 0)
    ref = A.reference_attention(q, K, K, sc, q_rope=qr, k_rope=kr)
    assert np.max(A.row_rel_err(res["out"], ref)) < 1e-5
    # the same pin fails for the plausible mistakes it is meant to catch
    wrong_smooth = res["out"] / qs.astype(np.float64) * ksi.astype(np.float64)
    assert np.max(A.row_rel_err(wrong_smooth, ref)) > 0.1                     # k_smooth_inv for q_smooth
    assert np.max(A.row_rel_err(res["out"] * D, ref)) > 0.1                   # missing / 512


def test_p_tilde_is_fp32_normal():
    """p~ = 2^(s - m) is an fp32 value in the normal range: 2^-126 and above stay (correctly
    rounded), results below 2^-126 are 0.  In a one-tile MXFP4 row, a 32-token block whose
    logits sit 125 below the tile maximum keeps p~ = 2^-125 and E8M0 scale 2^-127 (the MX rule
    floor(log2 amax) - 2 at its clamp), so its codes are RNE(2^-125 / 2^-127) = 4, not zero;
    a block 127.5 below (p~ would be 2^-127.5, subnormal) is all zero, and so is a block at
    -inf; zero_blocks counts exactly those two of the row's four blocks."""
    x = np.array([0.0, -1.0, -126.0, -125.5, -126.25, -127.0, -140.0, -np.inf])
    p = A.p_tilde_fp32(x)
    want = np.array([1.0, 0.5, 2.0 ** -126, F32(2.0 ** -125.5), 0.0, 0.0, 0.0, 0.0], F32)
    assert p.dtype == F32 and np.array_equal(p, want)
    s = np.full((1, 128), -np.inf, F32)
    s[0, :32] = 0.0
    s[0, 32:64] = -125.0
    s[0, 64:96] = -127.5
    vhat = np.ones((128, 4))
    res = A.attend(s, vhat, 128, KQ.MXFP4, partials=True)
    codes = res["p_codes"].reshape(4, 32)
    assert np.all(codes[0] == 6)                      # p~ = 1 over MX scale 2^-2 is 4: code 6
    assert np.all(codes[1] == 6)                      # 2^-125 / 2^-127 = 4: code 6
    assert np.all((codes[2] & 7) == 0) and np.all((codes[3] & 7) == 0)
    assert res["zero_blocks"] == 2
