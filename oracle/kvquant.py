"""KV-append quantizers: Outlier-Aware Key Quantization, value blocks, MLA latent tiles.

Test infrastructure only (see ``oracle/__init__``).

What the pages fix: keys get static smoothing, a Hadamard rotation and a
scale search under token-wise scaling ([Abstract]; [Blog/New] "Outlier-Aware
Key Quantization"; [Explainer/Analyse]: the search picks a better-fitted
factor for each group of values).  Values and the search details are not
described; the readings below fill them in.

Readings:
* R6   Scale search per block (a block = B consecutive channels of one token,
       B = 16 NVFP4 / 32 MXFP4).  Candidates in this order: NVFP4 scale codes
       c0, c0+1, c0-1, c0-2, c0-3 (kept in [0, 0x7E]); MXFP4 exponents e0,
       e0+1, e0-1 (kept in [-127, 127]).  Objective: err = sum_i fl32(d_i*d_i)
       accumulated in index order from +0 in fp32, d_i = fl32(x_i - xhat_i)
       with xhat the fp32 dequantised value.  The first candidate with a
       strictly smaller err wins (ties keep the earlier candidate).
* R4   Values are scaled channel-wise over blocks of B consecutive tokens
       (page aligned), because the P.V contraction runs over tokens and a
       block-scaled FP4 product needs its scales along the contraction axis.
       Values get no smoothing, rotation or search (the pages apply the outlier
       treatment to keys only) and use the default scale.
* R5   A partially filled token block (the sequence tail) is quantized as if
       the absent tokens were +0.0: the scale covers the present tokens and the
       absent slots hold code 0.  Re-quantizing the block on each append gives
       the same bytes as quantizing the final sequence in one go.
* R14  MLA: the latent (smoothed, rotated over its 512 channels) serves as key
       and as value, so its scale blocks are 2-D tiles of B tokens x B
       channels, searched like key blocks with the objective summed in
       (token, channel) index order.

Pins (tests/test_oracle_kvquant.py): the chosen candidate is the first
strict argmin of the objective over the window (checked by brute force over
all candidates), the search never does worse than the default scale, the
window holds the global optimum over all 127 E4M3 codes on most random
blocks (gap reported), codes and scales of one-shot vs. token-by-token tail
re-quantization agree, and decoded values reproduce the inputs within the
half-step bound.
"""
import numpy as np

from .codecs import E4M3_MAX_CODE, mx_shared_exp
from .blockfmt import (NV_BLOCK, MX_BLOCK, blocks, nvfp4_default_scale, nvfp4_encode,
                       nvfp4_dequant_f32, mx_encode, mx_dequant_f32, mx_scale_code)
from .transforms import rotate_keys

F32 = np.float32
NVFP4 = 0
MXFP4 = 1
NV_DELTAS = (1, -1, -2, -3)
MX_DELTAS = (1, -1)


def block_size(fmt):
    return NV_BLOCK if fmt == NVFP4 else MX_BLOCK


def _sse_f32(x, xhat):
    """sum_i fl32(d_i^2) in index order over the last axis, d_i = fl32(x_i - xhat_i)."""
    d = (np.asarray(x, F32) - np.asarray(xhat, F32)).astype(F32)
    err = np.zeros(d.shape[:-1], dtype=F32)
    for i in range(d.shape[-1]):
        err = (err + (d[..., i] * d[..., i]).astype(F32)).astype(F32)
    return err


def search_nvfp4(xb, G, search=True):
    """Scale search over NVFP4 blocks xb[N, n] with tensor scale G (scalar or [N]).

    Returns (scale_codes uint8 [N], codes uint8 [N, n]).  Reading R6.
    """
    xb = np.asarray(xb, F32)
    G = np.broadcast_to(np.asarray(G, F32), xb.shape[:-1])
    amax = np.max(np.abs(xb), axis=-1)
    c0 = nvfp4_default_scale(amax, G).astype(np.int64)
    best_c = c0.copy()
    best_codes = nvfp4_encode(xb, c0, G)
    best_err = _sse_f32(xb, nvfp4_dequant_f32(best_codes, c0, G))
    if search:
        for delta in NV_DELTAS:
            c = c0 + delta
            ok = (c >= 0) & (c <= E4M3_MAX_CODE)
            cc = np.clip(c, 0, E4M3_MAX_CODE)
            codes = nvfp4_encode(xb, cc, G)
            err = _sse_f32(xb, nvfp4_dequant_f32(codes, cc, G))
            better = ok & (err < best_err)
            best_c = np.where(better, cc, best_c)
            best_err = np.where(better, err, best_err)
            best_codes = np.where(better[..., None], codes, best_codes)
    return best_c.astype(np.uint8), best_codes.astype(np.uint8)


def search_mxfp4(xb, search=True):
    """Scale search over MXFP4 blocks xb[N, n].  Returns (E8M0 bytes [N], codes [N, n])."""
    xb = np.asarray(xb, F32)
    amax = np.max(np.abs(xb), axis=-1)
    e0 = mx_shared_exp(amax)
    best_e = e0.copy()
    best_codes = mx_encode(xb, e0)
    best_err = _sse_f32(xb, mx_dequant_f32(best_codes, e0))
    if search:
        for delta in MX_DELTAS:
            e = e0 + delta
            ok = (e >= -127) & (e <= 127)
            ec = np.clip(e, -127, 127)
            codes = mx_encode(xb, ec)
            with np.errstate(over="ignore", invalid="ignore"):
                err = _sse_f32(xb, mx_dequant_f32(codes, ec))
            better = ok & (err < best_err)
            best_e = np.where(better, ec, best_e)
            best_err = np.where(better, err, best_err)
            best_codes = np.where(better[..., None], codes, best_codes)
    return mx_scale_code(best_e), best_codes.astype(np.uint8)


def quantize_keys(K, k_smooth_inv, G, fmt, search=True, rotate=True):
    """Keys of one KV head, K float32 [L, d] -> (codes [L, d] 4-bit, scales [L, d/B]).

    x = FWHT(fl32(K * k_smooth_inv)); each token's blocks of B channels are
    scale-searched (R6) -- the token-wise scaling of [Abstract].
    """
    K = np.asarray(K, F32)
    L, d = K.shape
    B = block_size(fmt)
    x = rotate_keys(K, k_smooth_inv, rotate)
    xb = blocks(x, B).reshape(L * (d // B), B)
    if fmt == NVFP4:
        sc, codes = search_nvfp4(xb, G, search)
    else:
        sc, codes = search_mxfp4(xb, search)
    return codes.reshape(L, d), sc.reshape(L, d // B)


def quantize_values(V, G, fmt):
    """Values of one KV head, V float32 [L, d] -> (codes [Lpad, d] token-major, scales [d, Lpad/B]).

    Channel-wise scaling over page-aligned blocks of B tokens (R4), default
    scale, partial tail block zero-filled (R5).  Lpad = ceil(L/B)*B.
    """
    V = np.asarray(V, F32)
    L, d = V.shape
    B = block_size(fmt)
    nblk = -(-L // B)
    Vp = np.zeros((nblk * B, d), dtype=F32)
    Vp[:L] = V
    vb = Vp.reshape(nblk, B, d).transpose(2, 0, 1)          # [d, nblk, B]
    amax = np.max(np.abs(vb), axis=-1)
    if fmt == NVFP4:
        sc = nvfp4_default_scale(amax, G)
        codes = nvfp4_encode(vb, sc, np.broadcast_to(np.asarray(G, F32), sc.shape))
    else:
        e = mx_shared_exp(amax)
        codes = mx_encode(vb, e)
        sc = mx_scale_code(e)
    codes_tm = codes.transpose(1, 2, 0).reshape(nblk * B, d)   # token-major
    return codes_tm.astype(np.uint8), sc.astype(np.uint8)


def quantize_latent(K, k_smooth_inv, G, fmt, search=True, rotate=True):
    """MLA latent of one sequence, K float32 [L, D] -> (codes [Lpad, D], tile scales [Lpad/B, D/B], x).

    x = FWHT_D(fl32(K * k_smooth_inv)) per token; 2-D tiles of B tokens x B
    channels share one scale, searched with the objective in (token, channel)
    order (R14); absent tail tokens are +0.0 (R5).  Also returns the fp32
    transformed latent x [L, D] (what the append path stages for the tail).
    """
    K = np.asarray(K, F32)
    L, D = K.shape
    B = block_size(fmt)
    x = rotate_keys(K, k_smooth_inv, rotate)
    nblk = -(-L // B)
    xp = np.zeros((nblk * B, D), dtype=F32)
    xp[:L] = x
    tiles = xp.reshape(nblk, B, D // B, B).transpose(0, 2, 1, 3).reshape(nblk * (D // B), B * B)
    if fmt == NVFP4:
        sc, codes = search_nvfp4(tiles, G, search)
    else:
        sc, codes = search_mxfp4(tiles, search)
    codes = codes.reshape(nblk, D // B, B, B).transpose(0, 2, 1, 3).reshape(nblk * B, D)
    return codes.astype(np.uint8), sc.reshape(nblk, D // B).astype(np.uint8), x
