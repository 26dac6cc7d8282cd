"""Paged cache layout (oracle side): scatter one sequence's quantized data into pages
and gather it back, byte for byte as the library lays it out.

Test infrastructure only (see ``oracle/__init__``).

The pages say the cache is paged and read in full at every decode step
([Abstract]; [Blog/Why]); the byte layout below is this library's own
format, written here independently of the HIP code from the format's
definition.  P = page size (tokens), B = scale block (16 NVFP4 / 32 MXFP4),
h = KV head, a physical page holds ``P`` consecutive tokens of one sequence,
and a token's page is ``block_table[seq][pos // P]``, its slot ``pos % P``.

GQA (per page, per KV head; head_dim d = 128):
  k_codes  uint8 [num_pages][Hkv][P][d/2]   token-major, byte j = c[2j] | c[2j+1] << 4
  k_scales uint8 [num_pages][Hkv][P*d/B]    one scale per (token t, channel block q) at
                                            kscale_index(t, q): NVFP4 t*8 + q; MXFP4
                                            (((t//32)*4 + t%4)*4 + q)*8 + (t%32)//4
  v_codes  uint8 [num_pages][Hkv][d][P/2]   channel-major, byte j = tok[2j] | tok[2j+1] << 4
  v_scales uint8 [num_pages][Hkv][d*P/B]    one scale per (channel c, token block j) at
                                            ((j//J)*16 + c%16)*8*J + (c//16)*J + j%J,
                                            J = min(P, 32)//B blocks per 32-token span
MLA (one latent head, D = 512, rope r = 64):
  k_codes  uint8 [num_pages][1][P][D/2]     token-major latent (key and value)
  k_scales uint8 [num_pages][1][P/B][D/B]   one scale per (B-token, B-channel) tile
  k_rope   bf16  [num_pages][1][P][r]       unquantized rope key (stored as uint16 here)
"""
import numpy as np

from .codecs import pack_nibbles, unpack_nibbles
from .kvquant import block_size


def n_pages(L, P):
    return -(-L // P)


def kscale_index(t, q, fmt):
    """Byte offset of the key scale of (page-local token t, channel block q)."""
    t, q = np.asarray(t), np.asarray(q)
    if fmt == 0:
        return t * 8 + q
    return (((t // 32) * 4 + t % 4) * 4 + q) * 8 + (t % 32) // 4


def vscale_index(c, j, P, fmt):
    """Byte offset of the value scale of (channel c, page-local token block j)."""
    c, j = np.asarray(c), np.asarray(j)
    J = min(P, 32) // block_size(fmt)
    return ((j // J) * 16 + c % 16) * 8 * J + (c // 16) * J + j % J


def scatter_gqa(cache, h, bt_row, L, kc, ks, vc, vs, fmt):
    """Write one sequence's KV-head-h data (from quantize_keys/quantize_values) into the pages."""
    P = cache["k_codes"].shape[2]
    d = cache["k_codes"].shape[3] * 2
    B = block_size(fmt)
    kpk = pack_nibbles(kc)
    for lp in range(n_pages(L, P)):
        pg = int(bt_row[lp])
        t0, t1 = lp * P, min(L, (lp + 1) * P)
        cache["k_codes"][pg, h, : t1 - t0] = kpk[t0:t1]
        ki = kscale_index(np.arange(t1 - t0)[:, None], np.arange(ks.shape[1])[None, :], fmt)
        cache["k_scales"][pg, h, ki] = ks[t0:t1]
        # value blocks present in this page (the tail block is written whole)
        b0, b1 = t0 // B, -(-t1 // B)
        tv1 = b1 * B
        seg = vc[t0:tv1].T                                  # [d, tokens]
        cache["v_codes"][pg, h, :, : (tv1 - t0) // 2] = pack_nibbles(seg)
        vi = vscale_index(np.arange(d)[:, None], np.arange(b1 - b0)[None, :], P, fmt)
        cache["v_scales"][pg, h, vi] = vs[:, b0:b1]


def gather_gqa(cache, h, bt_row, L, fmt):
    """Read back (kc [L, d], ks [L, d/B], vc [Lpad, d] token-major, vs [d, Lpad/B])."""
    P = cache["k_codes"].shape[2]
    d = cache["k_codes"].shape[3] * 2
    B = block_size(fmt)
    nblk = -(-L // B)
    kc = np.zeros((L, d), np.uint8)
    ks = np.zeros((L, d // B), np.uint8)
    vc = np.zeros((nblk * B, d), np.uint8)
    vs = np.zeros((d, nblk), np.uint8)
    for lp in range(n_pages(L, P)):
        pg = int(bt_row[lp])
        t0, t1 = lp * P, min(L, (lp + 1) * P)
        kc[t0:t1] = unpack_nibbles(cache["k_codes"][pg, h, : t1 - t0])
        ki = kscale_index(np.arange(t1 - t0)[:, None], np.arange(d // B)[None, :], fmt)
        ks[t0:t1] = cache["k_scales"][pg, h, ki]
        b0, b1 = t0 // B, -(-t1 // B)
        tv1 = b1 * B
        vc[t0:tv1] = unpack_nibbles(cache["v_codes"][pg, h, :, : (tv1 - t0) // 2]).T
        vi = vscale_index(np.arange(d)[:, None], np.arange(b1 - b0)[None, :], P, fmt)
        vs[:, b0:b1] = cache["v_scales"][pg, h, vi]
    return kc, ks, vc, vs


def scatter_mla(cache, bt_row, L, lc, ls, k_rope_bits, fmt):
    """Write one MLA sequence: latent codes [Lpad, D], tile scales [Lpad/B, D/B], rope uint16 [L, r]."""
    P = cache["k_codes"].shape[2]
    B = block_size(fmt)
    lpk = pack_nibbles(lc)
    for lp in range(n_pages(L, P)):
        pg = int(bt_row[lp])
        t0, t1 = lp * P, min(L, (lp + 1) * P)
        b0, b1 = t0 // B, -(-t1 // B)
        tv1 = b1 * B
        cache["k_codes"][pg, 0, : tv1 - t0] = lpk[t0:tv1]
        cache["k_scales"][pg, 0, : b1 - b0] = ls[b0:b1]
        cache["k_rope"][pg, 0, : t1 - t0] = k_rope_bits[t0:t1]


def gather_mla(cache, bt_row, L, fmt):
    """Read back (lc [Lpad, D], ls [Lpad/B, D/B], k_rope uint16 [L, r])."""
    P = cache["k_codes"].shape[2]
    D = cache["k_codes"].shape[3] * 2
    r = cache["k_rope"].shape[3]
    B = block_size(fmt)
    nblk = -(-L // B)
    lc = np.zeros((nblk * B, D), np.uint8)
    ls = np.zeros((nblk, D // B), np.uint8)
    kr = np.zeros((L, r), np.uint16)
    for lp in range(n_pages(L, P)):
        pg = int(bt_row[lp])
        t0, t1 = lp * P, min(L, (lp + 1) * P)
        b0, b1 = t0 // B, -(-t1 // B)
        tv1 = b1 * B
        lc[t0:tv1] = unpack_nibbles(cache["k_codes"][pg, 0, : tv1 - t0])
        ls[b0:b1] = cache["k_scales"][pg, 0, : b1 - b0]
        kr[t0:t1] = cache["k_rope"][pg, 0, : t1 - t0]
    return lc, ls, kr
