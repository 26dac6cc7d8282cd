"""The hardware FP4 conversion that quantizes the probabilities (v_cvt_scalef32_pk_fp4_f32,
through the library's fp4kv_pack_e2m1) against the oracle's E2M1 encoder (round to nearest,
ties to the even code, saturation at 6): every decision threshold (the ties), its fp32
neighbours, the grid points, values past 6 and infinity, zeros and subnormals, and random
values, at several power-of-two scales.  Probabilities are never negative, so the decode only
relies on the non-negative half; the negative half is checked as well, its signed zero
reported."""
import numpy as np
import pytest

from oracle import codecs as C
from _gpu import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from fp4_kv_cache_amd import lib
    lib.load()
    return torch


def _inputs():
    F = np.float32
    th = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], F)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], F)
    near = np.concatenate([np.nextafter(th, F(0)), th, np.nextafter(th, F(np.inf))])
    big = np.array([6.0, np.nextafter(F(6), F(np.inf)), 7.0, 100.0, 3.0e38, np.inf], F)
    small = np.array([0.0, 1e-45, 1e-40, 1.17e-38, 1e-10, 0.1], F)
    rng = np.random.default_rng(60)
    rand = (rng.random(4000) * 8).astype(F)
    pos = np.concatenate([near, grid, big, small, rand])
    x = np.concatenate([pos, -pos])
    pad = (-len(x)) % 8
    return np.concatenate([x, np.zeros(pad, F)])


@pytest.mark.parametrize("e", [0, -10, -3, 4, -19])
def test_hardware_fp4_convert_matches_the_encoder(torch_dev, e):
    import torch
    from fp4_kv_cache_amd import lib as L
    base = _inputs()
    with np.errstate(over="ignore"):
        x = (base.astype(np.float64) * 2.0 ** e).astype(np.float32)
    # the encoder sees exactly what the hardware divides: x / 2^e (equal to base except
    # where the scaling overflowed or underflowed)
    base = (x.astype(np.float64) / 2.0 ** e).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    out = torch.zeros(len(x) // 2, dtype=torch.uint8, device="cuda")
    L.check(L.fp4kv_pack_e2m1(xt.data_ptr(), len(x), e, out.data_ptr(),
                              torch.cuda.current_stream().cuda_stream), "fp4kv_pack_e2m1")
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    got = np.stack([o & 0xF, o >> 4], axis=-1).reshape(-1)
    want = C.e2m1_encode(base)
    nonneg = ~np.signbit(base)
    bad = np.nonzero(got[nonneg] != want[nonneg])[0]
    assert bad.size == 0, [(float(base[nonneg][i]), int(got[nonneg][i]), int(want[nonneg][i])) for i in bad[:10]]
    neg_diff = np.nonzero(got[~nonneg] != want[~nonneg])[0]
    say("scale 2^%d: %d non-negative values agree; negative half: %d differ (%s)"
        % (e, int(nonneg.sum()), neg_diff.size,
           sorted({(float(base[~nonneg][i]), int(got[~nonneg][i]), int(want[~nonneg][i])) for i in neg_diff[:6]})))
    # every negative value that does not round to zero agrees
    nz = ~nonneg & ((want & 7) != 0)
    assert np.array_equal(got[nz], want[nz])



def _verify_slice(start, n, codes, e):
    """Oracle codes of the fp32 patterns start .. start + n - 1 divided by 2^e, against the
    hardware's codes (one nibble per pattern); NaN patterns are skipped.  Returns
    (patterns checked, first mismatches)."""
    x = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        base = x * np.float32(2.0 ** -e)   # exact unless it overflows to infinity or underflows
    want = C.e2m1_encode(base)
    got = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(-1)
    keep = ~np.isnan(x)
    bad = np.nonzero((got != want) & keep)[0]
    return int(keep.sum()), [(hex(start + int(i)), int(got[i]), int(want[i])) for i in bad[:4]]


@pytest.mark.parametrize("e", [0, -10])
def test_hardware_fp4_convert_exhaustive(torch_dev, e):
    """Every fp32 bit pattern except the NaNs (a caller error for the encoder), both signs,
    through the hardware conversion at scale 2^e: its code equals the oracle's encoder's code
    of x / 2^e (a power-of-two division, rounded only where it overflows to infinity or
    underflows, and those values land on the same code either way).  The patterns are made on
    the GPU; the oracle checks them in slices on a thread pool."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from fp4_kv_cache_amd import lib as L
    CH, SL = 1 << 26, 1 << 22
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty(CH // 2, dtype=torch.uint8, device="cuda")
    checked, bad = 0, []
    with ThreadPoolExecutor(8) as pool:
        for start in range(0, 1 << 32, CH):
            u = torch.arange(start, start + CH, dtype=torch.int64, device="cuda")
            xt = torch.where(u >= (1 << 31), u - (1 << 32), u).to(torch.int32).view(torch.float32)
            L.check(L.fp4kv_pack_e2m1(xt.data_ptr(), CH, e, out.data_ptr(), stream), "fp4kv_pack_e2m1")
            o = out.cpu().numpy()
            res = list(pool.map(lambda k: _verify_slice(start + k, SL, o[k // 2:(k + SL) // 2], e), range(0, CH, SL)))
            checked += sum(r[0] for r in res)
            bad += [b for r in res for b in r[1]]
            assert not bad, ("scale 2^%d" % e, bad[:8])
    say("scale 2^%d: all %d non-NaN fp32 patterns give the oracle's E2M1 code" % (e, checked))
    assert checked == (1 << 32) - 2 * ((1 << 23) - 1)
