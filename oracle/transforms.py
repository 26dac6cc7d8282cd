"""Static smoothing and the Hadamard rotation used by the key and query paths.

Test infrastructure only (see ``oracle/__init__``).

The method suppresses key outliers by combining a static per-channel
smoothing with a Hadamard rotation over head_dim before token-wise scaling
([Abstract]; [Blog/New]; [Explainer/Analyse] says smoothing and rotation
spread the outlier energy).  The queries receive the inverse smoothing and
the same rotation so logits are unchanged.

Readings:
* R7  The smoothing vector is a caller input per KV head: keys are
      multiplied by ``k_smooth_inv`` and queries by ``q_smooth`` with
      q_smooth * k_smooth_inv == 1 exactly (powers of two).
* R8  The rotation is the plain Sylvester Hadamard matrix, unnormalised,
      applied as a fast Walsh-Hadamard transform whose stages run with
      h = 1, 2, 4, ..., n/2 in that order; each stage replaces the pair
      (u_i, u_{i+h}), i & h == 0, by (fl32(u_i + u_{i+h}), fl32(u_i - u_{i+h})).
      <x H, y H> = n <x, y>, so the 1/n is folded into the logit coefficient.

Pins (tests/test_oracle_transforms.py): equals u @ scipy.linalg.hadamard(n)
exactly on integer inputs (no rounding happens) and within the fp32 error
bound log2(n) * eps * sum|u| on random inputs; fwht(fwht(u)) == n * u on
integer inputs; logit invariance <(q*l)H, (k/l)H> / n == <q, k> in fp64.
"""
import numpy as np

F32 = np.float32


def fwht_f32(u):
    """Unnormalised fast Walsh-Hadamard transform over the last axis in float32 (R8)."""
    u = np.array(u, dtype=F32, copy=True, order="C")
    n = u.shape[-1]
    assert n >= 1 and (n & (n - 1)) == 0, "length must be a power of two"
    lead = u.shape[:-1]
    h = 1
    while h < n:
        v = u.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return u


def smooth(x, factors):
    """fl32(x * factors) with the per-channel factors broadcast over the last axis (R7)."""
    return (np.asarray(x, dtype=F32) * np.asarray(factors, dtype=F32)).astype(F32)


def rotate_keys(k, k_smooth_inv, rotate=True):
    """x = FWHT(fl32(k * k_smooth_inv)) -- the transformed key the cache stores."""
    x = smooth(k, k_smooth_inv)
    return fwht_f32(x) if rotate else x


def rotate_queries(q, q_smooth, rotate=True):
    """y = FWHT(fl32(q * q_smooth)) -- the transformed query the dual quantizer sees."""
    y = smooth(q, q_smooth)
    return fwht_f32(y) if rotate else y
