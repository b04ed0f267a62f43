"""The KeyDiff tolerance the GPU tests use (keydiff_bound) holds against a change of summation
order, checked on the CPU.

The library's binary64 KeyDiff cosine (GateSight Sec. 5.1, baselines paragraph) adds the column
sums, the dot products with the mean and the squared norms in another order than the oracle's
plain loops.  `keydiff_bound` states how far the two binary64 cosines may lie apart.  Here three
orders written out independently in numpy (sequential loops; a blocked order shaped like the
kernel's: per-lane partial sums of 8 elements, a tree over 16 lanes, strided row groups reduced
in a tree; and a fully reversed order) and the oracle's own (numpy's pairwise sums and BLAS dot
products) are compared pairwise against that bound, on ordinary keys, on keys whose sum cancels
(the bound's ratio term), on one key and on D = 8.
"""

import numpy as np
import pytest

import oracle
from test_gpu_parity import keydiff_bound, rand_keys


def _seq(v):
    """Sum over the last axis, left to right."""
    acc = v[..., 0].copy()
    for e in range(1, v.shape[-1]):
        acc = acc + v[..., e]
    return acc


def _tree(v):
    """Sum over the last axis (a power of two long) in a pairwise tree."""
    while v.shape[-1] > 1:
        v = v[..., 0::2] + v[..., 1::2]
    return v[..., 0]


def _cosines(k, col_sum, row_dot):
    """-cos(k_i, mean) per row of one list k [n][D] in binary64, from the given reductions."""
    n, D = k.shape
    mean = col_sum(k) / n
    mm = row_dot(mean[None, :], mean[None, :])[0]
    dot = row_dot(k, np.broadcast_to(mean, k.shape))
    kk = row_dot(k, k)
    den = np.sqrt(kk) * np.sqrt(mm)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(den > 0, -(dot / np.where(den > 0, den, 1.0)), 0.0)
    return c


def _seq_col(k):
    acc = k[0].copy()
    for i in range(1, k.shape[0]):
        acc = acc + k[i]
    return acc


def _rev_col(k):
    return _seq_col(k[::-1])


def _blocked_col(k, groups=32):
    """Rows r0 + 32 s summed by their group r0 over s in order, then a tree over the groups."""
    n, D = k.shape
    steps = -(-n // groups)
    pad = np.zeros((steps * groups, D))
    pad[:n] = k
    per_group = _seq_col(pad.reshape(steps, groups, D))  # [groups][D]
    return _tree(np.moveaxis(per_group, 0, -1))


def _seq_dot(a, b):
    return _seq(a * b)


def _rev_dot(a, b):
    return _seq((a * b)[..., ::-1])


def _blocked_dot(a, b):
    """Products in 16-byte vectors of 8 summed in order, then a tree over the vectors."""
    p = a * b
    D = p.shape[-1]
    if D % 8 or (D // 8) & (D // 8 - 1):
        return _seq(p)
    return _tree(_seq(p.reshape(*p.shape[:-1], D // 8, 8)))


def _cases():
    yield "batch shape", oracle.bf16_to_f64(rand_keys((1, 1088, 128), seed=3))[0]
    yield "D = 8", oracle.bf16_to_f64(rand_keys((1, 300, 8), seed=4))[0]
    yield "one key", oracle.bf16_to_f64(rand_keys((1, 1, 128), seed=5))[0]
    # pairs of nearly opposite keys and one more: the sum of the 1023 keys cancels to a small
    # remainder, and the mean divides by a count that is not a power of two
    base = oracle.bf16_to_f64(rand_keys((1, 511, 128), seed=6))[0]
    tweak = oracle.bf16_to_f64(rand_keys((1, 511, 128), seed=7))[0] * 2.0 ** -6
    extra = oracle.bf16_to_f64(rand_keys((1, 1, 128), seed=8))[0] * 2.0 ** -4
    k = np.concatenate([base, -base + tweak, extra])
    bits = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # back to bf16
    yield "cancelling sum", oracle.bf16_to_f64(bits[None])[0]


@pytest.mark.parametrize("name,k", list(_cases()), ids=[c[0] for c in _cases()])
def test_summation_orders_within_bound(name, k):
    n, D = k.shape
    bits = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)[None]
    assert np.array_equal(oracle.bf16_to_f64(bits)[0], k)  # the keys are bf16 values
    bound = keydiff_bound(bits)[0]
    orders = {
        "oracle": oracle.score_keydiff(bits, 0, binary64=True)[0],
        "sequential": _cosines(k, _seq_col, _seq_dot),
        "blocked": _cosines(k, _blocked_col, _blocked_dot),
        "reversed": _cosines(k, _rev_col, _rev_dot),
    }
    names = list(orders)
    worst = 0.0
    for i, a in enumerate(names):
        for b in names[i + 1:]:
            d = np.abs(orders[a] - orders[b])
            assert np.all(d <= bound), (name, a, b, float(d.max()), bound)
            worst = max(worst, float(d.max()) / bound if bound > 0 else 0.0)
    # the orders do differ where the mean is inexact (a count that is not a power of two), so
    # the check is not vacuous there; with few significant bits the rest can be exact in
    # binary64, and then every order agrees
    if name in ("batch shape", "cancelling sum"):
        assert not np.array_equal(orders["sequential"], orders["blocked"])
        assert not np.array_equal(orders["oracle"], orders["reversed"])
    print(f"{name}: largest difference {worst:.3g} of the bound")
