"""Oracle pins for the KeyDiff key score (GateSight Sec. 5.1, baselines paragraph): a key
scores minus its cosine to the plain average of its head's keys, so a per-head top-K keeps
the keys that point away from that average."""

import math

import numpy as np

import oracle


def bf16_bits(x) -> np.ndarray:
    """float values exactly representable in bf16 -> uint16 bits."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "values must be exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_worked_example():
    # keys (1,0), (0,1), (1,1): mean (2/3, 2/3); cos = 1/sqrt2, 1/sqrt2, 1
    keys = bf16_bits([[[1, 0], [0, 1], [1, 1]]])
    s = oracle.score_keydiff(keys, 0)[0]
    assert np.allclose(s, [-1 / math.sqrt(2), -1 / math.sqrt(2), -1.0], rtol=0, atol=1e-7)
    assert s[0] == s[1] == np.float32(-1 / math.sqrt(2))
    # the least similar keys rank first: (1,0) and (0,1) before (1,1)
    assert list(oracle.select_topk(s[None, :], 2, 0)[0]) == [0, 1]


def test_identical_keys_orthogonal_and_opposite():
    v = [1.5, -2.0, 0.25, 4.0]
    keys = bf16_bits([[v] * 5])
    assert np.all(oracle.score_keydiff(keys, 0) == np.float32(-1.0))   # cos = 1 everywhere
    # mean (1, 0) from rows (2,0), (0,1), (0,-1): the vertical keys are orthogonal -> 0
    keys = bf16_bits([[[2, 0], [0, 1], [0, -1]]])
    s = oracle.score_keydiff(keys, 0)[0]
    assert s[0] == np.float32(-1.0) and s[1] == 0.0 and s[2] == 0.0
    # a key opposite to the mean: cos = -1, score +1
    keys = bf16_bits([[[3, 0], [3, 0], [-1, 0]]])
    assert oracle.score_keydiff(keys, 0)[0, 2] == np.float32(1.0)


def test_zero_key_zero_mean_and_prompt():
    keys = bf16_bits([[[0, 0], [1, 2], [3, 1], [2, 2]], [[1, 2], [-1, -2], [3, -1], [-3, 1]]])
    s = oracle.score_keydiff(keys, 1)
    assert np.isposinf(s[0, 0]) and np.isposinf(s[1, 0])  # the prompt is pinned
    assert np.all(s[1, 1:] == 0.0)                           # the second list's mean is 0
    assert np.all(np.isfinite(s[:, 1:]))
    z = oracle.score_keydiff(bf16_bits([[[0, 0], [1, 0]]]), 0)[0]
    assert z[0] == 0.0 and math.copysign(1, z[0]) > 0       # zero key: +0


def test_scale_invariance_and_range():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((3, 40, 16)).astype(np.float32)
    k = (k.view(np.uint32) & 0xFFFF0000).view(np.float32)  # exact bf16 values
    s1 = oracle.score_keydiff(bf16_bits(k), 4)
    s2 = oracle.score_keydiff(bf16_bits(k * 4), 4)         # exact: a power-of-two scale
    assert np.array_equal(s1, s2)
    fin = s1[:, 4:]
    assert np.all(fin >= -1.0000001) and np.all(fin <= 1.0000001)
    # against a direct cosine written with numpy's norm routine
    kk = k.astype(np.float64)
    mean = kk.mean(axis=1, keepdims=True)
    cos = (kk * mean).sum(-1) / (np.linalg.norm(kk, axis=-1) * np.linalg.norm(mean, axis=-1))
    assert np.allclose(fin, -cos[:, 4:], rtol=1e-6, atol=1e-7)
