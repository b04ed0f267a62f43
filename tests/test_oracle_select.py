"""Pins of the oracle's per-head and global selection.

Per head (Random Attention blog summary, Algorithm 1): the prompt is pinned to
+inf and the top-K entries are kept; ties go to the lower position.  Global
(GateSight problem statement; KVzip-style global top-B over (layer, head,
token)): the prompt of every list is kept in addition to B entries, with
B = lists * round(p*(n-prot)).

Pins: brute-force enumeration on tiny inputs, numpy's stable argsort (a library
routine), closed-form special cases (recency, constant scores, n = K, p = 0/1),
and the budget identity.
"""

import itertools

import numpy as np
import pytest

import oracle


def canon(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(np.isnan(x), -np.inf, x)


def brute_force_topk(s, K, prot):
    """The unique K-subset containing the prompt whose kept entries all outrank the dropped ones."""
    n = len(s)
    v = canon(s)

    def beats(a, b):  # a ranks above b: larger score, or equal score and lower position
        return v[a] > v[b] or (v[a] == v[b] and a < b)

    found = []
    body = list(range(prot, n))
    for comb in itertools.combinations(body, K - prot):
        keep = set(comb)
        drop = [i for i in body if i not in keep]
        if all(beats(a, b) for a in keep for b in drop):
            found.append(sorted(list(range(prot)) + list(comb)))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    prot = int(rng.integers(0, n + 1))
    K = int(rng.integers(prot, n + 1))
    kind = seed % 3
    if kind == 0:
        s = rng.random(n).astype(np.float32)
    elif kind == 1:
        s = rng.integers(0, 3, n).astype(np.float32)  # many ties
    else:
        s = rng.choice(np.array([np.nan, -0.0, 0.0, 1.0, -np.inf, np.inf], dtype=np.float32), n)
    got = oracle.select_topk(s[None, :], K, prot)[0]
    assert got.tolist() == brute_force_topk(s, K, prot)


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(1)
    lists, n, K, prot = 50, 700, 500, 37
    s = (rng.integers(0, 50, (lists, n)) / 50.0).astype(np.float32)
    s[:, :prot] = np.inf
    got = oracle.select_topk(s, K, prot)
    for row in range(lists):
        order = np.argsort(-canon(s[row]), kind="stable")
        expect = np.sort(order[:K])
        assert np.array_equal(got[row], expect)


def test_topk_special_cases():
    n, K, prot = 300, 200, 20
    pos = np.arange(n, dtype=np.float32)[None, :]
    # recency: score = position keeps the prompt and the most recent K - prot entries
    got = oracle.select_topk(pos, K, prot)[0]
    assert got.tolist() == list(range(prot)) + list(range(n - (K - prot), n))
    # constant scores keep the oldest K entries
    got = oracle.select_topk(np.zeros((1, n), np.float32), K, prot)[0]
    assert got.tolist() == list(range(K))
    # n == K is the identity
    got = oracle.select_topk(np.random.default_rng(0).random((1, n)).astype(np.float32), n, prot)[0]
    assert got.tolist() == list(range(n))
    # prot == K keeps only the prompt
    got = oracle.select_topk(np.random.default_rng(0).random((1, n)).astype(np.float32), prot, prot)[0]
    assert got.tolist() == list(range(prot))
    # NaN ranks below -inf; -0 ties with +0 (lower position wins)
    s = np.array([[np.nan, 0.0, -0.0, -np.inf, np.nan, 1.0]], np.float32)
    assert oracle.select_topk(s, 3, 0)[0].tolist() == [1, 2, 5]
    s = np.array([[-0.0, 0.0, 0.0]], np.float32)
    assert oracle.select_topk(s, 1, 0)[0].tolist() == [0]
    s = np.array([[np.nan, -np.inf, np.nan]], np.float32)
    assert oracle.select_topk(s, 1, 0)[0].tolist() == [0]


def test_topk_invariants_random_draw():
    """Prompt always survives, indices strictly increase, |S| = K (blog summary keep-log)."""
    L, H, n, K, prot = 2, 8, 1088, 1024, 128
    s = oracle.score_random(L, H, n, prot, 0, 0, False, 0, 4 * L * H)
    kept = oracle.select_topk(s, K, prot)
    assert kept.shape == (4 * L * H, K)
    assert np.all(np.diff(kept, axis=1) > 0)
    assert np.all(kept[:, :prot] == np.arange(prot))
    assert kept.min() >= 0 and kept.max() < n


def brute_force_global(s, prot, B):
    lists, n = s.shape
    v = canon(s)
    cands = [(l, i) for l in range(lists) for i in range(prot, n)]

    def beats(a, b):
        fa, fb = a[0] * n + a[1], b[0] * n + b[1]
        return v[a] > v[b] or (v[a] == v[b] and fa < fb)

    found = []
    for comb in itertools.combinations(cands, B):
        keep = set(comb)
        drop = [c for c in cands if c not in keep]
        if all(beats(a, b) for a in keep for b in drop):
            found.append(keep)
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(8))
def test_global_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    lists, n = 3, 5
    prot = int(rng.integers(0, 3))
    p = [0.0, 0.25, 0.5, 0.75, 1.0, 0.34, 0.5, 0.6][seed]
    s = (rng.integers(0, 4, (lists, n)) / 4.0).astype(np.float32) if seed % 2 else \
        rng.random((lists, n)).astype(np.float32)
    kept, counts, B = oracle.select_global(s, prot, p)
    assert B == lists * int(np.round(p * (n - prot)))  # numpy rounds half to even
    keep = brute_force_global(s, prot, B)
    for l in range(lists):
        expect = sorted(list(range(prot)) + [i for (ll, i) in keep if ll == l])
        assert counts[l] == len(expect)
        assert kept[l, :counts[l]].tolist() == expect
        assert np.all(kept[l, counts[l]:] == -1)


def test_global_budget_identity_and_closed_forms():
    rng = np.random.default_rng(5)
    lists, n, prot, p = 64, 600, 40, 0.25
    s = rng.random((lists, n)).astype(np.float32)
    kept, counts, B = oracle.select_global(s, prot, p)
    assert B == lists * round(p * (n - prot))
    assert int(counts.sum()) == lists * prot + B
    for l in range(lists):
        c = counts[l]
        assert np.all(np.diff(kept[l, :c]) > 0) and np.all(kept[l, :prot] == np.arange(prot))
    # identical score arrays in every list: each list keeps prot + round(p(n-prot)), and the
    # keep set equals the per-head top-K with K = prot + round(p(n-prot))
    row = rng.permutation(n).astype(np.float32)
    same = np.tile(row, (lists, 1))
    kept, counts, B = oracle.select_global(same, prot, p)
    per = round(p * (n - prot))
    assert np.all(counts == prot + per)
    ref = oracle.select_topk(same, prot + per, prot)
    assert np.array_equal(kept[:, :prot + per], ref)
    # well-separated lists: the best lists are kept whole, in order
    sep = rng.random((8, 50)).astype(np.float32) + 10.0 * np.arange(8, dtype=np.float32)[:, None]
    kept, counts, B = oracle.select_global(sep, 0, 0.5)
    assert B == 8 * 25
    assert counts.tolist() == [0, 0, 0, 0, 50, 50, 50, 50]
    # p = 0 keeps only the prompts; p = 1 keeps everything
    kept, counts, B = oracle.select_global(s, prot, 0.0)
    assert B == 0 and np.all(counts == prot)
    kept, counts, B = oracle.select_global(s, prot, 1.0)
    assert np.all(counts == n) and np.all(kept == np.arange(n))


def test_budget_rounding_half_even():
    assert oracle.budget(1, 7, 2, 0.5) == 2    # 2.5 -> 2
    assert oracle.budget(1, 9, 2, 0.5) == 4    # 3.5 -> 4
    assert oracle.budget(64, 32768, 256, 0.25) == 16 * 4 * 8128 == 520192
