"""Pins of the oracle's random scorer (Random Attention blog summary, Algorithm 1).

The pages leave `rand` unspecified; the reading is Philox4x64-10 (Salmon et al.,
SC 2011).  The oracle's generator is pinned to numpy's independent Philox
implementation (a library routine), the score layout to its stated definition,
and the draw's statistics to what a uniform independent draw must satisfy.
"""

import math

import numpy as np
import pytest

import oracle

MASK64 = (1 << 64) - 1


def numpy_philox_block(counter, key):
    """Philox4x64-10 block via numpy.random.Philox (it bumps the counter before each block)."""
    c = sum(int(w) << (64 * k) for k, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = [(c >> (64 * k)) & MASK64 for k in range(4)]
    # uint64 arrays: numpy routes a list of large Python ints through float64
    g = np.random.Philox(key=np.array([int(key[0]), int(key[1])], dtype=np.uint64),
                         counter=np.array(words, dtype=np.uint64))
    return [int(x) for x in g.random_raw(4)]


@pytest.mark.parametrize("seed", [0, 1, 12345, 2**63 + 17])
def test_philox_matches_numpy(seed):
    rng = np.random.default_rng(seed % 1000)
    cases = [([0, 0, 0, 0], [0, 0]), ([1, 0, 0, 0], [seed & MASK64, 0]),
             ([MASK64] * 4, [MASK64, MASK64])]
    for _ in range(40):
        ctr = [int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.uint64)]
        ctr[0] |= 1  # avoid the all-borrow counter edge in the numpy helper
        key = [seed & MASK64, int(rng.integers(0, 2**63, dtype=np.uint64))]
        cases.append((ctr, key))
    for ctr, key in cases:
        if all(w == 0 for w in ctr):
            # numpy cannot start below zero; check the block at counter 0 through counter MAX+1 wrap
            g = np.random.Philox(key=np.array(key, dtype=np.uint64),
                                 counter=np.array([MASK64] * 4, dtype=np.uint64))
            expect = [int(x) for x in g.random_raw(4)]
        else:
            expect = numpy_philox_block(ctr, key)
        got = [int(x) for x in oracle.philox4x64_10(ctr, key)]
        assert got == expect, (ctr, key)


def test_random_draw_layout_matches_numpy():
    """Score of slot i = top 24 bits of word i%4 of the block at (i//4, head, layer, req<<32|round)."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        seed = int(rng.integers(0, 2**63))
        req = int(rng.integers(0, 1000))
        layer = int(rng.integers(0, 64))
        head = int(rng.integers(0, 16))
        rnd = int(rng.integers(0, 100))
        i = int(rng.integers(4, 40000))
        words = numpy_philox_block([i // 4, head, layer, (req << 32) | rnd], [seed, 0])
        expect = (words[i % 4] >> 40) / float(1 << 24)
        assert oracle.random_draw(seed, req, layer, head, rnd, i) == expect


def test_scores_shape_prompt_and_grid():
    L, H, n, prot = 3, 4, 1088, 32
    s = oracle.score_random(L, H, n, prot, seed=0, round_id=0, shared_draw=False,
                            list_begin=0, list_end=2 * L * H)
    assert s.shape == (2 * L * H, n)
    assert np.all(np.isposinf(s[:, :prot]))
    body = s[:, prot:].astype(np.float64)
    assert np.all(body >= 0.0) and np.all(body < 1.0)
    scaled = body * (1 << 24)
    assert np.all(scaled == np.floor(scaled))  # 24-bit grid, exact in fp32


def test_list_numbering_matches_draw():
    """List (req*L + layer)*H + head draws from (req, layer, head); shared lists from head 0."""
    L, H, n, prot, seed, rnd = 3, 4, 40, 5, 99, 7
    s = oracle.score_random(L, H, n, prot, seed, rnd, False, 0, 2 * L * H)
    sh = oracle.score_random(L, H, n, prot, seed, rnd, True, 0, 2 * L)
    for req in range(2):
        for layer in range(L):
            for head in range(H):
                row = s[(req * L + layer) * H + head]
                for i in range(prot, n):
                    assert row[i] == np.float32(oracle.random_draw(seed, req, layer, head, rnd, i))
            assert np.array_equal(sh[req * L + layer], s[(req * L + layer) * H + 0])


def test_uniformity_chi2():
    """256-bin chi-square of 1M draws stays below the 99.9% quantile (df=255 -> ~330.5)."""
    s = oracle.score_random(36, 8, 4096, 0, seed=3, round_id=0, shared_draw=False,
                            list_begin=0, list_end=256)
    counts = np.bincount((s.ravel() * 256).astype(np.int64), minlength=256)
    expect = s.size / 256.0
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 330.5, chi2


def rco(a, b, N):
    """Random-corrected overlap of two keep sets (WakeKV, Sec. 2.1 head churn)."""
    K = min(len(a), len(b))
    inter = len(set(a.tolist()) & set(b.tolist()))
    return max(0.0, (inter / K - K / N) / (1 - K / N))


def test_heads_independent_shared_identical():
    """Per-head draws give keep sets with chance-level overlap; the shared draw gives one set."""
    L, H, n, K, prot = 1, 8, 1088, 1024, 128
    s = oracle.score_random(L, H, n, prot, seed=11, round_id=0, shared_draw=False,
                            list_begin=0, list_end=64 * H)
    kept = oracle.select_topk(s, K, prot)
    N, k = n - prot, K - prot
    inters = []
    for req in range(64):
        a = kept[req * H + 0, prot:]
        b = kept[req * H + 1, prot:]
        inters.append(len(set(a.tolist()) & set(b.tolist())))
    # |A & B| of two independent uniform k-subsets of N is hypergeometric, mean k^2/N.
    mean = k * k / N
    var = k * (k / N) * ((N - k) / N) * ((N - k) / (N - 1))
    got = float(np.mean(inters))
    assert abs(got - mean) < 4 * math.sqrt(var / len(inters)), (got, mean)
    assert rco(kept[0, prot:], kept[1, prot:], N) < 0.35
    sh = oracle.score_random(L, H, n, prot, seed=11, round_id=0, shared_draw=True,
                             list_begin=0, list_end=4)
    ks = oracle.select_topk(sh, K, prot)
    assert np.array_equal(ks[0], kept[0])  # shared draw == head 0's per-head draw
    assert rco(ks[0, prot:], ks[0, prot:], N) == 1.0


def test_rounds_redraw():
    """Different round ids give uncorrelated draws (fresh draw every eviction)."""
    a = oracle.score_random(1, 1, 100000, 0, 5, 0, False, 0, 1)[0].astype(np.float64)
    b = oracle.score_random(1, 1, 100000, 0, 5, 1, False, 0, 1)[0].astype(np.float64)
    corr = np.corrcoef(a, b)[0, 1]
    assert abs(corr) < 0.02
