"""Oracle pins for page-granular random eviction (Random Attention blog summary, Algorithm 1
over the blocks of a paged cache; GateSight Sec. 4.3: per-layer block tables over one pool)."""

import itertools

import numpy as np
import pytest

import oracle


def test_page_scores_are_the_first_slot_draws():
    L, n, ps = 3, 160, 16
    kept = oracle.page_keep_sets(L, n, 64, 0, ps, seed=5, round_id=2, group_begin=0, group_end=6)
    # the 4 of the 10 pages whose first slots drew the largest head-0 scores (lower page on ties)
    for g in range(6):
        req, layer = divmod(g, L)
        sc = [oracle.random_draw(5, req, layer, 0, 2, b * ps) for b in range(n // ps)]
        order = sorted(range(n // ps), key=lambda b: (-sc[b], b))
        assert list(kept[g]) == sorted(order[:4]), g


def test_prompt_pages_pinned_and_counts():
    L, n, K, ps = 2, 2112, 2048, 16
    for prot in (0, 1, 557, 1024, 2048):
        kept = oracle.page_keep_sets(L, n, K, prot, ps, seed=0, round_id=0, group_begin=0,
                                     group_end=4)
        pp = -(-prot // ps)
        assert kept.shape == (4, K // ps)
        assert np.all(np.diff(kept, axis=1) > 0)                 # increasing
        assert np.all(kept[:, :pp] == np.arange(pp))             # prompt pages first, kept
        assert np.all((kept >= 0) & (kept < n // ps))
    with pytest.raises(ValueError):
        oracle.page_keep_sets(L, 2100, K, 0, ps, 0, 0, 0, 1)     # partial page
    with pytest.raises(ValueError):
        oracle.page_keep_sets(L, n, 64, 65, ps, 0, 0, 0, 1)      # prompt pages exceed the budget


def test_brute_force_tiny():
    """Every keep set of 3 of 6 pages with 1 prompt page: the kept set maximises the sorted
    score vector, the lower page winning ties (exhaustive on tiny inputs)."""
    L, n, K, prot, ps = 1, 24, 12, 3, 4
    kept = oracle.page_keep_sets(L, n, K, prot, ps, seed=9, round_id=1, group_begin=0, group_end=1)[0]
    sc = [np.inf] + [oracle.random_draw(9, 0, 0, 0, 1, b * ps) for b in range(1, 6)]
    best = None
    for c in itertools.combinations(range(1, 6), 2):
        key = (sorted((sc[b] for b in c), reverse=True), [-b for b in c])
        if best is None or key > best[0]:
            best = (key, c)
    assert list(kept) == [0] + list(best[1])


def test_page_table_edit_is_a_permutation_and_matches_the_token_gather():
    rng = np.random.default_rng(1)
    G, P, ps, Kp = 3, 10, 4, 6
    pool = 40
    pt = np.concatenate([rng.permutation(pool)[:G * P].reshape(G, P),
                         np.full((G, 2), 77)], axis=1).astype(np.int32)  # pt_ld = P + 2
    kept = np.stack([np.sort(rng.choice(P, Kp, replace=False)) for _ in range(G)]).astype(np.int32)
    new, freed = oracle.page_table_edit(pt, kept, P)
    for g in range(G):
        assert sorted(list(new[g, :Kp]) + freed[g]) == sorted(pt[g, :P])  # ids conserved
        assert np.all(new[g, Kp:P] == -1) and np.all(new[g, P:] == 77)
    # reading a paged store through the new table equals the gather of the expanded token list
    H, D = 2, 8
    store = rng.integers(0, 1 << 16, (pool, ps, H, D), dtype=np.uint16)
    for g in range(G):
        tokens = (kept[g][:, None] * ps + np.arange(ps)).reshape(-1)      # kept token slots
        before = np.stack([store[pt[g, t // ps], t % ps] for t in tokens])
        after = np.stack([store[new[g, j // ps], j % ps] for j in range(Kp * ps)])
        assert np.array_equal(before, after)
