"""Repeated eviction rounds with the oracle: the survival law.

Random Attention blog summary (survival paragraph): survivors are redrawn at
every eviction, so an old entry survives n rounds with probability about
0.94^n at K=1024, r=64 -- exactly (K/(K+r))^n when no prompt is pinned, since
each round keeps a uniform K-subset of K+r entries.  With a pinned prompt of
prot entries a non-prompt entry survives a round with q = (K-prot)/(K+r-prot).
The applied-round counter (blog summary, benchmark-fixes paragraph) must equal
the number of rounds run.
"""

import math

import numpy as np
import pytest

import oracle


def run_rounds(lists, K, r, prot, rounds, seed):
    """Track original token ids through rounds; returns survival fraction after each round."""
    n = K + r
    # slot -> original token id; tokens >= n arrive later
    ids = np.tile(np.arange(n, dtype=np.int64), (lists, 1))
    next_id = n
    tracked = np.arange(prot, n)  # initial non-prompt entries
    surv = []
    applied = 0
    for rnd in range(rounds):
        s = oracle.score_random(1, 1, n, prot, seed, rnd, False, 0, lists)
        # each row is drawn from list (request=row) -- independent per row
        kept = oracle.select_topk(s, K, prot)
        applied += 1
        ids = np.take_along_axis(ids, kept.astype(np.int64), axis=1)
        new = np.arange(next_id, next_id + r, dtype=np.int64)
        next_id += r
        ids = np.concatenate([ids, np.tile(new, (lists, 1))], axis=1)
        alive = np.isin(ids, tracked).sum() / (lists * len(tracked))
        surv.append(alive)
        assert np.all(ids[:, :prot] == np.arange(prot))  # prompt survival 1.000
    return np.array(surv), applied


@pytest.mark.parametrize("prot", [0, 300])
def test_survival_law(prot):
    K, r, rounds, lists = 1024, 64, 12, 96
    surv, applied = run_rounds(lists, K, r, prot, rounds, seed=21)
    assert applied == rounds
    q = (K - prot) / (K + r - prot)
    N = lists * (K + r - prot)
    for t, got in enumerate(surv, start=1):
        expect = q ** t
        sigma = math.sqrt(expect * (1 - expect) / N)
        assert abs(got - expect) < 3 * sigma + 1e-12, (t, got, expect)
    if prot == 0:
        # the page's approximation: 1024/1088 = 0.941..., printed as 0.94
        assert round(K / (K + r), 2) == 0.94


def test_survival_tracker_bookkeeping():
    """The bench's survival tracker carries token ids through kept indices exactly as the
    definition does (checked against a direct replay), on CPU tensors."""
    import types

    import torch

    from kv_cache_eviction_05_amd.configs import LONGGEN
    from kv_cache_eviction_05_amd.rounds import SurvivalTracker

    cfg = LONGGEN.small(R=1, L=2, H=4, K=40, r=8, prot=5)
    n = cfg.K + cfg.r
    st = types.SimpleNamespace(cfg=cfg, device=torch.device("cpu"), n=n, kept=None)
    tr = SurvivalTracker(st, stride=3)
    ids = np.tile(np.arange(n, dtype=np.int64), (cfg.lists, 1))
    next_id = n
    for rnd in range(6):
        s = oracle.score_random(cfg.L, cfg.H, n, cfg.prot, 11, rnd, False, 0, cfg.lists)
        kept = oracle.select_topk(s, cfg.K, cfg.prot)
        st.kept = torch.from_numpy(kept)
        tr.after_round(st)
        ids = np.concatenate([np.take_along_axis(ids, kept.astype(np.int64), axis=1),
                              np.tile(np.arange(next_id, next_id + cfg.r), (cfg.lists, 1))], axis=1)
        next_id += cfg.r
        assert np.array_equal(tr.ids.numpy(), ids[::3])
        alive = np.isin(ids[::3, :cfg.K], np.arange(cfg.prot, n)).sum() / (len(ids[::3]) * (n - cfg.prot))
        assert abs(tr.curve[-1] - alive) < 1e-12
    rep = tr.report(st)
    assert rep["prompt_survival"] == 1.0 and rep["slot_coverage"] == 1.0
    q = (cfg.K - cfg.prot) / (cfg.K + cfg.r - cfg.prot)
    assert rep["law_q_pow_t"][0] == round(q, 6)
