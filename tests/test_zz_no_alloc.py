"""kvevict_select_global_noalloc, the global top-B on the library's static workspace, against
kvevict_select_global with a caller workspace on the same inputs: budget, per-list counts and
kept indices bit for bit, on calls in a row that shrink (the static array keeps what the last
call left; each call must clear what it relies on)."""

import sys

import numpy as np
import pytest
import torch

from kv_cache_eviction_05_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def scores_of(kind, lists, n, prot, seed):
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        s = rng.random((lists, n), dtype=np.float32)
    elif kind == "ties":
        s = (rng.integers(0, 7, (lists, n)) / 7.0).astype(np.float32)
    else:
        s = rng.standard_normal((lists, n)).astype(np.float32)
    s[:, :prot] = np.inf
    return s


def both(s, prot, p):
    lists, n = s.shape
    ld, kept_ld = n + 3, n + 1
    pad = np.full((lists, ld), 7.0, np.float32)
    pad[:, :n] = s
    scores = torch.from_numpy(pad).to(DEV)
    out = []
    for variant in ("workspace", "noalloc"):
        kept = torch.full((lists, kept_ld), -3, dtype=torch.int32, device=DEV)
        counts = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
        if variant == "workspace":
            wsb = B.kvevict_select_global_workspace(lists, n, prot, ld=ld, kept_ld=kept_ld, p=p)
            ws = torch.full((max(wsb, 256),), 0x5A, dtype=torch.uint8, device=DEV)
            budget = B.kvevict_select_global(kept, kept_ld, counts, scores, ld, lists, n, prot, p,
                                             ws, wsb)
        else:
            budget = B.kvevict_select_global_noalloc(kept, kept_ld, counts, scores, ld, lists, n,
                                                     prot, p)
        torch.cuda.synchronize()
        out.append((budget, counts.cpu().numpy(), kept.cpu().numpy()))
    return out


@pytest.mark.parametrize("calls", [
    # the three-level flow (512 items), then the two-level flow (256), then a small call
    [(64, 65536, 256, 0.25, "uniform"), (64, 32768, 256, 0.25, "normal"),
     (5, 9000, 100, 0.3, "ties")],
    # ties split at the threshold, then a call with nothing to choose, then keep-all
    [(128, 32768, 256, 0.25, "ties"), (3, 100, 100, 0.5, "uniform"), (4, 5000, 10, 1.0, "normal")],
])
def test_noalloc_matches_workspace_call(calls):
    for i, (lists, n, prot, p, kind) in enumerate(calls):
        say(f"select_global_noalloc call {i}: lists={lists} n={n} prot={prot} p={p} kind={kind}")
        s = scores_of(kind, lists, n, prot, seed=lists * n + i)
        (b1, c1, k1), (b2, c2, k2) = both(s, prot, p)
        assert b1 == b2
        assert np.array_equal(c1, c2)
        assert np.array_equal(k1, k2)  # indices up to each count, -3 (untouched) beyond
        assert int(c1.sum()) == lists * prot + b1


def test_noalloc_random_sequence():
    """Twelve calls in a row of random sizes (1 to 96 lists, up to 70,000 candidates, both the
    two-level and the three-level flow, ties and special values), each equal to the workspace
    call: whatever the previous call left in the static array, the next one clears what it
    relies on."""
    rng = np.random.default_rng(2024)
    for i in range(12):
        lists = int(rng.integers(1, 97))
        n = int(rng.integers(1, max(2, min(70000, 4_000_000 // lists))))
        prot = int(rng.integers(0, min(n, 400) + 1))
        p = float(rng.choice([0.0, 0.1, 0.25, 0.5, 0.9, 1.0]))
        kind = str(rng.choice(["uniform", "ties", "normal"]))
        say(f"select_global_noalloc random call {i}: lists={lists} n={n} prot={prot} p={p} "
            f"kind={kind}")
        s = scores_of(kind, lists, n, prot, seed=3000 + i)
        (b1, c1, k1), (b2, c2, k2) = both(s, prot, p)
        assert b1 == b2, i
        assert np.array_equal(c1, c2), i
        assert np.array_equal(k1, k2), i


def test_noalloc_rejects_more_than_the_array_holds():
    """A call whose workspace would exceed the static array returns KVEVICT_ERR_WORKSPACE and
    leaves its outputs untouched."""
    lists, n, prot = 65600, 100, 10
    kept = torch.full((lists, n), -3, dtype=torch.int32, device=DEV)
    counts = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
    scores = torch.zeros((lists, n), dtype=torch.float32, device=DEV)
    with pytest.raises(B.KvevictError) as e:
        B.kvevict_select_global_noalloc(kept, n, counts, scores, n, lists, n, prot, 0.3)
    assert e.value.status == B.KVEVICT_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((kept == -3).all()) and bool((counts == -1).all())


def test_noalloc_replays_from_a_graph():
    """The call recorded in a HIP graph (the use it is for) and replayed three times, each
    replay after the outputs were cleared and after an eager call on other inputs had left the
    static array dirty: every replay equals the eager result bit for bit."""
    lists, n, prot, p = 64, 32768, 256, 0.25
    s = scores_of("normal", lists, n, prot, seed=91)
    scores = torch.from_numpy(s).to(DEV)
    other = torch.from_numpy(scores_of("ties", 5, 9000, 100, seed=92)).to(DEV)
    o_kept = torch.empty((5, 9000), dtype=torch.int32, device=DEV)
    o_counts = torch.empty((5,), dtype=torch.int32, device=DEV)
    say("select_global_noalloc graph: eager reference")
    kept_e = torch.full((lists, n), -3, dtype=torch.int32, device=DEV)
    counts_e = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
    budget = B.kvevict_select_global_noalloc(kept_e, n, counts_e, scores, n, lists, n, prot, p)
    torch.cuda.synchronize()
    kept = torch.full((lists, n), -3, dtype=torch.int32, device=DEV)
    counts = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
    say("select_global_noalloc graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b = B.kvevict_select_global_noalloc(kept, n, counts, scores, n, lists, n, prot, p)
    assert b == budget
    for rep in range(3):
        say(f"select_global_noalloc graph: replay {rep}")
        kept.fill_(-3)
        counts.fill_(-1)
        B.kvevict_select_global_noalloc(o_kept, 9000, o_counts, other, 9000, 5, 9000, 100, 0.3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(counts, counts_e), rep
        assert torch.equal(kept, kept_e), rep
    assert int(counts_e.sum()) == lists * prot + budget
