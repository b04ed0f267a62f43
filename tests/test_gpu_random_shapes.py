"""GPU parity on seeded random shapes: the selects, the gathers and the one-launch round.

Each case draws its shape from a seeded generator (list counts, lengths, prompt
lengths, budgets, head widths, layouts, score distributions), runs the HIP
library through the C ABI and compares with the CPU oracle on the same inputs:
bit-exact for kept indices, counts and moved bytes.  The fixed-shape tests pin
the boundaries one by one; these sweep the combinations between them.
"""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_eviction_05_amd import binding as B
from test_gpu_parity import (bf16_from_bits, check_inplace, make_scores, make_store, rand_bits,
                             say, to_np, u16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
KINDS = ["uniform", "ties", "normal", "special"]


def case_rng(case, salt):
    return np.random.default_rng(7919 * case + salt)


def draw_prot_k(rng, n):
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.8 else 0
    return prot, int(rng.integers(prot, n + 1))


@pytest.mark.parametrize("case", range(12))
def test_random_select_topk(case):
    rng = case_rng(case, 1)
    long = case >= 9  # past 15,360 candidates: 1024-thread workgroups, LDS or global keys
    n = int(rng.integers(15400, 60000)) if long else int(rng.integers(1, 3000))
    lists = int(rng.integers(1, 4)) if long else int(rng.integers(1, 40))
    prot, K = draw_prot_k(rng, n)
    kind = str(rng.choice(KINDS))
    say(f"random select_topk case={case} lists={lists} n={n} K={K} prot={prot} kind={kind}")
    s = make_scores(kind, lists, n, seed=case)
    kept = torch.full((lists, K + 1), -7, dtype=torch.int32, device=DEV)
    B.kvevict_select_topk(kept, K + 1, torch.from_numpy(s).to(DEV), n, lists, n, K, prot)
    torch.cuda.synchronize()
    got = to_np(kept)
    assert np.array_equal(got[:, :K], oracle.select_topk(s, K, prot))
    assert np.all(got[:, K:] == -7)


@pytest.mark.parametrize("case", range(10))
def test_random_select_random(case):
    rng = case_rng(case, 2)
    R, L, H = (int(x) for x in rng.integers(1, 4, 3))
    n = int(rng.integers(1, 4000)) if case < 8 else int(rng.integers(15400, 30000))
    prot, K = draw_prot_k(rng, n)
    shared = bool(rng.random() < 0.3)
    seed, rnd = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**31))
    lists = R * L * (1 if shared else H)
    say(f"random select_random case={case} R={R} L={L} H={H} n={n} K={K} prot={prot} "
        f"shared={shared}")
    want = oracle.select_topk(oracle.score_random(L, H, n, prot, seed, rnd, shared, 0, lists), K,
                              prot)
    got = torch.full((lists, K + 2), -9, dtype=torch.int32, device=DEV)
    B.kvevict_select_random(got, K + 2, R, L, H, n, K, prot, seed, rnd, shared)
    torch.cuda.synchronize()
    g = to_np(got)
    assert np.array_equal(g[:, :K], want)
    assert np.all(g[:, K:] == -9)


@pytest.mark.parametrize("case", range(10))
def test_random_select_global(case):
    rng = case_rng(case, 3)
    lists = int(rng.integers(1, 30))
    n = int(rng.integers(1, max(2, 300000 // lists)))
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.8 else 0
    p = float(np.round(rng.random(), 3))
    kind = str(rng.choice(KINDS + ["constant"]))
    say(f"random select_global case={case} lists={lists} n={n} prot={prot} p={p} kind={kind}")
    s = make_scores(kind, lists, n, seed=100 + case)
    kept = torch.full((lists, n + 1), -3, dtype=torch.int32, device=DEV)
    counts = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
    wsb = B.kvevict_select_global_workspace(lists, n, prot, p=p)
    ws = torch.full((max(wsb, 256),), 0x5A, dtype=torch.uint8, device=DEV)
    budget = B.kvevict_select_global(kept, n + 1, counts, torch.from_numpy(s).to(DEV), n, lists, n,
                                     prot, p, ws, wsb)
    torch.cuda.synchronize()
    want_kept, want_counts, want_B = oracle.select_global(s, prot, p)
    assert budget == want_B
    got_counts, got = to_np(counts), to_np(kept)
    assert np.array_equal(got_counts, want_counts)
    for l in range(lists):
        c = want_counts[l]
        assert np.array_equal(got[l, :c], want_kept[l, :c]), l
        assert np.all(got[l, c:] == -3), l


@pytest.mark.parametrize("case", range(12))
def test_random_compact(case):
    rng = case_rng(case, 4)
    ps = 16
    groups, H = int(rng.integers(1, 7)), int(rng.integers(1, 9))
    D = int(rng.choice([8, 16, 24, 40, 64, 128, 256]))
    n = int(rng.integers(1, 700))
    prot, K = draw_prot_k(rng, n)
    K = max(K, 1)
    src_paged, dst_paged = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    shared = bool(rng.random() < 0.3)
    variable = bool(rng.random() < 0.4)
    ipg = 1 if shared else H
    idx_lists = groups * ipg
    say(f"random compact case={case} groups={groups} H={H} D={D} n={n} K={K} prot={min(prot, K)} "
        f"src_paged={src_paged} dst_paged={dst_paged} shared={shared} variable={variable}")
    kept = oracle.select_topk(rng.random((idx_lists, n), dtype=np.float32), K, min(prot, K))
    counts = rng.integers(0, K + 1, idx_lists).astype(np.int32) if variable else None

    def store(paged, rows, seed):
        if paged:
            pages = -(-rows // ps)
            pool = groups * pages + int(rng.integers(0, 5))
            pt = rng.permutation(pool)[:groups * pages].reshape(groups, pages).astype(np.int32)
            bits = rand_bits((pool, ps, H, D), seed)
            desc = B.paged_desc(D, H, ps, pool, torch.from_numpy(pt).to(DEV))
            return bits, desc, {"paged": True, "page_table": pt}
        bits = rand_bits((groups * H, rows, D), seed)
        return bits, B.contig_desc(D, H, rows), {"list_stride": rows * D}

    ks, sdesc, so = store(src_paged, n, 30 + case)
    vs = rand_bits(ks.shape, 31 + case)
    kd0, ddesc, do = store(dst_paged, K, 32 + case)
    vd0 = rand_bits(kd0.shape, 33 + case)
    k_dst, v_dst = bf16_from_bits(kd0), bf16_from_bits(vd0)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.kvevict_compact(sdesc, bf16_from_bits(ks), bf16_from_bits(vs), ddesc, k_dst, v_dst,
                      torch.from_numpy(kept).to(DEV), K,
                      torch.from_numpy(counts).to(DEV) if variable else None, K, groups, ipg, err)
    torch.cuda.synchronize()
    kd, vd = kd0.copy(), vd0.copy()
    oracle.compact(so, ks, vs, do, kd, vd, kept, K, D, H, 0, groups, ipg=ipg, kept_count=counts,
                   page_size=ps)
    assert np.array_equal(u16(k_dst), kd) and np.array_equal(u16(v_dst), vd)
    assert int(err.item()) == 0


@pytest.mark.parametrize("case", range(10))
def test_random_evict_random_inplace(case):
    rng = case_rng(case, 5)
    ps = 16
    layout = "paged" if rng.random() < 0.5 else "contig"
    R, L, H = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 6))
    D = int(rng.choice([8, 24, 64, 128, 256]))
    n = int(rng.integers(1, 1500))
    prot, K = draw_prot_k(rng, n)
    shared = bool(rng.random() < 0.3)
    seed, rnd = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**31))
    groups = R * L
    ipg = 1 if shared else H
    lists = groups * ipg
    say(f"random evict_random_inplace case={case} {layout} R={R} L={L} H={H} D={D} n={n} K={K} "
        f"prot={prot} shared={shared}")
    kept = np.ascontiguousarray(oracle.select_topk(
        oracle.score_random(L, H, n, prot, seed, rnd, shared, 0, lists), K, prot))
    desc, pt, ks, vs, k, v = make_store(layout, groups, H, D, n, ps, seed=50 + case)
    freed = torch.full((groups * (n // ps + 1) + 1,), -5, dtype=torch.int32, device=DEV)
    fcount = torch.zeros(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = torch.full((lists, K + 1), -9, dtype=torch.int32, device=DEV)
    B.kvevict_evict_random_inplace(desc, k, v, R, L, n, K, prot, seed, rnd, shared, got, K + 1,
                                   freed, fcount, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    g = to_np(got)
    assert np.array_equal(g[:, :K], kept)
    assert np.all(g[:, K:] == -9)
    check_inplace(layout, ks, vs, k, v, kept, None, groups, H, ipg, pt, ps, n, K, D, freed, fcount)
