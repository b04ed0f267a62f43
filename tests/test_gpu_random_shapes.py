"""GPU parity on seeded random shapes: scorers, selects, gathers and the fused rounds.

Each case draws its shape from a seeded generator (list counts, lengths, prompt
lengths, budgets, head widths, layouts, score distributions), runs the HIP
library through the C ABI and compares with the CPU oracle on the same inputs:
bit-exact for random scores, kept indices, counts, page tables and moved bytes;
within a relative 1e-5 (weighted) or the stated precision (KeyDiff: the fp32
rounding of the oracle's binary64 cosine, or its neighbour next to a midpoint)
for the binary64 scorers.  The fixed-shape tests pin
the boundaries one by one; these sweep the combinations between them.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from kv_cache_eviction_05_amd import binding as B
from kv_cache_eviction_05_amd.configs import gdn_windows
from test_gpu_parity import test_score_select_global as fused_score_select_check
from test_gpu_parity import (assert_keydiff_close, assert_weighted_close, bf16_from_bits,
                             check_inplace, keep_sets, make_scores, make_store, rand_bits,
                             rand_keys, say, to_np, u16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
KINDS = ["uniform", "ties", "normal", "special"]


# KVEVICT_RANDOM_SCALE=k runs k times as many seeded cases of every test below (the
# first ones are the default cases).
SCALE = max(1, int(os.environ.get("KVEVICT_RANDOM_SCALE", "1")))


def cases(n):
    return range(n * SCALE)


def case_rng(case, salt):
    return np.random.default_rng(7919 * case + salt)


def draw_prot_k(rng, n):
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.8 else 0
    return prot, int(rng.integers(prot, n + 1))


@pytest.mark.parametrize("case", cases(12))
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


@pytest.mark.parametrize("case", cases(10))
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


@pytest.mark.parametrize("case", cases(10))
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


@pytest.mark.parametrize("case", cases(4))
def test_random_select_global_many_items(case):
    """Calls of 16 to 768 items (runs of up to 8,192 candidates): the two-level flow up to 256
    items and the three-level one above, on random lengths, prompts, fractions and scores."""
    rng = case_rng(case, 13)
    lists = int(rng.integers(8, 65))
    n = int(rng.integers(2 * 8192, 12 * 8192))
    prot = int(rng.integers(0, 300))
    p = float(rng.choice([0.05, 0.25, 0.5, 0.9]))
    kind = KINDS[case % len(KINDS)]
    say(f"random select_global many items case={case} lists={lists} n={n} prot={prot} p={p} "
        f"kind={kind}")
    s = make_scores(kind, lists, n, seed=900 + case)
    kept = torch.full((lists, n), -3, dtype=torch.int32, device=DEV)
    counts = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
    wsb = B.kvevict_select_global_workspace(lists, n, prot, p=p)
    ws = torch.full((max(wsb, 256),), 0x5A, dtype=torch.uint8, device=DEV)
    budget = B.kvevict_select_global(kept, n, counts, torch.from_numpy(s).to(DEV), n, lists, n,
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


@pytest.mark.parametrize("case", cases(6))
def test_random_score_select_global(case):
    """The fused weighted score + global top-B on random model shapes: bit for bit the two
    calls it replaces, and the oracle's top-B of those scores."""
    rng = case_rng(case, 16)
    L = int(rng.integers(1, 21))
    G = 3 * L
    H = int(rng.integers(1, 7))
    Hg = int(rng.choice([4, 8, 16, 48, 70]))
    n = int(rng.integers(1, max(2, min(40000, 8_000_000 // (G * Hg)))))
    prot = int(rng.integers(0, min(n, 300) + 1))
    width = int(rng.choice([4, 6]))
    p = float(np.round(rng.random(), 3))
    fused_score_select_check(G, L, H, Hg, n, prot, width, p)


@pytest.mark.parametrize("case", cases(12))
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


@pytest.mark.parametrize("case", cases(8))
def test_random_compact_ordered(case):
    """kvevict_compact_ordered against kvevict_compact (bit for bit, error count included) and
    the oracle: paged destinations of 16-token pages whose rows hold 1024 elements (the
    physical-order walk) or not (its fallback), pools from one to five times the pages written,
    per-head or shared lists, per-list counts, now and then a page id outside the pool."""
    rng = case_rng(case, 14)
    ps = 16
    H, D = [(8, 128), (4, 256), (16, 64), (2, 512), (8, 64), (3, 40)][int(rng.integers(0, 6))]
    groups = int(rng.integers(1, 13))
    n = int(rng.integers(1, 2200))
    prot, K = draw_prot_k(rng, n)
    K = max(K, 1)
    src_paged = bool(rng.random() < 0.7)
    shared = bool(rng.random() < 0.3)
    variable = bool(rng.random() < 0.4)
    bad_page = bool(rng.random() < 0.15)
    slack = float(rng.choice([1.0, 1.5, 2.0, 3.0, 5.0]))
    ipg = 1 if shared else H
    idx_lists = groups * ipg
    say(f"random compact_ordered case={case} groups={groups} H={H} D={D} n={n} K={K} "
        f"prot={min(prot, K)} src_paged={src_paged} shared={shared} variable={variable} "
        f"slack={slack} bad_page={bad_page}")
    kept = oracle.select_topk(rng.random((idx_lists, n), dtype=np.float32), K, min(prot, K))
    counts = rng.integers(0, K + 1, idx_lists).astype(np.int32) if variable else None
    if src_paged:
        sp = -(-n // ps)
        pool_s = groups * sp + int(rng.integers(0, 5))
        pt_s = rng.permutation(pool_s)[:groups * sp].reshape(groups, sp).astype(np.int32)
        ks = rand_bits((pool_s, ps, H, D), 60 + case)
        sdesc = B.paged_desc(D, H, ps, pool_s, torch.from_numpy(pt_s).to(DEV))
        so = {"paged": True, "page_table": pt_s}
    else:
        ks = rand_bits((groups * H, n, D), 60 + case)
        sdesc, so = B.contig_desc(D, H, n), {"list_stride": n * D}
    vs = rand_bits(ks.shape, 61 + case)
    dp = -(-K // ps)
    pool_d = int(groups * dp * slack) + int(rng.integers(0, 3))
    pt_d = rng.permutation(pool_d)[:groups * dp].reshape(groups, dp).astype(np.int32)
    if bad_page:
        pt_d[int(rng.integers(0, groups)), int(rng.integers(0, dp))] = pool_d + 1
    kd0 = rand_bits((pool_d, ps, H, D), 62 + case)
    vd0 = rand_bits(kd0.shape, 63 + case)
    ddesc = B.paged_desc(D, H, ps, pool_d, torch.from_numpy(pt_d).to(DEV))
    kept_t = torch.from_numpy(kept).to(DEV)
    count_t = torch.from_numpy(counts).to(DEV) if variable else None
    wsb = B.kvevict_compact_ordered_workspace(ddesc)
    ws = torch.full((max(wsb, 256),), 0x7E, dtype=torch.uint8, device=DEV)
    outs = []
    for ordered in (False, True):
        k_dst, v_dst = bf16_from_bits(kd0), bf16_from_bits(vd0)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        args = (sdesc, bf16_from_bits(ks), bf16_from_bits(vs), ddesc, k_dst, v_dst, kept_t, K,
                count_t, K, groups, ipg)
        if ordered:
            B.kvevict_compact_ordered(*args, ws, wsb, err)
        else:
            B.kvevict_compact(*args, err)
        torch.cuda.synchronize()
        outs.append((u16(k_dst), u16(v_dst), int(err.item())))
    assert np.array_equal(outs[1][0], outs[0][0]) and np.array_equal(outs[1][1], outs[0][1])
    assert outs[1][2] == outs[0][2]
    if bad_page:
        return
    assert outs[0][2] == 0
    kd, vd = kd0.copy(), vd0.copy()
    oracle.compact(so, ks, vs, {"paged": True, "page_table": pt_d}, kd, vd, kept, K, D, H, 0,
                   groups, ipg=ipg, kept_count=counts, page_size=ps)
    assert np.array_equal(outs[1][0], kd) and np.array_equal(outs[1][1], vd)


@pytest.mark.parametrize("case", cases(10))
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


@pytest.mark.parametrize("case", cases(8))
def test_random_score_random(case):
    rng = case_rng(case, 6)
    R, L, H = (int(x) for x in rng.integers(1, 5, 3))
    n = int(rng.integers(1, 5000))
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.8 else 0
    shared, pad = bool(rng.random() < 0.3), int(rng.integers(0, 9))
    seed, rnd = int(rng.integers(0, 2**64, dtype=np.uint64)), int(rng.integers(0, 2**32))
    lists = R * L * (1 if shared else H)
    say(f"random score_random case={case} R={R} L={L} H={H} n={n} prot={prot} shared={shared}")
    s = torch.full((lists, n + pad), float("nan"), dtype=torch.float32, device=DEV)
    B.kvevict_score_random(s, n + pad, R, L, H, n, prot, seed, rnd, shared)
    torch.cuda.synchronize()
    got = to_np(s)
    assert np.array_equal(got[:, :n], oracle.score_random(L, H, n, prot, seed, rnd, shared, 0, lists))
    assert np.all(np.isnan(got[:, n:]))


@pytest.mark.parametrize("case", cases(8))
def test_random_score_weighted(case):
    rng = case_rng(case, 7)
    L = int(rng.integers(1, 24))
    G = L * int(rng.integers(1, 5))
    H, Hg = int(rng.integers(1, 7)), int(rng.integers(1, 100))
    width = int(rng.integers(1, 8))
    n = int(rng.integers(1, 700))
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.7 else 0
    say(f"random score_weighted case={case} G={G} L={L} H={H} Hg={Hg} width={width} n={n} "
        f"prot={prot}")
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((G, n, Hg))))).astype(np.float32)
    vnorm = np.exp(rng.standard_normal((G, n, Hg))).astype(np.float32)
    w = rng.standard_normal((L, H, width, Hg)).astype(np.float32)
    begins, counts = gdn_windows(L, G, width)
    s = torch.full((L * H, n + 1), float("nan"), dtype=torch.float32, device=DEV)
    B.kvevict_score_weighted(s, n + 1, torch.from_numpy(beta).to(DEV),
                             torch.from_numpy(vnorm).to(DEV), n * Hg, Hg, 1,
                             torch.from_numpy(w).to(DEV), width, begins, counts, L, H, G, Hg, n,
                             prot)
    torch.cuda.synchronize()
    got = to_np(s)
    assert np.all(np.isnan(got[:, n:]))
    want = oracle.score_weighted(beta, vnorm, w, *oracle.gdn_windows(L, G, width), prot)
    assert_weighted_close(got[:, :n], want, prot)


@pytest.mark.parametrize("case", cases(8))
def test_random_score_keydiff(case):
    rng = case_rng(case, 8)
    groups, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    D = int(rng.choice([8, 16, 32, 64, 128, 256, 512]))
    n = int(rng.integers(1, 3000))
    cap = n + int(rng.integers(0, 20))
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.7 else 0
    lists = groups * H
    say(f"random score_keydiff case={case} groups={groups} H={H} D={D} n={n} cap={cap} prot={prot}")
    keys = rand_keys((lists, cap, D), seed=700 + case)
    s = torch.full((lists, n + 1), float("nan"), dtype=torch.float32, device=DEV)
    B.kvevict_score_keydiff(s, n + 1, B.contig_desc(D, H, cap), bf16_from_bits(keys), groups, n,
                            prot)
    torch.cuda.synchronize()
    got = to_np(s)
    assert np.all(np.isnan(got[:, n:]))
    assert_keydiff_close(got[:, :n], keys[:, :n], prot)


@pytest.mark.parametrize("case", cases(6))
def test_random_score_keydiff_whole_list(case):
    """D = 128 and at most 1088 keys in a contiguous store: the kernel that holds the whole
    list on chip, on random lengths (steps of 16 rows, whole, partial or skipped), padded
    stores and prompts."""
    rng = case_rng(case, 15)
    groups, H = int(rng.integers(1, 5)), int(rng.integers(1, 9))
    n = int(rng.integers(1, 1089))
    cap = n + int(rng.integers(0, 40))
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.6 else 0
    lists = groups * H
    say(f"random score_keydiff whole list case={case} groups={groups} H={H} n={n} cap={cap} "
        f"prot={prot}")
    keys = rand_keys((lists, cap, 128), seed=800 + case)
    s = torch.full((lists, n + 1), float("nan"), dtype=torch.float32, device=DEV)
    B.kvevict_score_keydiff(s, n + 1, B.contig_desc(128, H, cap), bf16_from_bits(keys), groups,
                            n, prot)
    torch.cuda.synchronize()
    got = to_np(s)
    assert np.all(np.isnan(got[:, n:]))
    assert_keydiff_close(got[:, :n], keys[:, :n], prot)


@pytest.mark.parametrize("case", cases(8))
def test_random_select_topk_layers(case):
    rng = case_rng(case, 9)
    R, L, H = int(rng.integers(1, 4)), int(rng.integers(1, 17)), int(rng.integers(1, 5))
    n = int(rng.integers(1, 3000)) if case < 6 else int(rng.integers(15400, 30000))
    prot = int(rng.integers(0, n + 1)) if rng.random() < 0.7 else 0
    kind = str(rng.choice(KINDS))
    lists = R * L * H
    budget = [int(x) for x in rng.integers(0, n - prot + 1, L)]
    say(f"random select_topk_layers case={case} R={R} L={L} H={H} n={n} prot={prot} kind={kind}")
    s = make_scores(kind, lists, n, seed=900 + case)
    kept = torch.full((lists, n + 1), -3, dtype=torch.int32, device=DEV)
    counts = torch.full((lists,), -1, dtype=torch.int32, device=DEV)
    B.kvevict_select_topk_layers(kept, n + 1, counts, torch.from_numpy(s).to(DEV), n, R * L, L, H,
                                 n, prot, budget)
    torch.cuda.synchronize()
    got, got_c = to_np(kept), to_np(counts)
    for lst in range(lists):
        K = prot + budget[(lst // H) % L]
        assert got_c[lst] == K
        assert np.array_equal(got[lst, :K], oracle.select_topk(s[lst:lst + 1], K, prot)[0]), lst
        assert np.all(got[lst, K:] == -3)


@pytest.mark.parametrize("case", cases(6))
def test_random_reduce_max_heads(case):
    rng = case_rng(case, 10)
    G, H, n = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 5000))
    pad = int(rng.integers(0, 5))
    say(f"random reduce_max_heads case={case} G={G} H={H} n={n}")
    s = make_scores(str(rng.choice(KINDS)), G * H, n, seed=1100 + case)
    s_pad = np.full((G * H, n + pad), 3.0, np.float32)
    s_pad[:, :n] = s
    out = torch.full((G, n + 1), 5.0, dtype=torch.float32, device=DEV)
    B.kvevict_reduce_max_heads(out, n + 1, torch.from_numpy(s_pad).to(DEV), n + pad, G, H, n)
    torch.cuda.synchronize()
    got = to_np(out)
    assert np.array_equal(got[:, :n].view(np.uint32), oracle.shared_max_scores(s, H).view(np.uint32))
    assert np.all(got[:, n:] == 5.0)


@pytest.mark.parametrize("case", cases(10))
def test_random_compact_inplace(case):
    rng = case_rng(case, 11)
    ps = 16
    layout = "paged" if rng.random() < 0.5 else "contig"
    groups, H = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    D = int(rng.choice([8, 24, 40, 64, 128, 256]))
    n = int(rng.integers(1, 1200))
    prot, K = draw_prot_k(rng, n)
    shared, variable = bool(rng.random() < 0.3), bool(rng.random() < 0.5)
    ipg = 1 if shared else H
    say(f"random compact_inplace case={case} {layout} groups={groups} H={H} D={D} n={n} K={K} "
        f"prot={prot} shared={shared} variable={variable}")
    kept, counts = keep_sets(groups * ipg, n, K, prot, seed=1200 + case, variable=variable)
    desc, pt, ks, vs, k, v = make_store(layout, groups, H, D, n, ps, seed=60 + case)
    freed = torch.full((groups * (n // ps + 1) + 1,), -5, dtype=torch.int32, device=DEV)
    fcount = torch.zeros(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.kvevict_compact_inplace(desc, k, v, torch.from_numpy(kept).to(DEV), K,
                              torch.from_numpy(counts).to(DEV) if variable else None, K, n,
                              groups, ipg, freed, fcount, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_inplace(layout, ks, vs, k, v, kept, counts if variable else None, groups, H, ipg, pt, ps,
                  n, K, D, freed, fcount)


@pytest.mark.parametrize("case", cases(8))
def test_random_evict_pages_random(case):
    rng = case_rng(case, 12)
    ps = int(rng.choice([1, 2, 4, 8, 16, 32]))
    R, L = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    P = int(rng.integers(1, min(300, 4000 // ps) + 1))
    n = P * ps
    Kp = int(rng.integers(0, P + 1))
    K = Kp * ps
    prot = int(rng.integers(0, K + 1)) if rng.random() < 0.7 else 0
    seed, rnd = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**31))
    groups = R * L
    say(f"random evict_pages_random case={case} R={R} L={L} ps={ps} n={n} K={K} prot={prot}")
    pt_ld = P + int(rng.integers(0, 4))
    pool = groups * P + 5
    pt = np.full((groups, pt_ld), 99, dtype=np.int32)
    pt[:, :P] = rng.permutation(pool)[: groups * P].reshape(groups, P)
    want_kept = oracle.page_keep_sets(L, n, K, prot, ps, seed, rnd, 0, groups)
    want_pt, want_freed = oracle.page_table_edit(pt, want_kept, P)
    dpt = torch.from_numpy(pt).to(DEV)
    kept = torch.full((groups, Kp + 1), -9, dtype=torch.int32, device=DEV)
    freed = torch.full((groups * (P - Kp) + 1,), -5, dtype=torch.int32, device=DEV)
    fcount = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.kvevict_evict_pages_random(dpt, pt_ld, ps, R, L, n, K, prot, seed, rnd, kept, Kp + 1, freed,
                                 fcount)
    torch.cuda.synchronize()
    got = to_np(kept)
    assert np.array_equal(got[:, :Kp], want_kept)
    assert np.all(got[:, Kp:] == -9)
    assert np.array_equal(to_np(dpt), want_pt)
    nf = int(fcount.item())
    assert nf == groups * (P - Kp)
    got_freed = to_np(freed)[:nf]
    assert sorted(got_freed.tolist()) == sorted(x for f in want_freed for x in f)
