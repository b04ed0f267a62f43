"""The five workloads at their real sizes, in the launch configuration the
benchmark times, checked against the oracle.

Keep sets are compared with the oracle's on every list: the oracle draws the
scores and sorts each list itself, spread over the host's cores (its C calls
release the interpreter lock).  Compacted K/V are compared on every list with
a torch gather (contiguous) or page walk (paged) of the source through the
oracle's kept indices, and on sampled lists with the oracle's own row copies.
Weighted scores are compared with the oracle's at every position.
"""

import gc
import math
import os
import sys
import types
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from kv_cache_eviction_05_amd import binding as B
from kv_cache_eviction_05_amd import configs, rounds, synth
from test_gpu_parity import assert_keydiff_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_kept_properties(kept, K, prot, n):
    """Strictly increasing, prompt first, in range -- on every list, on the GPU."""
    assert kept.shape[1] >= K
    k = kept[:, :K]
    if K > 1:
        assert bool((k[:, 1:] > k[:, :-1]).all())
    if prot:
        assert bool((k[:, :prot] == torch.arange(prot, device=k.device, dtype=k.dtype)).all())
    assert int(k.min()) >= 0 and int(k.max()) < n


THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_keep_sets(cfg, round_id, K=None, n=None):
    """The oracle's kept indices int32 [lists][K] of a random top-K round on every list: its
    Philox draw and its stable sort, list ranges spread over the host threads."""
    K = cfg.K if K is None else K
    n = cfg.n if n is None else n
    lists = cfg.lists
    out = np.empty((lists, K), np.int32)
    step = max(64, -(-lists // (4 * THREADS)))

    def part(l0):
        l1 = min(lists, l0 + step)
        sc = oracle.score_random(cfg.L, cfg.H, n, cfg.prot, cfg.seed, round_id, cfg.shared, l0, l1)
        out[l0:l1] = oracle.select_topk(sc, K, cfg.prot)

    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(part, range(0, lists, step)))
    return out


def oracle_select_all(scores, K, prot):
    """The oracle's top-K int32 [lists][K] of the given scores [lists][n], list ranges spread
    over the host threads."""
    lists = scores.shape[0]
    out = np.empty((lists, K), np.int32)
    step = max(64, -(-lists // (4 * THREADS)))

    def part(l0):
        l1 = min(lists, l0 + step)
        out[l0:l1] = oracle.select_topk(np.ascontiguousarray(scores[l0:l1]), K, prot)

    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(part, range(0, lists, step)))
    return out


def assert_keep_sets(got, want, what):
    """Every list's kept indices equal the oracle's; the first differing list is named."""
    g = got.cpu().numpy() if torch.is_tensor(got) else got
    g = g[:, :want.shape[1]]
    if not np.array_equal(g, want):
        bad = np.nonzero(np.any(g != want, axis=1))[0]
        raise AssertionError(f"{what}: {len(bad)} of {len(want)} lists differ, first {bad[0]}")


def check_paged_gather(st, cfg, kept, K, chunk=128):
    """Every group's destination pages against a page walk of the source through `kept`: for
    list (g, h) and j < K, the row of head h at token j of g's destination table equals the
    row of head h at token kept[j] of its source table (one index list per group when the draw
    is shared).  Runs on the GPU over groups in chunks."""
    ps, H, D, groups = cfg.page_size, cfg.H, cfg.D, cfg.groups
    per_head = kept.shape[0] == groups * H
    j = torch.arange(K, device=DEV)
    heads = torch.arange(H, device=DEV)
    for src, dst in ((st.k_src, st.k_dst), (st.v_src, st.v_dst)):
        pool_s = src.view(torch.int16).reshape(-1, H, D)  # token-major rows [pages*ps][H][D]
        pool_d = dst.view(torch.int16).reshape(-1, H, D)
        for g0 in range(0, groups, chunk):
            g1 = min(groups, g0 + chunk)
            gc_ = g1 - g0
            rows = kept[g0 * H:g1 * H] if per_head else kept[g0:g1]
            idx = torch.from_numpy(np.ascontiguousarray(rows[:, :K])).to(DEV).long()
            idx = idx.view(gc_, H if per_head else 1, K)
            spt = st.src_pt[g0:g1].long()
            dpt = st.dst_pt[g0:g1].long()
            src_tok = torch.gather(spt, 1, (idx // ps).reshape(gc_, -1)).view_as(idx) * ps + idx % ps
            dst_tok = dpt[:, j // ps] * ps + j % ps                        # [gc, K]
            if per_head:
                want = pool_s[src_tok, heads[None, :, None]]               # [gc, H, K, D]
                got = pool_d[dst_tok[:, None, :], heads[None, :, None]]
            else:
                want = pool_s[src_tok[:, 0, :]]                            # [gc, K, H, D]
                got = pool_d[dst_tok]
            assert torch.equal(got, want), (g0, g1)
            del want, got


def check_contig_gather(st, K, counts=None, chunk=1024, kept=None):
    """dst[list][j] == src[list][idx[list][j]] for every list (torch gather in chunks), with
    idx the oracle's kept indices `kept` (host) when given, else the round's own."""
    lists = st.k_src.shape[0]
    for l0 in range(0, lists, chunk):
        l1 = min(lists, l0 + chunk)
        if kept is not None:
            idx = torch.from_numpy(np.ascontiguousarray(kept[l0:l1, :K])).to(DEV).long()
        else:
            idx = st.kept[l0:l1, :K].long()
        if counts is not None:
            valid = torch.arange(K, device=DEV)[None, :] < counts[l0:l1, None]
            idx = torch.where(valid, idx, torch.zeros_like(idx))
        for src, dst in ((st.k_src, st.k_dst), (st.v_src, st.v_dst)):
            g = torch.gather(src[l0:l1].view(torch.int16), 1,
                             idx[:, :, None].expand(-1, -1, src.shape[2]))
            d = dst[l0:l1, :K].view(torch.int16)
            if counts is not None:
                eq = (g == d) | ~valid[:, :, None]
                assert bool(eq.all())
            else:
                assert torch.equal(g, d)


def sample_lists(total, k, seed):
    rng = np.random.default_rng(seed)
    base = {0, 1, total - 1, total // 2}
    base.update(int(x) for x in rng.choice(total, size=min(k, total), replace=False))
    return sorted(x for x in base if 0 <= x < total)


def test_tiny_round_full():
    """Tiny workload: every score, index and byte against the oracle."""
    cfg = configs.TINY
    say("tiny round")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st, round_id=0)  # draw + top-K in one launch, then the gather
    rounds.score(st, 0)               # the standalone scorer, for its own parity
    torch.cuda.synchronize()
    want_s = oracle.score_random(cfg.L, cfg.H, cfg.n, cfg.prot, cfg.seed, 0, False, 0, cfg.lists)
    assert np.array_equal(st.scores.cpu().numpy(), want_s)
    want_k = oracle.select_topk(want_s, cfg.K, cfg.prot)
    assert np.array_equal(st.kept.cpu().numpy(), want_k)
    ks, vs = u16(st.k_src), u16(st.v_src)
    kd = np.zeros((cfg.lists, cfg.K, cfg.D), np.uint16)
    vd = np.zeros_like(kd)
    oracle.compact({"list_stride": cfg.n * cfg.D}, ks, vs, {"list_stride": cfg.K * cfg.D}, kd, vd,
                   want_k, cfg.K, cfg.D, cfg.H, 0, cfg.groups, ipg=cfg.H)
    assert np.array_equal(u16(st.k_dst), kd) and np.array_equal(u16(st.v_dst), vd)
    assert int(st.errors.item()) == 0
    # the page's byte accounting: 2 heads x 1024 kept x (K + V) x 256 B, read and written
    assert st.kv_bytes_moved() == 2 * 1024 * 2 * 256 * 2


def test_batch_round_full_and_deterministic():
    """Decode-time batch round (128 x 36 x 8 lists): every list's keep set and compacted rows
    against the oracle's, sampled lists through the oracle's own row copies, determinism."""
    cfg = configs.BATCH
    say("batch round: allocating")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st, round_id=0)
    torch.cuda.synchronize()
    assert int(st.errors.item()) == 0
    say("batch round: the oracle's keep sets of all 36,864 lists")
    want_all = oracle_keep_sets(cfg, 0)
    assert_keep_sets(st.kept, want_all, "batch round")
    say("batch round: every list's rows against a gather through the oracle's indices")
    check_contig_gather(st, cfg.K, kept=want_all)
    del want_all
    say("batch round: sampled lists through the oracle's scorer and row copies")
    rounds.score(st, 0)  # the standalone scorer (the round drew its scores on chip)
    torch.cuda.synchronize()
    for l in sample_lists(cfg.lists, 24, seed=2):
        want_s = oracle.score_random(cfg.L, cfg.H, cfg.n, cfg.prot, cfg.seed, 0, False, l, l + 1)
        assert np.array_equal(st.scores[l:l + 1].cpu().numpy(), want_s), l
        want_k = oracle.select_topk(want_s, cfg.K, cfg.prot)
        assert np.array_equal(st.kept[l:l + 1].cpu().numpy(), want_k), l
        ks, vs = u16(st.k_src[l:l + 1]), u16(st.v_src[l:l + 1])
        kd = np.zeros((1, cfg.K, cfg.D), np.uint16)
        vd = np.zeros_like(kd)
        # one list of a per-head store is a group of one head
        oracle.compact({"list_stride": cfg.n * cfg.D}, ks, vs, {"list_stride": cfg.K * cfg.D}, kd,
                       vd, want_k, cfg.K, cfg.D, 1, 0, 1, ipg=1)
        assert np.array_equal(u16(st.k_dst[l:l + 1]), kd), l
        assert np.array_equal(u16(st.v_dst[l:l + 1]), vd), l
    say("batch round: determinism")
    kept1 = st.kept.clone()
    sum1 = st.k_dst.view(torch.int16).to(torch.int64).sum(dim=(1, 2))
    rounds.run_round(st, round_id=0)
    torch.cuda.synchronize()
    assert torch.equal(kept1, st.kept)
    assert torch.equal(sum1, st.k_dst.view(torch.int16).to(torch.int64).sum(dim=(1, 2)))
    del st, kept1, sum1
    free()


@pytest.mark.parametrize("cfg", [configs.PAGED, configs.PAGED_SHARED, configs.PAGED_SINGLE],
                         ids=["per_head", "shared", "single_request"])
def test_paged_round_full(cfg):
    """Paged round (64 or 1 request(s) x 36 x 8, 16-token pages): every keep set against the
    oracle's, every group's destination pages against a page walk of the source through the
    oracle's indices, sampled groups through the oracle's own page-table copies."""
    say(f"paged round {cfg.name}: allocating")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st, round_id=3)
    torch.cuda.synchronize()
    assert int(st.errors.item()) == 0
    say(f"paged round {cfg.name}: the oracle's keep sets of all {cfg.lists} lists")
    want_all = oracle_keep_sets(cfg, 3)
    assert_keep_sets(st.kept, want_all, cfg.name)
    say(f"paged round {cfg.name}: every group's pages against a walk through the oracle's indices")
    check_paged_gather(st, cfg, want_all, cfg.K)
    del want_all
    ps, H, D = cfg.page_size, cfg.H, cfg.D
    src_pt, dst_pt = st.src_pt.cpu().numpy(), st.dst_pt.cpu().numpy()
    say(f"paged round {cfg.name}: sampled oracle parity")
    rounds.score(st, 3)  # the standalone scorer (the round drew its scores on chip)
    torch.cuda.synchronize()
    for g in sample_lists(cfg.groups, 10, seed=3):
        l0 = g if cfg.shared else g * H
        l1 = l0 + (1 if cfg.shared else H)
        want_s = oracle.score_random(cfg.L, H, cfg.n, cfg.prot, cfg.seed, 3, cfg.shared, l0, l1)
        assert np.array_equal(st.scores[l0:l1].cpu().numpy(), want_s), g
        want_k = oracle.select_topk(want_s, cfg.K, cfg.prot)
        assert np.array_equal(st.kept[l0:l1].cpu().numpy(), want_k), g
        # the group's pages, renumbered into a small host pool
        sp = torch.from_numpy(src_pt[g].astype(np.int64)).to(DEV)
        dp = torch.from_numpy(dst_pt[g].astype(np.int64)).to(DEV)
        ks, vs = u16(st.k_src[sp]), u16(st.v_src[sp])
        pt_s = np.arange(len(src_pt[g]), dtype=np.int32)[None, :]
        pt_d = np.arange(len(dst_pt[g]), dtype=np.int32)[None, :]
        kd = np.zeros((len(dst_pt[g]), ps, H, D), np.uint16)
        vd = np.zeros_like(kd)
        oracle.compact({"paged": True, "page_table": pt_s}, ks, vs,
                       {"paged": True, "page_table": pt_d}, kd, vd, want_k, cfg.K, D, H, 0, 1,
                       ipg=1 if cfg.shared else H, page_size=ps)
        assert np.array_equal(u16(st.k_dst[dp]), kd), g
        assert np.array_equal(u16(st.v_dst[dp]), vd), g
    # page accounting: 132 source pages per group become 128
    assert st.src_pt.shape[1] == 132 and st.dst_pt.shape[1] == 128
    del st
    free()


def test_global_round():
    """GateSight-shaped global round: scores within rel 1e-5, selection bit-exact given
    identical scores, budget identity, compaction equal to the gather of the kept rows."""
    cfg = configs.GLOBAL
    say("global round: allocating")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st)
    torch.cuda.synchronize()
    lists = cfg.L * cfg.H
    B_want = oracle.budget(lists, cfg.n, cfg.prot, cfg.p)
    assert st.budget == B_want == 520192
    counts = st.kept_count
    assert int(counts.sum()) == lists * cfg.prot + B_want
    assert int(st.errors.item()) == 0
    say("global round: weighted scores at all 64 x 32,768 positions against the oracle's")
    beta, vnorm, w = st.beta.cpu().numpy(), st.vnorm.cpu().numpy(), st.weights.cpu().numpy()
    got = st.scores.cpu().numpy()[:, :cfg.n]
    want = np.empty((lists, cfg.n), np.float32)
    wins = oracle.gdn_windows(cfg.L, cfg.G, cfg.win_width)
    step = -(-cfg.n // (4 * THREADS))

    def part(t0):
        t1 = min(cfg.n, t0 + step)
        want[:, t0:t1] = oracle.score_weighted(beta, vnorm, w, *wins, cfg.prot, t_begin=t0,
                                               t_end=t1)[:, t0:t1]

    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(part, range(0, cfg.n, step)))
    fin = np.isfinite(want)
    assert np.array_equal(np.isposinf(got), np.isposinf(want))
    rel = np.abs(got[fin].astype(np.float64) - want[fin]) / np.maximum(np.abs(want[fin]), 1e-30)
    assert rel.max() <= 1e-5, float(rel.max())
    say(f"  bit-identical fraction {float(np.mean(got[fin] == want[fin])):.6f}, "
        f"largest relative difference {float(rel.max()):.3g}")
    say("global round: the oracle's top-B of the round's own scores, every list")
    want_kept, want_counts, _ = oracle.select_global(got, cfg.prot, cfg.p)
    assert np.array_equal(st.kept_count.cpu().numpy(), want_counts)
    got_kept = st.kept.cpu().numpy()
    for l in range(lists):
        assert np.array_equal(got_kept[l, :want_counts[l]], want_kept[l, :want_counts[l]]), l
    say("global round: every list's rows against a gather through the oracle's indices")
    check_contig_gather(st, cfg.n, counts=torch.from_numpy(want_counts).to(DEV), chunk=8,
                        kept=want_kept)
    del beta, vnorm, got, want
    say("global round: selection on identical (oracle-side) scores")
    s = synth.uniform_scores(lists, cfg.n, seed=17, device="cpu").numpy()
    s[:, :cfg.prot] = np.inf
    st.scores.copy_(torch.from_numpy(s))
    rounds.select(st)
    torch.cuda.synchronize()
    want_kept, want_counts, _ = oracle.select_global(s, cfg.prot, cfg.p)
    assert np.array_equal(st.kept_count.cpu().numpy(), want_counts)
    got_kept = st.kept.cpu().numpy()
    for l in range(lists):
        assert np.array_equal(got_kept[l, :want_counts[l]], want_kept[l, :want_counts[l]]), l
    del st
    free()


def test_global_fused_round_matches_three_calls():
    """The GateSight-shaped round with the weighted score and the top-B in one call: scores,
    budget, counts, kept indices and compacted rows equal the three-call round's, bit for
    bit, and the kept set is the oracle's top-B of those scores."""
    say("global fused round: allocating")
    st3 = rounds.make_state(configs.GLOBAL, DEV)
    rounds.run_round(st3)
    torch.cuda.synchronize()
    want = {k: getattr(st3, k).clone() for k in ("scores", "kept", "kept_count")}
    want_k, want_v, want_budget = st3.k_dst.clone(), st3.v_dst.clone(), st3.budget
    del st3
    free()
    cfg = configs.GLOBAL_FUSED
    st = rounds.make_state(cfg, DEV)
    for rep in range(2):
        rounds.run_round(st)
        torch.cuda.synchronize()
        assert st.budget == want_budget == 520192
        for k, v in want.items():
            got = getattr(st, k)
            assert torch.equal(got.view(torch.int32), v.view(torch.int32)), (k, rep)
        assert torch.equal(st.k_dst.view(torch.int16), want_k.view(torch.int16))
        assert torch.equal(st.v_dst.view(torch.int16), want_v.view(torch.int16))
        assert int(st.errors.item()) == 0
    say("global fused round: the oracle's top-B of the GPU scores")
    s = st.scores.cpu().numpy()
    want_kept, want_counts, _ = oracle.select_global(s[:, :cfg.n], cfg.prot, cfg.p)
    assert np.array_equal(st.kept_count.cpu().numpy(), want_counts)
    got_kept = st.kept.cpu().numpy()
    for l in range(cfg.L * cfg.H):
        assert np.array_equal(got_kept[l, :want_counts[l]], want_kept[l, :want_counts[l]]), l
    del st, want, want_k, want_v
    free()


def test_longgen_rounds_replayed_by_oracle():
    """30 consecutive rounds (K=3072, r=64, prot=557) on one request's 288 lists, replayed
    round by round by the oracle; survival of the first cache's entries follows q^t."""
    cfg = configs.LONGGEN.small(R=1)
    say("longgen replay")
    st = rounds.make_state(cfg, DEV)
    lists, n, K, r, D = cfg.lists, cfg.n, cfg.K, cfg.r, cfg.D
    host_k, host_v = u16(st.k_src), u16(st.v_src)
    ids = np.tile(np.arange(n, dtype=np.int64), (lists, 1))
    next_id = n
    surv = []
    for rnd in range(cfg.rounds):
        rounds.run_round(st, round_id=rnd)
        torch.cuda.synchronize()
        want_s = oracle.score_random(cfg.L, cfg.H, n, cfg.prot, cfg.seed, rnd, False, 0, lists)
        want_k = oracle.select_topk(want_s, K, cfg.prot)
        assert np.array_equal(st.kept.cpu().numpy(), want_k), rnd
        kd = np.zeros((lists, n, D), np.uint16)
        vd = np.zeros_like(kd)
        oracle.compact({"list_stride": n * D}, host_k, host_v, {"list_stride": n * D}, kd, vd,
                       want_k, K, D, cfg.H, 0, cfg.groups, ipg=cfg.H)
        assert np.array_equal(u16(st.k_dst[:, :K]), kd[:, :K]), rnd
        assert np.array_equal(u16(st.v_dst[:, :K]), vd[:, :K]), rnd
        rounds.append_tokens(st, rnd)
        torch.cuda.synchronize()
        kd[:, K:] = u16(st.k_dst[:, K:])
        vd[:, K:] = u16(st.v_dst[:, K:])
        host_k, host_v = kd, vd
        ids = np.concatenate([np.take_along_axis(ids, want_k.astype(np.int64), axis=1),
                              np.tile(np.arange(next_id, next_id + r), (lists, 1))], axis=1)
        next_id += r
        surv.append(np.isin(ids, np.arange(cfg.prot, n)).sum() / (lists * (n - cfg.prot)))
        rounds.swap(st)
    assert st.applied_rounds == cfg.rounds == 30
    assert int(st.errors.item()) == 0
    q = (K - cfg.prot) / (K + r - cfg.prot)
    N = lists * (n - cfg.prot)
    for t, got in enumerate(surv, start=1):
        e = q ** t
        assert abs(got - e) < 3 * math.sqrt(e * (1 - e) / N) + 1e-12, (t, got, e)
    del st
    free()


def test_paged_shared_max_round_full():
    """Paged round with one list per (request, layer) by the max of the per-head scores and a
    kept count rounded down to a multiple of four: every group's shared scores and keep set
    against the oracle's, every group's destination pages against a page walk of the source
    through the oracle's indices."""
    cfg = configs.PAGED_SHARED_MAX
    say("paged shared-max round: allocating")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st, round_id=5)
    torch.cuda.synchronize()
    assert int(st.errors.item()) == 0
    K4 = cfg.kept_shared
    assert K4 % 4 == 0 and K4 == oracle.shared_kept_count(cfg.K, cfg.prot)
    H, groups = cfg.H, cfg.groups
    got_s = st.scores[:groups].cpu().numpy()
    want_k = np.empty((groups, K4), np.int32)
    bad = []
    step = max(16, -(-groups // (4 * THREADS)))

    def part(g0):
        g1 = min(groups, g0 + step)
        heads = oracle.score_random(cfg.L, H, cfg.n, cfg.prot, cfg.seed, 5, False, g0 * H, g1 * H)
        want_s = oracle.shared_max_scores(heads, H)
        if not np.array_equal(got_s[g0:g1], want_s):
            bad.append(g0)
        want_k[g0:g1] = oracle.select_topk(want_s, K4, cfg.prot)

    say(f"paged shared-max round: the oracle's scores and keep sets of all {groups} groups")
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(part, range(0, groups, step)))
    assert not bad, f"shared scores differ in the group ranges starting at {sorted(bad)[:4]}"
    assert_keep_sets(st.kept[:, :K4], want_k, cfg.name)
    check_paged_gather(st, cfg, want_k, K4)
    del st
    free()


def test_layers_round():
    """GateSight's per-layer allocation at the global round's shape: every head of layer l
    keeps prot + K_l, the K_l sum to the flat total, selection bit-exact on identical scores,
    compaction equal to the gather of the kept rows."""
    cfg = configs.LAYERS
    say("layers round: allocating")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st)
    torch.cuda.synchronize()
    lists, n_body = cfg.L * cfg.H, cfg.n - cfg.prot
    gate = synth.layer_gates(cfg.L, synth.SEED_GATES)
    want_b = oracle.layer_power_budget(gate, n_body, cfg.p)
    assert st.layer_budget == want_b
    assert sum(want_b) == cfg.L * oracle.budget(1, n_body, 0, cfg.p)
    counts = st.kept_count.cpu().numpy()
    assert np.array_equal(counts, cfg.prot + np.repeat(np.array(want_b), cfg.H))
    assert int(st.errors.item()) == 0
    say("layers round: compaction of every list")
    check_contig_gather(st, cfg.n, counts=st.kept_count, chunk=8)
    say("layers round: selection on identical (oracle-side) scores")
    s = synth.uniform_scores(lists, cfg.n, seed=23, device="cpu").numpy()
    s[:, :cfg.prot] = np.inf
    st.scores.copy_(torch.from_numpy(s))
    rounds.select(st)
    torch.cuda.synchronize()
    got = st.kept.cpu().numpy()
    want_l = np.zeros((lists, cfg.n), bool)
    for lst in range(lists):
        K = cfg.prot + want_b[lst // cfg.H]
        want_k = oracle.select_topk(s[lst:lst + 1], K, cfg.prot)[0]
        assert np.array_equal(got[lst, :K], want_k), lst
        want_l[lst, want_k] = True
    say("layers round: against the global top-B at the same total")
    cmp = rounds.compare_with_global(st)
    kg, cg, total_g = oracle.select_global(s, cfg.prot, cfg.p)
    want_g = np.zeros((lists, cfg.n), bool)
    for lst in range(lists):
        want_g[lst, kg[lst, :cg[lst]]] = True
    body = slice(cfg.prot, cfg.n)
    assert cmp["total_kept_global"] == total_g == cmp["total_kept_layers"] == sum(want_b) * cfg.H
    assert cmp["per_layer_kept_layers"] == [b * cfg.H for b in want_b]
    assert cmp["per_layer_kept_global"] == list((cg - cfg.prot).reshape(cfg.L, cfg.H).sum(1))
    inter = int((want_l[:, body] & want_g[:, body]).sum())
    assert cmp["kept_overlap"] == inter / cmp["total_kept_layers"]
    del st
    free()


def test_keydiff_round():
    """The batch round scored by KeyDiff: every list's keep set against the oracle's top-K of
    the GPU's scores (selection bit-exact given identical scores) and every compacted row
    against a gather through those oracle indices; the scores themselves on 60 sampled lists
    against the oracle's (the stated precision: the oracle's fp32 rounding, or its neighbour
    next to a midpoint), since the oracle's plain per-row loop would take minutes for all."""
    cfg = configs.KEYDIFF
    say("keydiff round: allocating")
    st = rounds.make_state(cfg, DEV)
    rounds.run_round(st)
    torch.cuda.synchronize()
    assert int(st.errors.item()) == 0
    got_s = st.scores.cpu().numpy()
    say(f"keydiff round: the oracle's top-K of all {cfg.lists} lists' scores")
    want_k = oracle_select_all(got_s, cfg.K, cfg.prot)
    assert_keep_sets(st.kept, want_k, cfg.name)
    check_contig_gather(st, cfg.K, kept=want_k)
    del want_k
    say("keydiff round: sampled scores against the oracle's")
    for l in sample_lists(cfg.lists, 60, seed=8):
        assert_keydiff_close(got_s[l:l + 1], u16(st.k_src[l:l + 1]), cfg.prot)
    del st
    free()


@pytest.mark.parametrize("base", [configs.PAGED_INPLACE, configs.PAGED_FUSED], ids=lambda c: c.name)
def test_paged_inplace_round_full(base):
    """Paged round compacted in place (three launches, or the one-launch fused round): every
    keep set against the oracle's; for every group and head, the first K rows walked through
    the group's own page table equal the rows of the cache before the round at the oracle's
    indices, and every tail page (rows past K) is untouched; every group returns its 4 tail
    pages (132 -> 128) and the free list holds exactly those pages."""
    cfg = base
    say(f"{cfg.name} round: allocating")
    st = rounds.make_state(cfg, DEV)
    ps, n, K = cfg.page_size, cfg.n, cfg.K
    k0, v0 = st.k_src.clone(), st.v_src.clone()  # the cache before the round
    rounds.run_round(st, round_id=1)
    torch.cuda.synchronize()
    assert int(st.errors.item()) == 0
    say(f"{cfg.name} round: the oracle's keep sets of all {cfg.lists} lists")
    want = oracle_keep_sets(cfg, 1)
    assert_keep_sets(st.kept, want, cfg.name)
    say(f"{cfg.name} round: every group's moved rows and tail pages")
    before = types.SimpleNamespace(k_src=k0, v_src=v0, k_dst=st.k_src, v_dst=st.v_src,
                                   src_pt=st.src_pt, dst_pt=st.src_pt)
    check_paged_gather(before, cfg, want, K)
    del want
    tail = st.src_pt[:, K // ps:].reshape(-1).long()
    assert torch.equal(st.k_src[tail], k0[tail]) and torch.equal(st.v_src[tail], v0[tail])
    del k0, v0, before
    pt = st.src_pt.cpu().numpy()
    nf = int(st.freed_count.item())
    assert nf == cfg.groups * (-(-n // ps) - K // ps) == cfg.groups * 4
    assert sorted(st.freed[:nf].cpu().tolist()) == sorted(pt[:, K // ps:].reshape(-1).tolist())
    del st
    free()


@pytest.mark.parametrize("base", [configs.LONGGEN_INPLACE, configs.LONGGEN_FUSED],
                         ids=lambda c: c.name)
def test_longgen_inplace_rounds_replayed_by_oracle(base):
    """30 rounds compacted in place on one request's 288 lists, replayed by the oracle."""
    cfg = base.small(R=1)
    say(f"{cfg.name} replay")
    st = rounds.make_state(cfg, DEV)
    lists, n, K, D = cfg.lists, cfg.n, cfg.K, cfg.D
    host_k, host_v = u16(st.k_src), u16(st.v_src)
    for rnd in range(cfg.rounds):
        rounds.run_round(st, round_id=rnd)
        torch.cuda.synchronize()
        want_s = oracle.score_random(cfg.L, cfg.H, n, cfg.prot, cfg.seed, rnd, False, 0, lists)
        want_k = oracle.select_topk(want_s, K, cfg.prot)
        assert np.array_equal(st.kept.cpu().numpy(), want_k), rnd
        kd = np.zeros((lists, K, D), np.uint16)
        vd = np.zeros_like(kd)
        oracle.compact({"list_stride": n * D}, host_k, host_v, {"list_stride": K * D}, kd, vd,
                       want_k, K, D, cfg.H, 0, cfg.groups, ipg=cfg.H)
        gk, gv = u16(st.k_src), u16(st.v_src)
        assert np.array_equal(gk[:, :K], kd), rnd
        assert np.array_equal(gv[:, :K], vd), rnd
        rounds.append_tokens(st, rnd)
        torch.cuda.synchronize()
        host_k, host_v = u16(st.k_src), u16(st.v_src)
        rounds.swap(st)
    assert st.applied_rounds == cfg.rounds and int(st.errors.item()) == 0
    del st
    free()


def test_paged_pages_round():
    """Page-granular round at the paged workload's full shape (2304 groups x 132 pages): kept
    pages and edited tables equal the oracle's on sampled groups, every group frees 4 pages,
    the free list holds exactly the evicted ids, and reading the unchanged store through the
    new table equals the gather of the kept pages' slots through the old one."""
    cfg = configs.PAGED_PAGES
    say("paged page-draw round: allocating")
    st = rounds.make_state(cfg, DEV)
    ps, H, D, n, K = cfg.page_size, cfg.H, cfg.D, cfg.n, cfg.K
    P, Kp = n // ps, K // ps
    old_pt = st.src_pt.cpu().numpy().copy()
    rounds.run_round(st, round_id=4)
    torch.cuda.synchronize()
    new_pt = st.src_pt.cpu().numpy()
    kept = st.kept.cpu().numpy()
    assert np.all(np.diff(kept, axis=1) > 0)
    assert np.all(kept[:, :cfg.prot // ps] == np.arange(cfg.prot // ps))
    for g in sample_lists(cfg.groups, 16, seed=5):
        want = oracle.page_keep_sets(cfg.L, n, K, cfg.prot, ps, cfg.seed, 4, g, g + 1)
        assert np.array_equal(kept[g:g + 1], want), g
        want_pt, _ = oracle.page_table_edit(old_pt[g:g + 1], want, P)
        assert np.array_equal(new_pt[g:g + 1], want_pt), g
        # the store through the new table = the kept pages' slots through the old table
        k_new = u16(st.k_src[torch.from_numpy(new_pt[g, :Kp].astype(np.int64)).to(DEV)])
        k_old = u16(st.k_src[torch.from_numpy(old_pt[g, kept[g]].astype(np.int64)).to(DEV)])
        assert np.array_equal(k_new, k_old), g
    nf = int(st.freed_count.item())
    assert nf == cfg.groups * (P - Kp)
    evicted = [old_pt[g, b] for g in range(cfg.groups) for b in sorted(set(range(P)) - set(kept[g]))]
    assert sorted(st.freed[:nf].cpu().tolist()) == sorted(int(x) for x in evicted)
    assert st.kv_bytes_moved() == 0
    del st
    free()


def test_fused_and_three_launch_rounds_agree():
    """The batch round with the draw inside the select and with the standalone scorer and
    select (three launches) keeps the same entries and writes the same bytes."""
    fused = configs.BATCH.small(R=4)
    plain = configs.BATCH.small(R=4, fuse_draw=False)
    assert fused.fused_select and not plain.fused_select
    say("batch round: fused vs three launches")
    a = rounds.make_state(fused, DEV)
    b = rounds.make_state(plain, DEV)
    rounds.run_round(a, round_id=6)
    rounds.run_round(b, round_id=6)
    torch.cuda.synchronize()
    assert torch.equal(a.kept, b.kept)
    assert torch.equal(a.k_dst, b.k_dst) and torch.equal(a.v_dst, b.v_dst)
    assert int(a.errors.item()) == 0 and int(b.errors.item()) == 0
    del a, b
    free()


def check_inplace_gather(st, before_k, before_v, kept, K, chunk=2048):
    """In place: each list's first K rows are the rows of the cache before the round at the
    oracle's kept indices, and its rows past K are unchanged (torch, in chunks of lists)."""
    lists = st.k_src.shape[0]
    for l0 in range(0, lists, chunk):
        l1 = min(lists, l0 + chunk)
        idx = torch.from_numpy(np.ascontiguousarray(kept[l0:l1, :K])).to(DEV).long()
        for now, before in ((st.k_src, before_k), (st.v_src, before_v)):
            b = before[l0:l1].view(torch.int16)
            g = torch.gather(b, 1, idx[:, :, None].expand(-1, -1, b.shape[2]))
            assert torch.equal(now[l0:l1, :K].view(torch.int16), g), (l0, l1)
            assert torch.equal(now[l0:l1, K:].view(torch.int16), b[:, K:]), (l0, l1)


@pytest.mark.parametrize("base", [configs.LONGGEN, configs.LONGGEN_INPLACE, configs.LONGGEN_FUSED],
                         ids=lambda c: c.name)
def test_longgen_full_size_two_rounds(base):
    """The 30-round workload at its full size (36,864 lists of 3136 rows): two rounds of the
    driver exactly as the benchmark runs them.  Every list's keep set against the oracle's
    (its draw and sort of each round), every list's rows against a gather of the cache before
    the round through the oracle's indices, sampled lists through the oracle's row copies."""
    cfg = base
    say(f"{cfg.name} full size: allocating")
    st = rounds.make_state(cfg, DEV)
    n, K, D = cfg.n, cfg.K, cfg.D
    inplace = cfg.inplace
    samples = sample_lists(cfg.lists, 10, seed=11)
    idx = torch.tensor(samples, device=DEV)
    for rnd in range(2):
        before_k, before_v = u16(st.k_src[idx]), u16(st.v_src[idx])
        if inplace:  # the round overwrites its source: keep a copy of the whole cache
            whole_k, whole_v = st.k_src.clone(), st.v_src.clone()
        rounds.run_round(st, round_id=rnd)
        torch.cuda.synchronize()
        assert int(st.errors.item()) == 0
        say(f"{cfg.name} full size: round {rnd}, the oracle's keep sets of all lists")
        want_all = oracle_keep_sets(cfg, rnd)
        assert_keep_sets(st.kept, want_all, f"{cfg.name} round {rnd}")
        say(f"{cfg.name} full size: round {rnd}, every list's rows")
        if inplace:
            check_inplace_gather(st, whole_k, whole_v, want_all, K)
            del whole_k, whole_v
        else:
            check_contig_gather(st, K, kept=want_all)
        out = (st.k_src if inplace else st.k_dst, st.v_src if inplace else st.v_dst)
        out_k, out_v = u16(out[0][idx][:, :K]), u16(out[1][idx][:, :K])
        for a, l in enumerate(samples):
            want_s = oracle.score_random(cfg.L, cfg.H, n, cfg.prot, cfg.seed, rnd, False, l, l + 1)
            want_k = oracle.select_topk(want_s, K, cfg.prot)
            assert np.array_equal(want_k[0], want_all[l]), (rnd, l)
            kd = np.zeros((1, K, D), np.uint16)
            vd = np.zeros_like(kd)
            oracle.compact({"list_stride": n * D}, before_k[a:a + 1], before_v[a:a + 1],
                           {"list_stride": K * D}, kd, vd, want_k, K, D, 1, 0, 1, ipg=1)
            assert np.array_equal(out_k[a], kd[0]), (rnd, l)
            assert np.array_equal(out_v[a], vd[0]), (rnd, l)
        del want_all
        say(f"{cfg.name} full size: round {rnd} ok")
        rounds.append_tokens(st, rnd)
        rounds.swap(st)
    del st
    free()


@pytest.mark.parametrize("name", ["tiny", "global", "global_fused", "paged_shared", "paged_single"])
def test_graph_replay_matches_eager(name):
    """A round captured as a HIP graph gives the eager round's outputs on every replay,
    with eager work (clearing every output) and synchronisations between the replays."""
    say(f"graph replay {name}")
    cfg = configs.ALL[name]
    st = rounds.make_state(cfg, DEV)

    def outputs():
        outs = [st.kept, st.k_dst, st.v_dst, st.errors]
        return outs + ([st.kept_count] if st.kept_count is not None else [])

    def clear():
        st.kept.fill_(-1)
        st.k_dst.zero_()
        st.v_dst.zero_()
        st.scores.fill_(-5.0)
        if st.kept_count is not None:
            st.kept_count.fill_(-1)

    clear()
    rounds.run_round(st, 0)
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs()]
    assert int(st.errors.item()) == 0
    g = rounds.capture_rounds(st, [0])
    for rep in range(3):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outputs(), want):
            assert torch.equal(got, ref), (name, rep)
    # several rounds in one graph: the outputs are the last round's
    clear()
    rounds.run_round(st, 2)
    torch.cuda.synchronize()
    want2 = [t.clone() for t in outputs()]
    g2 = rounds.capture_rounds(st, [1, 2])
    for rep in range(2):
        clear()
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outputs(), want2):
            assert torch.equal(got, ref), (name, "two rounds", rep)
    del g, g2, st, want, want2
    gc.collect()
    torch.cuda.empty_cache()
