"""Pins of the oracle's chronological compaction.

Kept rows are copied verbatim, in increasing index order, to the front of the
destination list (Random Attention blog summary: per-KV-head physical eviction
with chronological compaction; GateSight Sec. 4.3: each layer moves the
entries it keeps to the front of its pages).  Paged stores follow a page table
per (request, layer) with token-major pages [page][16][H][D].

Pins: numpy advanced indexing (a library routine) on the contiguous layout,
and an independent per-row dictionary walk of the page tables for the paged
layout; byte accounting of the GateSight cache (64 KiB per token).
"""

import numpy as np
import pytest

import oracle


def rand_rows(shape, seed):
    return np.random.default_rng(seed).integers(0, 1 << 16, shape, dtype=np.uint16)


def test_contig_matches_numpy_indexing():
    groups, H, n, K, D, prot = 3, 4, 50, 30, 16, 5
    rng = np.random.default_rng(0)
    cap = 64
    k_src = rand_rows((groups * H, cap, D), 1)
    v_src = rand_rows((groups * H, cap, D), 2)
    scores = rng.random((groups * H, n)).astype(np.float32)
    kept = oracle.select_topk(scores, K, prot)
    k_dst = np.zeros((groups * H, K, D), np.uint16)
    v_dst = np.zeros((groups * H, K, D), np.uint16)
    oracle.compact({"list_stride": cap * D}, k_src, v_src, {"list_stride": K * D}, k_dst, v_dst,
                   kept, K, D, H, 0, groups, ipg=H)
    lists = np.arange(groups * H)[:, None]
    assert np.array_equal(k_dst, k_src[lists, kept])
    assert np.array_equal(v_dst, v_src[lists, kept])
    assert np.array_equal(k_dst[:, :prot], k_src[:, :prot])  # prompt is a byte-identical prefix


def test_contig_shared_and_variable_counts():
    groups, H, n, D = 2, 3, 20, 8
    k_src = rand_rows((groups * H, n, D), 3)
    v_src = rand_rows((groups * H, n, D), 4)
    kept = np.array([[0, 2, 5, 9, 19, -1], [1, 3, 4, -1, -1, -1]], np.int32)
    k_dst = np.zeros((groups * H, 6, D), np.uint16)
    v_dst = np.zeros_like(k_dst)
    # shared draw: one index list per group, applied to all heads
    oracle.compact({"list_stride": n * D}, k_src, v_src, {"list_stride": 6 * D}, k_dst, v_dst,
                   np.where(kept < 0, 0, kept).astype(np.int32), 5, D, H, 0, groups, ipg=1,
                   kept_count=np.array([5, 3], np.int32))
    for g in range(groups):
        c = [5, 3][g]
        for h in range(H):
            assert np.array_equal(k_dst[g * H + h, :c], k_src[g * H + h, kept[g, :c]])
            assert np.all(k_dst[g * H + h, c:] == 0)  # rows beyond the count are untouched


def walk_paged(pool, pt, g, t, h, ps=16):
    page = int(pt[g][t // ps])
    return pool[page, t % ps, h]


@pytest.mark.parametrize("shared", [False, True])
def test_paged_against_page_walk(shared):
    groups, H, D, ps, n, K, prot = 4, 3, 8, 16, 70, 40, 10
    src_pages = -(-n // ps)
    dst_pages = -(-K // ps)
    pool_src = 40
    pool_dst = 30
    rng = np.random.default_rng(5)
    pt_src = rng.permutation(pool_src)[:groups * src_pages].reshape(groups, src_pages).astype(np.int32)
    pt_dst = rng.permutation(pool_dst)[:groups * dst_pages].reshape(groups, dst_pages).astype(np.int32)
    k_src = rand_rows((pool_src, ps, H, D), 6)
    v_src = rand_rows((pool_src, ps, H, D), 7)
    k_dst = np.zeros((pool_dst, ps, H, D), np.uint16)
    v_dst = np.zeros_like(k_dst)
    lists = groups if shared else groups * H
    kept = oracle.select_topk(rng.random((lists, n)).astype(np.float32), K, prot)
    oracle.compact({"paged": True, "page_table": pt_src}, k_src, v_src,
                   {"paged": True, "page_table": pt_dst}, k_dst, v_dst, kept, K, D, H, 0, groups,
                   ipg=1 if shared else H)
    touched = set()
    for g in range(groups):
        for h in range(H):
            idx = kept[g] if shared else kept[g * H + h]
            for j in range(K):
                assert np.array_equal(walk_paged(k_dst, pt_dst, g, j, h),
                                      walk_paged(k_src, pt_src, g, int(idx[j]), h))
                assert np.array_equal(walk_paged(v_dst, pt_dst, g, j, h),
                                      walk_paged(v_src, pt_src, g, int(idx[j]), h))
                touched.add((int(pt_dst[g][j // ps]), j % ps, h))
    # nothing outside the kept destination rows was written
    for page in range(pool_dst):
        for slot in range(ps):
            for h in range(H):
                if (page, slot, h) not in touched:
                    assert np.all(k_dst[page, slot, h] == 0)


def test_page_and_byte_accounting():
    # GateSight model paragraph: 16 layers x 4 KV heads x (K and V) x 256 values per token = 64 KiB
    assert 16 * 4 * 2 * 256 * 2 == 64 * 1024
    # paged workload (n = 2112, K = 2048, 16-token pages): 132 source pages, 128 kept, 4 freed
    n, K, ps = 2112, 2048, 16
    assert -(-n // ps) == 132 and -(-K // ps) == 128
