"""CPU oracle for the KV-cache eviction round (ctypes wrapper over oracle.cpp).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it; the two meet only through the seeded
input generators, which hold none of the method's arithmetic.

Every function states the passage it follows; the C++ file carries the
definitions.  Arrays are numpy; bf16 rows are handled as ``uint16`` bytes.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_LIB = None

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.cpp with g++ into liboracle.so (no GPU code involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_philox4x64_10.argtypes = [_p, _p, _p]
        lib.oracle_philox4x64_10.restype = None
        lib.oracle_random_draw.argtypes = [_u64, _u64, _u64, _u64, _u64, _i64]
        lib.oracle_random_draw.restype = ctypes.c_float
        lib.oracle_score_random.argtypes = [_p, _i64, _i32, _i32, _i32, _i32, _u64, _u32, _i32,
                                            _i64, _i64]
        lib.oracle_score_random.restype = None
        lib.oracle_score_weighted.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _i32, _p,
                                              _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
        lib.oracle_score_weighted.restype = None
        lib.oracle_select_topk.argtypes = [_p, _i64, _p, _i64, _i64, _i32, _i32, _i32]
        lib.oracle_select_topk.restype = None
        lib.oracle_budget.argtypes = [_i64, _i32, _i32, _dbl]
        lib.oracle_budget.restype = _i64
        lib.oracle_select_global.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i32, _i32, _dbl]
        lib.oracle_select_global.restype = _i64
        lib.oracle_compact.argtypes = [_i32, _p, _p, _i64, _p, _i64,
                                       _i32, _p, _p, _i64, _p, _i64,
                                       _i32, _i32, _i32, _p, _i64, _p, _i32, _i64, _i64, _i32]
        lib.oracle_compact.restype = None
        _LIB = lib
    return _LIB


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------------------
# Random Attention scores (blog summary, Algorithm 1; shared-draw paragraph)
# ---------------------------------------------------------------------------

def philox4x64_10(counter, key) -> np.ndarray:
    """Philox4x64-10 block (Salmon et al., SC 2011) of a 4-word counter, 2-word key."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64))
    out = np.zeros(4, dtype=np.uint64)
    _lib().oracle_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def random_draw(seed, request, layer, head, round_id, i) -> float:
    """Score of slot i: top 24 bits of Philox word i%4 at counter (i//4, head, layer, req<<32|round)."""
    return float(_lib().oracle_random_draw(seed, request, layer, head, round_id, i))


def score_random(L, H, n, prot, seed, round_id, shared_draw, list_begin, list_end,
                 out: np.ndarray | None = None) -> np.ndarray:
    """Scores of lists [list_begin, list_end) as float32 [lists][n]; slots < prot are +inf."""
    rows = list_end - list_begin
    if out is None:
        out = np.empty((rows, n), dtype=np.float32)
    _lib().oracle_score_random(_ptr(out), out.shape[1], L, H, n, prot, seed, round_id,
                               1 if shared_draw else 0, list_begin, list_end)
    return out


# ---------------------------------------------------------------------------
# GateSight-style weighted score (Sec. 4.1 window; log effective write)
# ---------------------------------------------------------------------------

def gdn_windows(L: int, G: int, width: int = 6):
    """GDN layers read by each attention layer: (begins, counts), in GDN numbering.

    GateSight, model paragraph: a hybrid stack in which every fourth layer is full
    attention and the other three are Gated DeltaNet; Sec. 4.1: an attention
    layer's estimator reads the signals of the up-to-six GDN layers before it
    (three for the first attention layer).  Written as a walk over the stack:
    each attention layer is preceded by G // L GDN layers of its own block, the
    GDN layers are numbered in stack order, and attention layer a reads the
    last ``width`` GDN layers met before it.  GDN layers past the last attention
    layer are read by none.
    """
    per_block = G // L
    seen = []                     # GDN numbers met so far, in stack order
    begins, counts = [], []
    gdn_number = 0
    for _block in range(L):
        for _ in range(per_block):
            seen.append(gdn_number)
            gdn_number += 1
        window = seen[-width:] if width > 0 else []
        begins.append(window[0] if window else len(seen))
        counts.append(len(window))
    return begins, counts


def score_weighted(beta: np.ndarray, vnorm: np.ndarray, w: np.ndarray, win_begin, win_count,
                   prot: int, t_begin: int = 0, t_end: int | None = None) -> np.ndarray:
    """Weighted scores float32 [L*H][n] from planar signals [G][n][Hg] and weights [L][H][S][Hg]."""
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    vnorm = np.ascontiguousarray(vnorm, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    G, n, Hg = beta.shape
    L, H, S, Hg2 = w.shape
    assert Hg2 == Hg and vnorm.shape == beta.shape
    wb = np.ascontiguousarray(np.asarray(win_begin, dtype=np.int32))
    wc = np.ascontiguousarray(np.asarray(win_count, dtype=np.int32))
    assert wb.shape == (L,) and wc.shape == (L,)
    assert np.all(wc <= S) and np.all(wb >= 0) and np.all(wb + wc <= G)
    if t_end is None:
        t_end = n
    out = np.full((L * H, n), np.nan, dtype=np.float32)
    _lib().oracle_score_weighted(_ptr(out), n, _ptr(beta), _ptr(vnorm), n * Hg, Hg, 1, _ptr(w),
                                 S, _ptr(wb), _ptr(wc), L, H, Hg, n, prot, t_begin, t_end)
    return out


# ---------------------------------------------------------------------------
# Selection (Algorithm 1 top-K; GateSight budget B and KVzip-style global top-B)
# ---------------------------------------------------------------------------

def select_topk(scores: np.ndarray, K: int, prot: int) -> np.ndarray:
    """Ascending kept indices int32 [lists][K]: prompt plus the K-prot best other slots."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    lists, n = scores.shape
    assert 0 <= prot <= K <= n
    kept = np.zeros((lists, max(K, 1)), dtype=np.int32)
    _lib().oracle_select_topk(_ptr(kept), kept.shape[1], _ptr(scores), n, lists, n, K, prot)
    return kept[:, :K]


def budget(num_lists: int, n: int, prot: int, p: float) -> int:
    """B = num_lists * round(p*(n-prot)), ties to even."""
    return int(_lib().oracle_budget(num_lists, n, prot, p))


def select_global(scores: np.ndarray, prot: int, p: float):
    """Global top-B: returns (kept int32 [lists][n] with -1 padding, counts int32 [lists], B)."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    lists, n = scores.shape
    kept = np.full((lists, n), -1, dtype=np.int32)
    counts = np.zeros(lists, dtype=np.int32)
    B = _lib().oracle_select_global(_ptr(kept), n, _ptr(counts), _ptr(scores), n, lists, n,
                                    prot, p)
    return kept, counts, int(B)


# ---------------------------------------------------------------------------
# Chronological compaction (blog summary: per-KV-head physical eviction with
# chronological compaction; GateSight Sec. 4.3: kept entries to the front of
# the layer's pages)
# ---------------------------------------------------------------------------

def compact(src: dict, k_src: np.ndarray, v_src: np.ndarray, dst: dict, k_dst: np.ndarray,
            v_dst: np.ndarray, kept: np.ndarray, K: int, D: int, H: int,
            group_begin: int, group_end: int, ipg: int, kept_count: np.ndarray | None = None,
            page_size: int = 16) -> None:
    """Copy kept rows src -> dst in place on the numpy arrays.

    ``src``/``dst`` describe a store: ``{"paged": bool, "list_stride": int}`` or
    ``{"paged": True, "page_table": int32 [groups][pt_ld]}``.  K/V arrays are
    uint16 views of bf16 data, flat or shaped.
    """
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    kc = None if kept_count is None else np.ascontiguousarray(kept_count, dtype=np.int32)

    def desc(d):
        if d.get("paged"):
            pt = np.ascontiguousarray(d["page_table"], dtype=np.int32)
            return 1, 0, pt, pt.shape[1]
        return 0, int(d["list_stride"]), None, 0

    sp, sls, spt, sld = desc(src)
    dp, dls, dpt, dld = desc(dst)
    for a in (k_src, v_src, k_dst, v_dst):
        assert a.dtype == np.uint16 and a.flags["C_CONTIGUOUS"]
    _lib().oracle_compact(sp, _ptr(k_src), _ptr(v_src), sls, _ptr(spt), sld,
                          dp, _ptr(k_dst), _ptr(v_dst), dls, _ptr(dpt), dld,
                          D, H, page_size, _ptr(kept), kept.shape[1], _ptr(kc), K,
                          group_begin, group_end, ipg)


# ---------------------------------------------------------------------------
# Gate-proportional per-layer budgets (GateSight Sec. 4.2; Appendix G,
# layer_power_budget) and the shared list of a layer (Appendix H)
# ---------------------------------------------------------------------------

def layer_power_budget(gate, n_body: int, p: float) -> list:
    """Entries kept per KV head in each attention layer, beyond the protected prefix.

    GateSight Sec. 4.2: layer l keeps K_l proportional to its gate weight w_l per head, with
    the model-wide total of a flat allocation; Appendix G: integerised by largest remainder so
    that the total is L * round(p * n_body) (the page's 64 = 16 layers x 4 heads counts every
    head of every layer; per head the layers sum to L * round(...)), the prompt kept in addition.
    Readings: the gates are the float32 values given, taken exactly (rational arithmetic);
    equal remainders go to the lower layer; a layer is capped at n_body and the excess is
    shared among the others in proportion (the page's gates never reach the cap).
    """
    from fractions import Fraction

    w = [Fraction(float(np.float32(g))) for g in gate]
    if any(x <= 0 for x in w):
        raise ValueError("gates must be positive")
    L = len(w)
    T = L * budget(1, n_body, 0, p)  # L * round(p * n_body), binary64 product, ties to even
    capped: set = set()
    while True:
        free = [l for l in range(L) if l not in capped]
        S = sum(w[l] for l in free)
        T2 = T - len(capped) * n_body
        over = [l for l in free if T2 * w[l] > n_body * S]
        if not over:
            break
        capped.update(over)
    q = [Fraction(n_body) if l in capped else Fraction(T2) * w[l] / S for l in range(L)]
    K = [int(x.numerator // x.denominator) for x in q]
    left = T - sum(K)
    order = sorted((l for l in range(L) if l not in capped), key=lambda l: (-(q[l] - K[l]), l))
    for l in order[:left]:
        K[l] += 1
    return K


def shared_max_scores(scores: np.ndarray, H: int) -> np.ndarray:
    """One score row per group of H consecutive lists: at each position the score of the head
    that ranks best (GateSight Appendix H: the KV heads of a layer share one kept list, ranked
    by the larger of their per-head predictions).  Ranking as everywhere: NaN as -inf, -0 equal
    to +0; among equal ranks the lowest head's score (its bits) is taken."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    lists, n = s.shape
    assert lists % H == 0
    rank = s.astype(np.float64)
    rank[np.isnan(rank)] = -np.inf
    best = np.argmax(rank.reshape(-1, H, n), axis=1)  # first maximum: the lowest head
    return np.take_along_axis(s.reshape(-1, H, n), best[:, None, :], axis=1)[:, 0, :].copy()


def shared_kept_count(K: int, prot: int) -> int:
    """Kept count of a shared layer list: K rounded down to a multiple of four (GateSight
    Appendix H: the kept count of a layer is a multiple of four, for 4-token blocks)."""
    k4 = (K // 4) * 4
    if k4 < prot:
        raise ValueError("the prompt does not fit a multiple-of-four count below K")
    return k4


# ---------------------------------------------------------------------------
# KeyDiff key scores (GateSight Sec. 5.1, baselines paragraph): minus each
# key's cosine to its head's mean key, keys taken as stored; a per-head top-K
# then keeps the keys farthest from the mean
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 stored as uint16 -> float64 (exact: the 16 bits are the top of a float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def score_keydiff(keys: np.ndarray, prot: int, binary64: bool = False) -> np.ndarray:
    """Scores float32 [lists][n] from keys (uint16 bf16 bits) [lists][n][D].

    score_i = -cos(k_i, mean_j k_j), the mean over all n keys of the list, in binary64,
    rounded once to float32; higher is kept first, so the least similar keys survive.
    Readings: the mean runs over every entry of the list, prompt included; a key or a mean
    of norm zero gives cos = 0; a zero score is written as +0; slots < prot score +inf.
    With ``binary64`` the scores are returned as float64, before that rounding.
    """
    k = bf16_to_f64(keys)
    lists, n, D = k.shape
    out = np.empty((lists, n), dtype=np.float64 if binary64 else np.float32)
    for l in range(lists):
        mean = k[l].sum(axis=0) / n if n else np.zeros(D)
        mm = float(np.dot(mean, mean))
        for i in range(n):
            if i < prot:
                out[l, i] = np.inf
                continue
            kk = float(np.dot(k[l, i], k[l, i]))
            den = math.sqrt(kk) * math.sqrt(mm)
            cos = float(np.dot(k[l, i], mean)) / den if den > 0 else 0.0
            v = -cos if binary64 else np.float32(-cos)
            out[l, i] = v if v != 0 else 0.0  # -0 written as +0
    return out


# ---------------------------------------------------------------------------
# Page-granular random eviction: one draw per page, compaction as page-table
# edits (Random Attention blog summary, Algorithm 1 applied to blocks of a
# paged cache; GateSight Sec. 4.3: one block table per layer over a shared
# pool, freed blocks back to the pool)
# ---------------------------------------------------------------------------

def page_keep_sets(L: int, n: int, K: int, prot: int, ps: int, seed: int, round_id: int,
                   group_begin: int, group_end: int) -> np.ndarray:
    """Kept pages int32 [groups][K/ps] of groups (request*L + layer) in [group_begin, group_end).

    A page holds ps token slots of every KV head, so the draw is one per (request, layer, page):
    the shared (head-0) random score of the page's first slot.  Pages holding any prompt slot
    (the first ceil(prot/ps)) are kept; among the others the K/ps - ceil(prot/ps) with the
    largest scores, ties to the lower page; the kept pages are listed in increasing order.
    """
    if n % ps or K % ps:
        raise ValueError("n and K must be whole pages")
    pp, Kp = -(-prot // ps), K // ps
    if pp > Kp:
        raise ValueError("the prompt pages do not fit the budget")
    s = score_random(L, 1, n, prot, seed, round_id, True, group_begin, group_end)
    page_scores = np.ascontiguousarray(s[:, ::ps])  # slot b*ps of each page b
    page_scores[:, :pp] = np.inf                    # a page with a prompt slot is pinned whole
    return select_topk(page_scores, Kp, pp)


def page_table_edit(pt: np.ndarray, kept_pages: np.ndarray, P: int):
    """(new table, freed ids per group): kept pages' physical ids move to the front in order,
    entries Kp..P-1 become -1, and the ids of the evicted pages are freed (ascending page
    order).  Entries at and beyond P are left as they were."""
    new = np.array(pt, dtype=np.int32, copy=True)
    Kp = kept_pages.shape[1]
    freed = []
    for g in range(pt.shape[0]):
        new[g, :Kp] = pt[g, kept_pages[g]]
        new[g, Kp:P] = -1
        keep = set(int(b) for b in kept_pages[g])
        freed.append([int(pt[g, b]) for b in range(P) if b not in keep])
    return new, freed
