"""Round driver: device buffers for a workload and one eviction round over them.

A round is the sequence of C-ABI calls the pages describe ("Random Attention"
blog summary, Algorithm 1 and the engine's chronological compaction; GateSight
problem statement for the global budget):

    random draw:   kvevict_select_random (draw + top-K) -> kvevict_compact
                   (or kvevict_score_random -> kvevict_select_topk -> kvevict_compact)
    weighted:      kvevict_score_weighted -> kvevict_select_global -> kvevict_compact
    fused:         kvevict_evict_random_inplace (draw, pin, top-K, in-place move)
    page draw:     kvevict_evict_pages_random (draw per page, page-table edits)

Buffers are torch tensors used only as device memory; every step of the round
runs in the HIP library.  The repeated-round driver (persistent budget K,
recent buffer r, evict when n = K + r) ping-pongs two caches, appends r fresh
tokens between rounds (input synthesis, outside the round) and counts the
rounds it applied.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from . import binding as B
from . import synth
from .configs import RoundConfig, gdn_windows


@dataclass
class RoundState:
    cfg: RoundConfig
    device: torch.device
    k_src: torch.Tensor
    v_src: torch.Tensor
    k_dst: torch.Tensor
    v_dst: torch.Tensor
    scores: torch.Tensor
    kept: torch.Tensor
    src_desc: B.KvDesc
    dst_desc: B.KvDesc
    errors: torch.Tensor
    kept_count: torch.Tensor | None = None
    workspace: torch.Tensor | None = None
    workspace_bytes: int = 0
    src_pt: torch.Tensor | None = None
    dst_pt: torch.Tensor | None = None
    beta: torch.Tensor | None = None
    vnorm: torch.Tensor | None = None
    weights: torch.Tensor | None = None
    win_begin: list = field(default_factory=list)
    win_count: list = field(default_factory=list)
    n: int = 0
    applied_rounds: int = 0
    budget: int = 0
    layer_budget: list = field(default_factory=list)
    head_scores: torch.Tensor | None = None  # per-head scores before the max over heads
    k_pristine: torch.Tensor | None = None   # in place, one round: the cache before the round
    v_pristine: torch.Tensor | None = None
    freed: torch.Tensor | None = None        # in place, paged: the free-page list
    freed_count: torch.Tensor | None = None
    pt_pristine: torch.Tensor | None = None  # page draw, one round: the table before the round
    order_ws: torch.Tensor | None = None     # paged destination: the ordered gather's workspace
    order_ws_bytes: int = 0

    @property
    def idx_lists(self) -> int:
        return self.cfg.lists

    def kv_bytes_moved(self) -> int:
        """Read + write bytes of the kept K and V rows of one round (in place: of the rows
        that move, those whose kept index differs from their slot)."""
        c = self.cfg
        if c.page_draw:
            return 0  # whole pages stay where they are: only table entries change
        if c.inplace:
            K = c.kept_shared if c.shared_max else c.K
            j = torch.arange(K, device=self.kept.device, dtype=self.kept.dtype)
            moved = int((self.kept[:, :K] != j).sum().item())
            heads = c.H if (c.shared or c.shared_max) else 1
            return moved * heads * c.row_bytes * 2 * 2
        if c.select in ("global", "layers"):
            rows = int(self.kept_count.sum().item())
        elif c.shared_max:
            rows = c.groups * c.H * c.kept_shared
        else:
            rows = c.groups * c.H * c.K
        return rows * c.row_bytes * 2 * 2


    def algorithmic_bytes(self) -> dict:
        """Bytes one round must move at minimum, by kind: the K/V rows (kv_bytes_moved), the
        scores written once and read once (none when drawn inside the select), the kept
        indices written once and read once by the gather, and the inputs a scorer reads
        (GDN signals, or the keys for KeyDiff), or the page-table entries a page draw edits."""
        c = self.cfg
        n, K = self.n, c.K
        out = {"kv": self.kv_bytes_moved(), "scores": 0, "indices": 0, "inputs": 0}
        if c.page_draw:
            P, Kp = n // c.page_size, K // c.page_size
            out["inputs"] = c.groups * (P * 4 * 2 + (P - Kp) * 4)
            out["indices"] = c.groups * Kp * 4
            return out
        if c.select in ("global", "layers"):
            lists = c.L * c.H * c.R
            out["scores"] = lists * n * 4 * 2
            out["indices"] = int(self.kept_count.sum().item()) * 4 * 2 + lists * 4 * 2
            out["inputs"] = 2 * c.G * n * c.Hg * 4
            return out
        kept_lists = c.lists
        kk = c.kept_shared if c.shared_max else K
        out["indices"] = kept_lists * kk * 4 * (1 if c.fused else 2)
        if c.fused or c.fused_select:
            return out
        if c.shared_max:
            out["scores"] = (c.groups * c.H + c.groups) * n * 4 * 2
        else:
            out["scores"] = kept_lists * n * 4 * 2
        if c.scorer == "keydiff":
            out["inputs"] = c.groups * c.H * n * c.D * 2
        return out


def _desc_pair(cfg: RoundConfig, n_src: int, cap_dst: int, device, seed: int):
    """Allocate K/V source and destination stores and their descriptors."""
    D, H, G = cfg.D, cfg.H, cfg.groups
    if cfg.layout == "contig":
        k_src = synth.kv_normal((G * H, n_src, D), seed, device)
        v_src = synth.kv_normal((G * H, n_src, D), seed + 1000, device)
        k_dst = torch.zeros((G * H, cap_dst, D), dtype=torch.bfloat16, device=device)
        v_dst = torch.zeros_like(k_dst)
        return (k_src, v_src, k_dst, v_dst, B.contig_desc(D, H, n_src),
                B.contig_desc(D, H, cap_dst), None, None)
    ps = cfg.page_size
    src_pages = -(-n_src // ps)
    dst_pages = -(-cap_dst // ps)
    pool_src = G * src_pages
    pool_dst = G * dst_pages
    src_pt = synth.page_tables(G, src_pages, pool_src, synth.SEED_PAGES, device)
    dst_pt = synth.page_tables(G, dst_pages, pool_dst, synth.SEED_PAGES + 1, device)
    k_src = synth.kv_normal((pool_src, ps, H, D), seed, device)
    v_src = synth.kv_normal((pool_src, ps, H, D), seed + 1000, device)
    k_dst = torch.zeros((pool_dst, ps, H, D), dtype=torch.bfloat16, device=device)
    v_dst = torch.zeros_like(k_dst)
    return (k_src, v_src, k_dst, v_dst, B.paged_desc(D, H, ps, pool_src, src_pt),
            B.paged_desc(D, H, ps, pool_dst, dst_pt), src_pt, dst_pt)


def make_state(cfg: RoundConfig, device="cuda", kv_seed: int = synth.SEED_KV) -> RoundState:
    device = torch.device(device)
    if cfg.fused and not (cfg.inplace and cfg.scorer == "random" and cfg.select == "topk"
                          and not cfg.shared_max):
        raise ValueError("the fused round is the random draw, top-K and in-place move")
    if cfg.page_draw and not (cfg.inplace and cfg.layout == "paged" and cfg.scorer == "random"
                              and cfg.rounds == 1 and cfg.n % cfg.page_size == 0
                              and cfg.K % cfg.page_size == 0):
        raise ValueError("the page draw edits one paged round's tables in place")
    n = cfg.n
    cap_dst = n if cfg.select in ("global", "layers") else (cfg.K + cfg.r if cfg.rounds > 1 else cfg.K)
    if cfg.inplace:
        cap_dst = 1  # no destination store: rows move within the source
    ks, vs, kd, vd, sd, dd, spt, dpt = _desc_pair(cfg, n, cap_dst, device, kv_seed)
    lists = cfg.lists if cfg.select == "topk" else cfg.groups * cfg.H
    scores = torch.empty((lists, n), dtype=torch.float32, device=device)
    kept_cols = n if cfg.select in ("global", "layers") else cfg.K
    if cfg.page_draw:
        lists, kept_cols = cfg.groups, cfg.K // cfg.page_size  # kept pages per (request, layer)
    kept = torch.zeros((lists, kept_cols), dtype=torch.int32, device=device)
    st = RoundState(cfg, device, ks, vs, kd, vd, scores, kept, sd, dd,
                    torch.zeros(1, dtype=torch.int32, device=device), src_pt=spt, dst_pt=dpt, n=n)
    if cfg.shared_max:
        st.head_scores = torch.empty((cfg.groups * cfg.H, n), dtype=torch.float32, device=device)
    if cfg.inplace:
        st.k_dst, st.v_dst, st.dst_desc, st.dst_pt = st.k_src, st.v_src, st.src_desc, st.src_pt
        if cfg.rounds == 1 and not cfg.page_draw:
            st.k_pristine, st.v_pristine = ks.clone(), vs.clone()
        if cfg.layout == "paged":
            st.freed = torch.empty(cfg.groups * spt.shape[1], dtype=torch.int32, device=device)
            st.freed_count = torch.zeros(1, dtype=torch.int32, device=device)
        if cfg.page_draw:
            st.pt_pristine = spt.clone()
    if cfg.layout == "paged" and not cfg.inplace:
        # the gather visits the fresh destination pages in physical order
        st.order_ws_bytes = max(B.kvevict_compact_ordered_workspace(st.dst_desc),
                                B.kvevict_compact_ordered_workspace(st.src_desc))  # after a swap
        st.order_ws = torch.empty(max(st.order_ws_bytes, 256), dtype=torch.uint8, device=device)
    if cfg.select == "layers":
        st.kept_count = torch.zeros(lists, dtype=torch.int32, device=device)
        st.layer_budget = B.kvevict_layer_power_budget(synth.layer_gates(cfg.L, synth.SEED_GATES),
                                                       n - cfg.prot, cfg.p)
        st.budget = sum(st.layer_budget) * cfg.R * cfg.H  # non-prompt entries kept
    if cfg.select == "global":
        st.kept_count = torch.zeros(lists, dtype=torch.int32, device=device)
        st.workspace_bytes = B.kvevict_select_global_workspace(lists, n, cfg.prot, p=cfg.p)
        st.workspace = torch.empty(max(st.workspace_bytes, 256), dtype=torch.uint8, device=device)
    if cfg.scorer == "weighted":
        st.beta, st.vnorm = synth.gdn_signals(cfg.G, n, cfg.Hg, synth.SEED_SIGNALS, device)
        st.weights = synth.head_weights(cfg.L, cfg.H, cfg.win_width, cfg.Hg, synth.SEED_WEIGHTS,
                                        device)
        st.win_begin, st.win_count = gdn_windows(cfg.L, cfg.G, cfg.win_width)
    return st


# --- the steps of one round -------------------------------------------------------

def score(st: RoundState, round_id: int, stream=None):
    c = st.cfg
    if c.scorer == "random" and c.shared_max:
        # per-head draws, then one list per (request, layer) by the max over its heads
        hs = st.head_scores
        B.kvevict_score_random(hs, hs.shape[1], c.R, c.L, c.H, st.n, c.prot, c.seed, round_id,
                               False, stream)
        B.kvevict_reduce_max_heads(st.scores, st.scores.shape[1], hs, hs.shape[1], c.groups, c.H,
                                   st.n, stream)
    elif c.scorer == "random":
        B.kvevict_score_random(st.scores, st.scores.shape[1], c.R, c.L, c.H, st.n, c.prot, c.seed,
                               round_id, c.shared, stream)
    elif c.scorer == "keydiff":
        B.kvevict_score_keydiff(st.scores, st.scores.shape[1], st.src_desc, st.k_src, c.groups,
                                st.n, c.prot, stream)
    else:
        n = st.n
        B.kvevict_score_weighted(st.scores, st.scores.shape[1], st.beta, st.vnorm, n * c.Hg, c.Hg,
                                 1, st.weights, c.win_width, st.win_begin, st.win_count, c.L, c.H,
                                 c.G, c.Hg, n, c.prot, stream)


def score_select(st: RoundState, round_id: int, stream=None):
    """Weighted score and global top-B in one call (the scorer fills the first radix level)."""
    c, n = st.cfg, st.n
    st.budget = B.kvevict_score_select_global(st.kept, st.kept.shape[1], st.kept_count, st.scores,
                                              st.scores.shape[1], st.beta, st.vnorm, n * c.Hg,
                                              c.Hg, 1, st.weights, c.win_width, st.win_begin,
                                              st.win_count, c.L, c.H, c.G, c.Hg, n, c.prot, c.p,
                                              st.workspace, st.workspace_bytes, stream)


def select(st: RoundState, stream=None):
    c = st.cfg
    lists = st.scores.shape[0]
    if c.select == "topk":
        K = c.kept_shared if c.shared_max else c.K
        B.kvevict_select_topk(st.kept, st.kept.shape[1], st.scores, st.scores.shape[1], lists, st.n,
                              K, c.prot, stream)
    elif c.select == "layers":
        B.kvevict_select_topk_layers(st.kept, st.kept.shape[1], st.kept_count, st.scores,
                                     st.scores.shape[1], c.groups, c.L, c.H, st.n, c.prot,
                                     st.layer_budget, stream)
    else:
        st.budget = B.kvevict_select_global(st.kept, st.kept.shape[1], st.kept_count, st.scores,
                                            st.scores.shape[1], lists, st.n, c.prot, c.p,
                                            st.workspace, st.workspace_bytes, stream)


def compact(st: RoundState, stream=None):
    c = st.cfg
    if c.select == "topk":
        K, count = (c.kept_shared if c.shared_max else c.K), None
    else:
        K, count = st.n, st.kept_count
    ipg = 1 if (c.shared or c.shared_max) else c.H
    if c.inplace:
        B.kvevict_compact_inplace(st.src_desc, st.k_src, st.v_src, st.kept, st.kept.shape[1], count,
                                  K, st.n, c.groups, ipg, st.freed, st.freed_count, st.errors,
                                  stream)
        return
    if st.order_ws is not None:
        B.kvevict_compact_ordered(st.src_desc, st.k_src, st.v_src, st.dst_desc, st.k_dst,
                                  st.v_dst, st.kept, st.kept.shape[1], count, K, c.groups, ipg,
                                  st.order_ws, st.order_ws_bytes, st.errors, stream)
        return
    B.kvevict_compact(st.src_desc, st.k_src, st.v_src, st.dst_desc, st.k_dst, st.v_dst, st.kept,
                      st.kept.shape[1], count, K, c.groups, ipg, st.errors, stream)


def fused_round(st: RoundState, round_id: int, stream=None):
    """Random draw, pin, top-K and in-place compaction of every list in one launch."""
    c = st.cfg
    B.kvevict_evict_random_inplace(st.src_desc, st.k_src, st.v_src, c.R, c.L, st.n, c.K, c.prot,
                                   c.seed, round_id, c.shared, st.kept, st.kept.shape[1], st.freed,
                                   st.freed_count, st.errors, stream)


def pages_round(st: RoundState, round_id: int, stream=None):
    """One draw per page (shared draw of its first slot), top pages, page-table edits."""
    c = st.cfg
    B.kvevict_evict_pages_random(st.src_pt, st.src_pt.shape[1], c.page_size, c.R, c.L, st.n, c.K,
                                 c.prot, c.seed, round_id, st.kept, st.kept.shape[1], st.freed,
                                 st.freed_count, stream)


def draw_select(st: RoundState, round_id: int, stream=None):
    """Random scores drawn on chip and the per-list top-K, in one launch."""
    c = st.cfg
    B.kvevict_select_random(st.kept, st.kept.shape[1], c.R, c.L, c.H, st.n, c.K, c.prot, c.seed,
                            round_id, c.shared, stream)


def phases(cfg: RoundConfig):
    """The launches of one round as (name, fn(st, round_id)) in order."""
    if cfg.fused_select:
        return [("draw_select", draw_select), ("compact", lambda st, rid: compact(st))]
    if cfg.page_draw:
        return [("pages", pages_round)]
    if cfg.fused:
        return [("fused", fused_round)]
    if cfg.fuse_score:
        return [("score_select", score_select), ("compact", lambda st, rid: compact(st))]
    return [("score", score), ("select", lambda st, rid: select(st)),
            ("compact", lambda st, rid: compact(st))]


def run_round(st: RoundState, round_id: int = 0, stream=None):
    if st.cfg.fused_select:
        draw_select(st, round_id, stream)
        compact(st, stream)
    elif st.cfg.page_draw:
        pages_round(st, round_id, stream)
    elif st.cfg.fused:
        fused_round(st, round_id, stream)
    elif st.cfg.fuse_score:
        score_select(st, round_id, stream)
        compact(st, stream)
    else:
        score(st, round_id, stream)
        select(st, stream)
        compact(st, stream)
    st.applied_rounds += 1


def capture_rounds(st: RoundState, round_ids=(0,)) -> "torch.cuda.CUDAGraph":
    """Out-of-place rounds, one per round id, recorded in order as one HIP graph.

    Replaying the graph reruns the rounds' launches with the arguments they had
    at capture (round ids, budget and buffers included) without the host launch
    path, which dominates rounds of a few microseconds; several rounds per graph
    spread the graph's own launch over them.  The rounds run once eagerly first,
    so any one-time set-up of the library happens outside the capture.
    In-place, page-draw and repeated rounds change their own inputs, so replays
    would not repeat the same rounds; they are not captured.
    """
    c = st.cfg
    if c.inplace or c.page_draw or c.rounds > 1:
        raise ValueError(f"{c.name}: only single out-of-place rounds are captured")
    for rid in round_ids:
        for _, fn in phases(c):
            fn(st, rid)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for rid in round_ids:
            for _, fn in phases(c):
                fn(st, rid)
    return g


# --- repeated rounds (persistent budget K + recent buffer r) ------------------------

def append_tokens(st: RoundState, round_id: int):
    """Write r fresh N(0,1) tokens at rows [K, K+r) of the destination cache (input synthesis)."""
    c = st.cfg
    seed = synth.SEED_APPEND * 1_000_003 + round_id
    st.k_dst[:, c.K:c.K + c.r].copy_(synth.kv_normal((st.k_dst.shape[0], c.r, c.D), seed,
                                                     st.device))
    st.v_dst[:, c.K:c.K + c.r].copy_(synth.kv_normal((st.v_dst.shape[0], c.r, c.D), seed + 7,
                                                     st.device))


def restore(st: RoundState):
    """In place, one round: put the cache back as it was before the round (input set-up)."""
    if st.pt_pristine is not None:
        st.src_pt.copy_(st.pt_pristine)  # the K/V bytes never change under page edits
    else:
        st.k_src.copy_(st.k_pristine)
        st.v_src.copy_(st.v_pristine)
    if st.freed_count is not None:
        st.freed_count.zero_()


def swap(st: RoundState):
    """The compacted cache (K kept + r appended rows) becomes the next round's source
    (in place there is one cache: nothing to swap)."""
    if st.cfg.inplace:
        return
    st.k_src, st.k_dst = st.k_dst, st.k_src
    st.v_src, st.v_dst = st.v_dst, st.v_src
    st.src_desc, st.dst_desc = st.dst_desc, st.src_desc


# --- measurement: per-layer budgets against the model-wide top-B ---------------------

def compare_with_global(st: RoundState) -> dict:
    """Measurement only, outside the timed round: the model-wide top-B (global select) on the
    same scores at the same total, against the per-layer allocation the round just kept.
    Reports both totals, the non-prompt entries each rule keeps per layer, and the fraction of
    kept non-prompt entries the two rules share."""
    c = st.cfg
    lists, n = st.scores.shape
    kept_g = torch.zeros_like(st.kept)
    cnt_g = torch.zeros_like(st.kept_count)
    ws_bytes = B.kvevict_select_global_workspace(lists, n, c.prot, p=c.p)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=st.device)
    total_g = B.kvevict_select_global(kept_g, kept_g.shape[1], cnt_g, st.scores, n, lists, n,
                                      c.prot, c.p, ws, ws_bytes)

    def kept_mask(kept, cnt):
        m = torch.zeros((lists, n), dtype=torch.bool, device=st.device)
        valid = torch.arange(kept.shape[1], device=st.device)[None, :] < cnt[:, None]
        rows = torch.arange(lists, device=st.device)[:, None].expand_as(kept)
        m[rows[valid], kept[valid].long()] = True
        return m[:, c.prot:]

    ml, mg = kept_mask(st.kept, st.kept_count), kept_mask(kept_g, cnt_g)
    total_l = int(ml.sum().item())
    per_l = (st.kept_count - c.prot).view(c.R, c.L, c.H).sum(dim=(0, 2))
    per_g = (cnt_g - c.prot).view(c.R, c.L, c.H).sum(dim=(0, 2))
    return {"total_kept_layers": total_l, "total_kept_global": int(total_g),
            "kept_overlap": int((ml & mg).sum().item()) / max(total_l, 1),
            "per_layer_kept_layers": per_l.tolist(), "per_layer_kept_global": per_g.tolist()}


# --- measurement: survival of entries across repeated rounds ------------------------

class SurvivalTracker:
    """Original token id of every slot on sampled lists, carried through each round's kept
    indices (the HIP path's output).  Measurement only: it runs between rounds, outside the
    timed round, and moves no K/V data.

    Tokens present before the first round get ids 0..n-1 (their slots); each round's r
    appended tokens get the next r ids.  The curve is the fraction of the first cache's
    non-prompt entries still present after each round (Random Attention blog summary,
    survival paragraph: survivors are redrawn every round), next to the law q^t with
    q = (K - prot) / (K + r - prot) and the page's prompt-free (K / (K + r))^t.
    """

    def __init__(self, st: RoundState, stride: int = 16):
        c = st.cfg
        self.rows = torch.arange(0, c.lists, stride, device=st.device)
        self.ids = torch.arange(st.n, device=st.device, dtype=torch.int64).repeat(len(self.rows), 1)
        self.next_id = st.n
        self.cohort = (c.prot, st.n)
        self.curve: list[float] = []
        self.prompt_survival = 1.0
        self.slot_coverage = 1.0

    def after_round(self, st: RoundState):
        c = st.cfg
        kept_ids = torch.gather(self.ids, 1, st.kept[self.rows].long())
        ns = len(self.rows)
        new = torch.arange(self.next_id, self.next_id + c.r, device=st.device,
                           dtype=torch.int64).repeat(ns, 1)
        self.ids = torch.cat([kept_ids, new], 1)
        self.next_id += c.r
        lo, hi = self.cohort
        alive = int(((kept_ids >= lo) & (kept_ids < hi)).sum().item())
        self.curve.append(alive / (ns * (hi - lo)))
        prompt = torch.arange(c.prot, device=st.device, dtype=torch.int64)
        self.prompt_survival = min(self.prompt_survival,
                                   float((kept_ids[:, :c.prot] == prompt).float().mean().item())
                                   if c.prot else 1.0)
        # every kept slot holds a distinct token (strictly increasing ids)
        distinct = bool((kept_ids[:, 1:] > kept_ids[:, :-1]).all().item())
        self.slot_coverage = min(self.slot_coverage, 1.0 if distinct else 0.0)

    def report(self, st: RoundState) -> dict:
        c = st.cfg
        q = (c.K - c.prot) / (c.K + c.r - c.prot)
        N = len(self.rows) * (self.cohort[1] - self.cohort[0])
        law = [q ** t for t in range(1, len(self.curve) + 1)]
        z = [(m - e) / max(math.sqrt(e * (1 - e) / N), 1e-300) for m, e in zip(self.curve, law)]
        return {"lists_sampled": len(self.rows), "entries_tracked": N,
                "measured": [round(v, 6) for v in self.curve],
                "law_q_pow_t": [round(v, 6) for v in law],
                "page_approx_K_over_K_plus_r_pow_t": [round((c.K / (c.K + c.r)) ** t, 6)
                                                       for t in range(1, len(self.curve) + 1)],
                "max_abs_z": max(abs(v) for v in z) if z else 0.0,
                "prompt_survival": self.prompt_survival, "slot_coverage": self.slot_coverage}
