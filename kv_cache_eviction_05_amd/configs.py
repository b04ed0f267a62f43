"""Workload shapes of the eviction round.

Synthetic workloads, each a single-GPU share at its real shape:

  tiny      1 layer x 2 KV heads, D=128, n=1088 (K=1024 + r=64), prot=32,
            per-head random draw, contiguous storage.
  batch     128 requests x 36 layers x 8 KV heads, D=128, n=1088, K=1024,
            prot=128, per-head random draw, contiguous storage (decode-time
            round over a full batch).
  paged     64 requests x 36 layers x 8 KV heads, D=128, n=2112, K=2048,
            prot=1024, 16-token pages behind seed-shuffled page tables,
            per-head draw ("paged") or one draw per layer ("paged_shared"),
            compacted into freshly allocated pages.
  global    16 attention layers x 4 KV heads, D=256, n=32768, prot=256, p=0.25:
            weighted GDN-signal scores over the up-to-six preceding GDN layers
            x 48 heads, then one model-wide top-B (GateSight-shaped).
  longgen   128 x 36 x 8, D=128, K=3072, r=64, prot=557: 30 consecutive rounds,
            64 fresh tokens appended between rounds, rescored every round.
  layers    the global round's shape with GateSight's per-layer allocation:
            K_l proportional to a gate weight per layer, at the same total.
  paged_shared_max
            the paged round with one kept list per (request, layer), ranked
            by the larger of the per-head random scores, kept count a
            multiple of four.
  keydiff   the batch round scored by KeyDiff (-cosine of each key to the
            mean key of its head) instead of the random draw.
  paged_inplace, longgen_inplace
            the paged and the 30-round workloads compacted in place: kept rows
            move to the front of their own rows or pages, the unchanged prefix
            stays, freed tail pages go to a free list.
  paged_fused, longgen_fused
            the same two in-place rounds as one launch per round: random draw,
            pin, top-K and in-place move per (request, layer, head), with no
            score or index buffer in memory.
  paged_pages
            the paged round with one random draw per 16-token page (the
            shared draw of its first slot): whole pages are kept or evicted,
            so compaction is a page-table edit and no K/V byte moves.

The random top-K rounds compacted out of place draw their scores inside the
select (kvevict_select_random: one launch, no score buffer) unless fuse_draw
is off; the standalone scorer stays available and tested.

Budget and trigger follow the Random Attention blog summary (persistent budget
K, recent buffer r=64, evict when the buffer is full) and the GateSight
problem statement (B = L*H*round(p*(n-prot)), prot <= 256).
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class RoundConfig:
    name: str
    R: int            # requests
    L: int            # attention layers
    H: int            # KV heads per layer
    D: int            # head dim (bf16 elements per row)
    K: int            # kept entries per head (top-K mode, prompt included)
    r: int            # recent buffer; a round fires at n = K + r
    prot: int         # protected prompt prefix
    layout: str = "contig"     # "contig" or "paged"
    page_size: int = 16
    scorer: str = "random"     # "random", "weighted" or "keydiff"
    select: str = "topk"       # "topk", "global" or "layers" (gate-proportional budgets)
    shared: bool = False       # one draw per (request, layer), applied to all heads
    shared_max: bool = False   # one list per (request, layer) ranked by the max over heads
    inplace: bool = False      # compact in place (front of the same rows / pages)
    fused: bool = False        # draw + select + in-place move in one launch (random, top-K)
    page_draw: bool = False    # one draw per page; compaction as page-table edits (paged)
    fuse_draw: bool = True     # random top-K out of place: draw the scores inside the select
    fuse_score: bool = False   # weighted score and global top-B in one call
    p: float = 0.0             # kept fraction for the global budget
    rounds: int = 1
    seed: int = 0
    G: int = 48                # GDN layers (weighted scorer)
    Hg: int = 48               # GDN heads per layer
    win_width: int = 6         # GDN layers read by one attention layer
    n_override: int = 0        # n when it is not K + r (global mode)

    @property
    def fused_select(self) -> bool:
        """Random draw and top-K in one launch (out-of-place random top-K rounds)."""
        return (self.fuse_draw and self.scorer == "random" and self.select == "topk"
                and not self.shared_max and not self.inplace)

    @property
    def n(self) -> int:
        return self.n_override if self.n_override else self.K + self.r

    @property
    def groups(self) -> int:
        return self.R * self.L

    @property
    def lists(self) -> int:
        """Number of index lists: one per (request, layer, head), or per layer if shared."""
        return self.groups if (self.shared or self.shared_max) else self.groups * self.H

    @property
    def kept_shared(self) -> int:
        """Kept count of a shared-max list: K rounded down to a multiple of four."""
        return (self.K // 4) * 4

    @property
    def row_bytes(self) -> int:
        return self.D * 2

    def small(self, **kw) -> "RoundConfig":
        return replace(self, **kw)


def gdn_windows(L: int, G: int, width: int = 6):
    """GDN layers read by each attention layer, as (begin, count) lists.

    Hybrid stack of 64 layers with full attention at every fourth layer
    (GateSight, model paragraph): attention layer a follows GDN layers
    3a-3 .. 3a+2 (GDN numbering), i.e. the up-to-six preceding GDN layers, and
    only three for the first attention layer (Sec. 4.1).  ``width`` is the
    window size; the begin is clipped at 0.
    """
    per = G // L if L else 0  # GDN layers between consecutive attention layers
    begins, counts = [], []
    for a in range(L):
        end = per * (a + 1)
        b = max(0, end - width)
        begins.append(b)
        counts.append(end - b)
    return begins, counts


TINY = RoundConfig("tiny", R=1, L=1, H=2, D=128, K=1024, r=64, prot=32)
BATCH = RoundConfig("batch", R=128, L=36, H=8, D=128, K=1024, r=64, prot=128)
PAGED = RoundConfig("paged", R=64, L=36, H=8, D=128, K=2048, r=64, prot=1024, layout="paged")
PAGED_SHARED = replace(PAGED, name="paged_shared", shared=True)
GLOBAL = RoundConfig("global", R=1, L=16, H=4, D=256, K=0, r=0, prot=256, scorer="weighted",
                     select="global", p=0.25, n_override=32768)
LONGGEN = RoundConfig("longgen", R=128, L=36, H=8, D=128, K=3072, r=64, prot=557, rounds=30)
# next rows: GateSight's deployed per-layer allocation at the global round's shape and total,
# and the shared list of a layer ranked by the max over its KV heads (kept count % 4 == 0)
LAYERS = replace(GLOBAL, name="layers", select="layers")
# the global round with the weighted score and the top-B in one call (the scorer fills the
# select's first radix level)
GLOBAL_FUSED = replace(GLOBAL, name="global_fused", fuse_score=True)
PAGED_SHARED_MAX = replace(PAGED, name="paged_shared_max", shared_max=True)
# a content scorer that reads every key once more: KeyDiff at the batch round's shape
KEYDIFF = replace(BATCH, name="keydiff", scorer="keydiff")
# in-place compaction to the front of the same pages, freed tail pages to a pool
PAGED_INPLACE = replace(PAGED, name="paged_inplace", inplace=True)
LONGGEN_INPLACE = replace(LONGGEN, name="longgen_inplace", inplace=True)
PAGED_FUSED = replace(PAGED_INPLACE, name="paged_fused", fused=True)
LONGGEN_FUSED = replace(LONGGEN_INPLACE, name="longgen_fused", fused=True)
PAGED_PAGES = replace(PAGED_INPLACE, name="paged_pages", page_draw=True)
# one request of the paged shape: a single stream's whole-model round (36 layers x 8 KV heads)
PAGED_SINGLE = replace(PAGED, name="paged_single", R=1)

ALL = {c.name: c for c in (TINY, BATCH, PAGED, PAGED_SHARED, GLOBAL, GLOBAL_FUSED, LONGGEN, LAYERS,
                           PAGED_SHARED_MAX, KEYDIFF, PAGED_INPLACE, LONGGEN_INPLACE,
                           PAGED_FUSED, LONGGEN_FUSED, PAGED_PAGES, PAGED_SINGLE)}
