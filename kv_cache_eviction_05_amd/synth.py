"""Seeded synthetic inputs for the eviction round.

This module holds input generation only -- no scoring, selection or compaction
arithmetic.  Both the HIP path and the CPU oracle are fed from it (the oracle
receives host copies), so the two never share any step of the method itself.

Distributions follow the workloads the pages describe:
  * K/V rows: bf16 N(0, 1) values (the bytes are moved verbatim; their values
    never influence selection);
  * GDN signals: write gate beta = sigmoid(N(0,1)) in (0, 1) and write
    magnitude |v| = exp(N(0,1)) (log-normal), planar [G][n][Hg] fp32
    (GateSight, native GDN signals paragraph);
  * per-head weights N(0, 1), [L][H][slots][Hg] fp32;
  * page tables: seeded random permutations of a page pool;
  * layer gate weights: log-uniform over the page's measured range 0.022 to
    0.459 (GateSight Sec. 4.2), float32 [L].

Every generator takes an explicit seed and device; the same call on the same
device returns the same tensor.
"""

from __future__ import annotations

import torch

# Seed streams (fixed per input kind so inputs do not depend on call order).
SEED_KV = 1
SEED_SIGNALS = 2
SEED_WEIGHTS = 3
SEED_PAGES = 4
SEED_APPEND = 5
SEED_GATES = 6


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def kv_normal(shape, seed: int, device, chunk_rows: int | None = None) -> torch.Tensor:
    """bf16 tensor of N(0,1) values, drawn chunk by chunk along dim 0 to bound fp32 scratch."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    g = _gen(seed, device)
    first = shape[0] if len(shape) else 1
    per = 1
    for s in shape[1:]:
        per *= s
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 28) // max(per, 1))  # ~1 GiB of fp32 scratch per chunk
    for r0 in range(0, first, chunk_rows):
        r1 = min(first, r0 + chunk_rows)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        out[r0:r1].copy_(tmp)
        del tmp
    return out


def gdn_signals(G: int, n: int, Hg: int, seed: int, device):
    """(beta, vnorm) fp32 [G][n][Hg]: beta = sigmoid(N(0,1)), vnorm = exp(N(0,1))."""
    g = _gen(seed, device)
    beta = torch.sigmoid(torch.randn((G, n, Hg), generator=g, device=device))
    vnorm = torch.exp(torch.randn((G, n, Hg), generator=g, device=device))
    return beta.contiguous(), vnorm.contiguous()


def head_weights(L: int, H: int, slots: int, Hg: int, seed: int, device) -> torch.Tensor:
    """fp32 [L][H][slots][Hg] weights ~ N(0,1)."""
    g = _gen(seed, device)
    return torch.randn((L, H, slots, Hg), generator=g, device=device).contiguous()


def page_permutation(num_pages: int, seed: int, device) -> torch.Tensor:
    """int32 random permutation of [0, num_pages)."""
    g = _gen(seed, device)
    return torch.randperm(num_pages, generator=g, device=device).to(torch.int32)


def page_tables(groups: int, pages_per_group: int, pool_pages: int, seed: int,
                device) -> torch.Tensor:
    """int32 [groups][pages_per_group] of distinct physical pages drawn from a shuffled pool."""
    need = groups * pages_per_group
    if need > pool_pages:
        raise ValueError(f"pool of {pool_pages} pages cannot hold {need}")
    perm = page_permutation(pool_pages, seed, device)
    return perm[:need].reshape(groups, pages_per_group).contiguous()


def quantised_scores(lists: int, n: int, levels: int, seed: int, device) -> torch.Tensor:
    """fp32 [lists][n] scores taking only `levels` distinct values (tie stress)."""
    g = _gen(seed, device)
    q = torch.randint(0, levels, (lists, n), generator=g, device=device)
    return (q.to(torch.float32) / float(levels)).contiguous()


def uniform_scores(lists: int, n: int, seed: int, device) -> torch.Tensor:
    """fp32 [lists][n] scores uniform in [0, 1)."""
    g = _gen(seed, device)
    return torch.rand((lists, n), generator=g, device=device).contiguous()


def layer_gates(L: int, seed: int) -> list:
    """float32 gate weights [L], log-uniform over [0.022, 0.459] (host list)."""
    g = _gen(seed, "cpu")
    u = torch.rand((L,), generator=g, dtype=torch.float64)
    lo, hi = torch.log(torch.tensor(0.022, dtype=torch.float64)), torch.log(torch.tensor(0.459, dtype=torch.float64))
    return [float(x) for x in torch.exp(lo + u * (hi - lo)).to(torch.float32)]
