"""Thin ctypes binding of libkvevict.so (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors for the device pointers; it enqueues on the caller's current HIP stream
(torch.cuda.current_stream()) unless a stream is passed, and raises
KvevictError on a non-OK status.  No step of the eviction round runs here: if
the library is not built, loading it raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvevict.so")

KVEVICT_OK = 0
KVEVICT_ERR_INVALID_ARG = 1
KVEVICT_ERR_ALIGNMENT = 2
KVEVICT_ERR_WORKSPACE = 3
KVEVICT_ERR_UNSUPPORTED = 4
KVEVICT_ERR_HIP = 5

LAYOUT_CONTIG = 0
LAYOUT_PAGED = 1

EXPORTS = ("kvevict_score_random", "kvevict_score_weighted", "kvevict_select_topk",
           "kvevict_select_topk_layers", "kvevict_layer_power_budget", "kvevict_reduce_max_heads",
           "kvevict_score_keydiff", "kvevict_compact_inplace", "kvevict_evict_random_inplace",
           "kvevict_evict_pages_random", "kvevict_select_random", "kvevict_score_select_global",
           "kvevict_select_global", "kvevict_select_global_noalloc", "kvevict_compact",
           "kvevict_copy_pages", "kvevict_compact_ordered",
           "kvevict_status_string", "kvevict_abi_version")

# size of the static workspace array behind kvevict_select_global_noalloc (kvevict.h)
SELECT_GLOBAL_NOALLOC_BYTES = 1086208


class KvevictError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class KvDesc(ctypes.Structure):
    """Mirror of kvevict_kv_desc."""
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("list_stride", ctypes.c_int64),
        ("page_table", ctypes.c_void_p),
        ("pt_ld", ctypes.c_int64),
    ]


_i32, _i64, _u32, _u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
_p, _dbl, _sz = ctypes.c_void_p, ctypes.c_double, ctypes.c_size_t
_LIB = None


def load():
    """Load the built library (raises if it is missing: build it with kv_cache_eviction_05_amd.build)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m kv_cache_eviction_05_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.kvevict_score_random.argtypes = [_p, _i64, _i64, _i32, _i32, _i32, _i32, _u64, _u32, _i32, _p]
    lib.kvevict_score_weighted.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _i32, _p, _p,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _p]
    lib.kvevict_select_topk.argtypes = [_p, _i64, _p, _i64, _i64, _i32, _i32, _i32, _p]
    lib.kvevict_select_global.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i32, _i32, _dbl, _p,
                                          ctypes.POINTER(_sz), _p]
    lib.kvevict_select_global_noalloc.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i32, _i32,
                                                  _dbl, _p]
    lib.kvevict_score_select_global.argtypes = [_p, _i64, _p, _p, _p, _i64, _p, _p, _i64, _i64,
                                                _i64, _p, _i32, _p, _p, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _dbl, _p, ctypes.POINTER(_sz), _p]
    lib.kvevict_compact.argtypes = [ctypes.POINTER(KvDesc), _p, _p, ctypes.POINTER(KvDesc), _p, _p,
                                    _p, _i64, _p, _i32, _i64, _i32, _p, _p]
    lib.kvevict_select_topk_layers.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i32, _i32, _i32,
                                               _i32, _p, _p]
    lib.kvevict_layer_power_budget.argtypes = [_p, _i32, _i32, _dbl, _p]
    lib.kvevict_reduce_max_heads.argtypes = [_p, _i64, _p, _i64, _i64, _i32, _i32, _p]
    lib.kvevict_score_keydiff.argtypes = [_p, _i64, ctypes.POINTER(KvDesc), _p, _i64, _i32, _i32,
                                          _p]
    lib.kvevict_select_random.argtypes = [_p, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _u64, _u32,
                                          _i32, _p]
    lib.kvevict_evict_pages_random.argtypes = [_p, _i64, _i32, _i64, _i32, _i32, _i32, _i32, _u64,
                                               _u32, _p, _i64, _p, _p, _p]
    lib.kvevict_evict_random_inplace.argtypes = [ctypes.POINTER(KvDesc), _p, _p, _i64, _i32, _i32,
                                                 _i32, _i32, _u64, _u32, _i32, _p, _i64, _p, _p,
                                                 _p, _p]
    lib.kvevict_compact_ordered.argtypes = [ctypes.POINTER(KvDesc), _p, _p, ctypes.POINTER(KvDesc),
                                            _p, _p, _p, _i64, _p, _i32, _i64, _i32, _p, _p,
                                            ctypes.POINTER(_sz), _p]
    lib.kvevict_copy_pages.argtypes = [_p, _p, _i64, _p, _p, _p, _i64, _p, _i64, _i64, _p, _p]
    lib.kvevict_compact_inplace.argtypes = [ctypes.POINTER(KvDesc), _p, _p, _p, _i64, _p, _i32,
                                            _i32, _i64, _i32, _p, _p, _p, _p]
    for name in ("kvevict_score_random", "kvevict_score_weighted", "kvevict_select_topk",
                 "kvevict_select_topk_layers", "kvevict_layer_power_budget",
                 "kvevict_reduce_max_heads", "kvevict_score_keydiff", "kvevict_select_global",
                 "kvevict_compact", "kvevict_compact_inplace", "kvevict_evict_random_inplace",
                 "kvevict_evict_pages_random", "kvevict_select_random",
                 "kvevict_score_select_global", "kvevict_select_global_noalloc",
                 "kvevict_copy_pages", "kvevict_compact_ordered"):
        getattr(lib, name).restype = _i32
    lib.kvevict_status_string.argtypes = [_i32]
    lib.kvevict_status_string.restype = ctypes.c_char_p
    lib.kvevict_abi_version.argtypes = []
    lib.kvevict_abi_version.restype = _i32
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().kvevict_status_string(status).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, what: str):
    if st != KVEVICT_OK:
        raise KvevictError(st, what)


def _need(t, dtype, elems: int, what: str):
    """Host guard: a tensor argument lives on the GPU, has the dtype and holds `elems` elements."""
    if t is None or elems <= 0:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: tensor must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if t.numel() < elems:
        raise ValueError(f"{what}: {t.numel()} elements, need {elems}")


def _rows(count: int, ld: int, width: int) -> int:
    return 0 if count <= 0 or width <= 0 else (count - 1) * ld + width


def _store_elems(d: KvDesc, groups: int) -> int:
    if groups <= 0:
        return 0
    if d.layout == LAYOUT_CONTIG:
        return _rows(groups * d.heads, d.list_stride, d.capacity * d.head_dim)
    return d.capacity * d.page_size * d.heads * d.head_dim


def contig_desc(D: int, H: int, capacity: int, list_stride: int | None = None) -> KvDesc:
    return KvDesc(LAYOUT_CONTIG, D, H, 0, capacity,
                  capacity * D if list_stride is None else list_stride, None, 0)


def paged_desc(D: int, H: int, page_size: int, pool_pages: int, page_table) -> KvDesc:
    d = KvDesc(LAYOUT_PAGED, D, H, page_size, pool_pages, 0, _ptr(page_table),
               int(page_table.shape[1]) if page_table is not None else 1)
    d._pt = page_table  # keeps the table alive and lets the host guard check its size
    return d


def kvevict_score_random(scores, ld, num_requests, L, H, n, prot, seed, round_id, shared_draw,
                         stream=None):
    _need(scores, torch.float32, _rows(num_requests * L * (1 if shared_draw else H), ld, n), "scores")
    _check(load().kvevict_score_random(_ptr(scores), ld, num_requests, L, H, n, prot, seed,
                                       round_id, 1 if shared_draw else 0, _stream(stream)),
           "kvevict_score_random")


def kvevict_score_weighted(scores, ld, beta, vnorm, sg, st, sj, w, w_slots, win_begin, win_count,
                           L, H, G, Hg, n, prot, stream=None):
    _need(scores, torch.float32, _rows(L * H, ld, n), "scores")
    sig = (G - 1) * sg + (n - 1) * st + (Hg - 1) * sj + 1 if n > 0 else 0
    _need(beta, torch.float32, sig, "beta")
    _need(vnorm, torch.float32, sig, "vnorm")
    _need(w, torch.float32, L * H * w_slots * Hg, "w")
    if len(win_begin) != L or len(win_count) != L:
        raise ValueError("window arrays must have L entries")
    wb = (ctypes.c_int32 * L)(*[int(x) for x in win_begin])
    wc = (ctypes.c_int32 * L)(*[int(x) for x in win_count])
    _check(load().kvevict_score_weighted(_ptr(scores), ld, _ptr(beta), _ptr(vnorm), sg, st, sj,
                                         _ptr(w), w_slots, wb, wc, L, H, G, Hg, n, prot,
                                         _stream(stream)),
           "kvevict_score_weighted")


def kvevict_score_select_global(kept_idx, kept_ld, kept_count, scores, ld, beta, vnorm, sg, st, sj,
                                w, w_slots, win_begin, win_count, L, H, G, Hg, n, prot, p,
                                workspace, workspace_bytes, stream=None) -> int:
    """Weighted score + global top-B in one call (the budget B is returned)."""
    lists = L * H
    _need(scores, torch.float32, _rows(lists, ld, n), "scores")
    sig = (G - 1) * sg + (n - 1) * st + (Hg - 1) * sj + 1 if n > 0 else 0
    _need(beta, torch.float32, sig, "beta")
    _need(vnorm, torch.float32, sig, "vnorm")
    _need(w, torch.float32, L * H * w_slots * Hg, "w")
    _need(kept_idx, torch.int32, _rows(lists, kept_ld, n), "kept_idx")
    _need(kept_count, torch.int32, lists, "kept_count")
    _need(workspace, None, workspace_bytes // max(workspace.element_size(), 1), "workspace")
    if len(win_begin) != L or len(win_count) != L:
        raise ValueError("window arrays must have L entries")
    wb = (ctypes.c_int32 * L)(*[int(x) for x in win_begin])
    wc = (ctypes.c_int32 * L)(*[int(x) for x in win_count])
    budget = _i64(0)
    size = _sz(workspace_bytes)
    _check(load().kvevict_score_select_global(_ptr(kept_idx), kept_ld, _ptr(kept_count),
                                              ctypes.byref(budget), _ptr(scores), ld, _ptr(beta),
                                              _ptr(vnorm), sg, st, sj, _ptr(w), w_slots, wb, wc, L,
                                              H, G, Hg, n, prot, p, _ptr(workspace),
                                              ctypes.byref(size), _stream(stream)),
           "kvevict_score_select_global")
    return budget.value


def kvevict_select_topk(kept_idx, kept_ld, scores, ld, num_lists, n, K, prot, stream=None):
    _need(scores, torch.float32, _rows(num_lists, ld, n), "scores")
    _need(kept_idx, torch.int32, _rows(num_lists, kept_ld, K), "kept_idx")
    _check(load().kvevict_select_topk(_ptr(kept_idx), kept_ld, _ptr(scores), ld, num_lists, n, K,
                                      prot, _stream(stream)),
           "kvevict_select_topk")


def kvevict_score_keydiff(scores, ld, keys: KvDesc, k_cache, num_groups, n, prot, stream=None):
    _need(scores, torch.float32, _rows(num_groups * keys.heads, ld, n), "scores")
    _need(k_cache, torch.bfloat16, _store_elems(keys, num_groups), "k_cache")
    if keys.layout == LAYOUT_PAGED and num_groups > 0:
        _need(keys._pt, torch.int32, num_groups * keys.pt_ld, "page table")
    _check(load().kvevict_score_keydiff(_ptr(scores), ld, ctypes.byref(keys), _ptr(k_cache),
                                        num_groups, n, prot, _stream(stream)),
           "kvevict_score_keydiff")


def kvevict_select_topk_layers(kept_idx, kept_ld, kept_count, scores, ld, num_groups, L, H, n,
                               prot, layer_budget, stream=None):
    budget = [int(x) for x in layer_budget]
    if len(budget) != L:
        raise ValueError("layer_budget must have L entries")
    most = max(budget) if budget else 0
    _need(scores, torch.float32, _rows(num_groups * H, ld, n), "scores")
    _need(kept_idx, torch.int32, _rows(num_groups * H, kept_ld, prot + most), "kept_idx")
    _need(kept_count, torch.int32, num_groups * H, "kept_count")
    arr = (ctypes.c_int32 * L)(*budget)
    _check(load().kvevict_select_topk_layers(_ptr(kept_idx), kept_ld, _ptr(kept_count),
                                             _ptr(scores), ld, num_groups, L, H, n, prot, arr,
                                             _stream(stream)),
           "kvevict_select_topk_layers")


def kvevict_layer_power_budget(gate, n_body, p) -> list:
    """Host computation: per-layer kept counts per head (no GPU work)."""
    g = [float(x) for x in gate]
    L = len(g)
    garr = (ctypes.c_float * max(L, 1))(*g)
    out = (ctypes.c_int32 * max(L, 1))()
    _check(load().kvevict_layer_power_budget(garr, L, n_body, p, out),
           "kvevict_layer_power_budget")
    return [int(out[i]) for i in range(L)]


def kvevict_reduce_max_heads(shared, shared_ld, scores, ld, num_groups, H, n, stream=None):
    _need(scores, torch.float32, _rows(num_groups * H, ld, n), "scores")
    _need(shared, torch.float32, _rows(num_groups, shared_ld, n), "shared")
    _check(load().kvevict_reduce_max_heads(_ptr(shared), shared_ld, _ptr(scores), ld, num_groups,
                                           H, n, _stream(stream)),
           "kvevict_reduce_max_heads")


def kvevict_select_global_workspace(num_lists, n, prot, ld=None, kept_ld=None, p=0.0) -> int:
    size = _sz(0)
    _check(load().kvevict_select_global(None, kept_ld if kept_ld is not None else n, None, None,
                                        None, ld if ld is not None else n, num_lists, n, prot, p,
                                        None, ctypes.byref(size), None),
           "kvevict_select_global (workspace query)")
    return size.value


def kvevict_select_global(kept_idx, kept_ld, kept_count, scores, ld, num_lists, n, prot, p,
                          workspace, workspace_bytes, stream=None) -> int:
    _need(scores, torch.float32, _rows(num_lists, ld, n), "scores")
    _need(kept_idx, torch.int32, _rows(num_lists, kept_ld, n), "kept_idx")
    _need(kept_count, torch.int32, num_lists, "kept_count")
    _need(workspace, None, workspace_bytes // max(workspace.element_size(), 1), "workspace")
    budget = _i64(0)
    size = _sz(workspace_bytes)
    _check(load().kvevict_select_global(_ptr(kept_idx), kept_ld, _ptr(kept_count),
                                        ctypes.byref(budget), _ptr(scores), ld, num_lists, n, prot,
                                        p, _ptr(workspace), ctypes.byref(size), _stream(stream)),
           "kvevict_select_global")
    return budget.value


def kvevict_select_global_noalloc(kept_idx, kept_ld, kept_count, scores, ld, num_lists, n, prot,
                                  p, stream=None) -> int:
    """kvevict_select_global on the library's static workspace (no allocation)."""
    _need(scores, torch.float32, _rows(num_lists, ld, n), "scores")
    _need(kept_idx, torch.int32, _rows(num_lists, kept_ld, n), "kept_idx")
    _need(kept_count, torch.int32, num_lists, "kept_count")
    budget = _i64(0)
    _check(load().kvevict_select_global_noalloc(_ptr(kept_idx), kept_ld, _ptr(kept_count),
                                                ctypes.byref(budget), _ptr(scores), ld, num_lists,
                                                n, prot, p, _stream(stream)),
           "kvevict_select_global_noalloc")
    return budget.value


def _compact_guards(src, k_src, v_src, dst, k_dst, v_dst, kept_idx, kept_ld, kept_count, K,
                    num_groups, idx_lists_per_group, errors):
    _need(k_src, torch.bfloat16, _store_elems(src, num_groups), "k_src")
    _need(v_src, torch.bfloat16, _store_elems(src, num_groups), "v_src")
    _need(k_dst, torch.bfloat16, _store_elems(dst, num_groups), "k_dst")
    _need(v_dst, torch.bfloat16, _store_elems(dst, num_groups), "v_dst")
    idx_lists = num_groups * idx_lists_per_group
    _need(kept_idx, torch.int32, _rows(idx_lists, kept_ld, K), "kept_idx")
    _need(kept_count, torch.int32, idx_lists, "kept_count")
    _need(errors, torch.int32, 1, "errors")
    for d, what in ((src, "src"), (dst, "dst")):
        if d.layout == LAYOUT_PAGED and num_groups > 0:
            if d.page_table is None:
                raise ValueError(f"{what}: paged store without a page table")
    if src.layout == LAYOUT_PAGED and num_groups > 0:
        _need(src._pt, torch.int32, num_groups * src.pt_ld, "src page table")
    if dst.layout == LAYOUT_PAGED and num_groups > 0:
        _need(dst._pt, torch.int32, num_groups * dst.pt_ld, "dst page table")


def kvevict_compact(src: KvDesc, k_src, v_src, dst: KvDesc, k_dst, v_dst, kept_idx, kept_ld,
                    kept_count, K, num_groups, idx_lists_per_group, errors=None, stream=None):
    _compact_guards(src, k_src, v_src, dst, k_dst, v_dst, kept_idx, kept_ld, kept_count, K,
                    num_groups, idx_lists_per_group, errors)
    _check(load().kvevict_compact(ctypes.byref(src), _ptr(k_src), _ptr(v_src), ctypes.byref(dst),
                                  _ptr(k_dst), _ptr(v_dst), _ptr(kept_idx), kept_ld,
                                  _ptr(kept_count), K, num_groups, idx_lists_per_group,
                                  _ptr(errors), _stream(stream)),
           "kvevict_compact")


def kvevict_compact_ordered_workspace(dst: KvDesc) -> int:
    """Workspace bytes of kvevict_compact_ordered for this destination (0 if contiguous)."""
    size = _sz(0)
    _check(load().kvevict_compact_ordered(None, None, None, ctypes.byref(dst), None, None, None, 0,
                                          None, 0, 0, 1, None, None, ctypes.byref(size), None),
           "kvevict_compact_ordered (workspace query)")
    return size.value


def kvevict_compact_ordered(src: KvDesc, k_src, v_src, dst: KvDesc, k_dst, v_dst, kept_idx,
                            kept_ld, kept_count, K, num_groups, idx_lists_per_group, workspace,
                            workspace_bytes, errors=None, stream=None):
    _compact_guards(src, k_src, v_src, dst, k_dst, v_dst, kept_idx, kept_ld, kept_count, K,
                    num_groups, idx_lists_per_group, errors)
    _need(workspace, None, workspace_bytes // max(workspace.element_size(), 1), "workspace")
    size = _sz(workspace_bytes)
    _check(load().kvevict_compact_ordered(ctypes.byref(src), _ptr(k_src), _ptr(v_src),
                                          ctypes.byref(dst), _ptr(k_dst), _ptr(v_dst),
                                          _ptr(kept_idx), kept_ld, _ptr(kept_count), K,
                                          num_groups, idx_lists_per_group, _ptr(errors),
                                          _ptr(workspace), ctypes.byref(size), _stream(stream)),
           "kvevict_compact_ordered")


def kvevict_abi_version() -> int:
    return int(load().kvevict_abi_version())


def kvevict_copy_pages(k_src, v_src, src_ids, k_dst, v_dst, dst_ids, page_bytes, errors=None,
                       stream=None):
    """Whole pages of the K and V pools from src_ids to dst_ids (pools as flat tensors)."""
    count = int(src_ids.numel())
    for t, what in ((k_src, "k_src"), (v_src, "v_src"), (k_dst, "k_dst"), (v_dst, "v_dst")):
        _need(t, None, 1, what)
    _need(dst_ids, torch.int32, count, "dst_ids")
    _need(src_ids, torch.int32, count, "src_ids")
    src_pages = k_src.numel() * k_src.element_size() // page_bytes
    dst_pages = k_dst.numel() * k_dst.element_size() // page_bytes
    for t, pages, what in ((v_src, src_pages, "v_src"), (v_dst, dst_pages, "v_dst")):
        if t.numel() * t.element_size() < pages * page_bytes:
            raise ValueError(f"{what}: smaller than its K pool")
    _need(errors, torch.int32, 1, "errors")
    _check(load().kvevict_copy_pages(_ptr(k_src), _ptr(v_src), src_pages, _ptr(src_ids),
                                     _ptr(k_dst), _ptr(v_dst), dst_pages, _ptr(dst_ids), count,
                                     page_bytes, _ptr(errors), _stream(stream)),
           "kvevict_copy_pages")


def kvevict_compact_inplace(store: KvDesc, k, v, kept_idx, kept_ld, kept_count, K, n, num_groups,
                            idx_lists_per_group, freed_pages=None, freed_count=None, errors=None,
                            stream=None):
    _need(k, torch.bfloat16, _store_elems(store, num_groups), "k")
    _need(v, torch.bfloat16, _store_elems(store, num_groups), "v")
    idx_lists = num_groups * idx_lists_per_group
    _need(kept_idx, torch.int32, _rows(idx_lists, kept_ld, K), "kept_idx")
    _need(kept_count, torch.int32, idx_lists, "kept_count")
    _need(errors, torch.int32, 1, "errors")
    if store.layout == LAYOUT_PAGED and num_groups > 0:
        _need(store._pt, torch.int32, num_groups * store.pt_ld, "page table")
        _need(freed_pages, torch.int32, num_groups * -(-n // store.page_size), "freed_pages")
        _need(freed_count, torch.int32, 1, "freed_count")
    _check(load().kvevict_compact_inplace(ctypes.byref(store), _ptr(k), _ptr(v), _ptr(kept_idx),
                                          kept_ld, _ptr(kept_count), K, n, num_groups,
                                          idx_lists_per_group, _ptr(freed_pages),
                                          _ptr(freed_count), _ptr(errors), _stream(stream)),
           "kvevict_compact_inplace")


def kvevict_evict_random_inplace(store: KvDesc, k, v, num_requests, L, n, K, prot, seed, round_id,
                                 shared_draw, kept_idx=None, kept_ld=0, freed_pages=None,
                                 freed_count=None, errors=None, stream=None):
    num_groups = num_requests * L
    _need(k, torch.bfloat16, _store_elems(store, num_groups), "k")
    _need(v, torch.bfloat16, _store_elems(store, num_groups), "v")
    lists = num_groups * (1 if shared_draw else store.heads)
    _need(kept_idx, torch.int32, _rows(lists, kept_ld, K), "kept_idx")
    _need(errors, torch.int32, 1, "errors")
    if store.layout == LAYOUT_PAGED and num_groups > 0:
        _need(store._pt, torch.int32, num_groups * store.pt_ld, "page table")
        _need(freed_pages, torch.int32, num_groups * -(-n // store.page_size), "freed_pages")
        _need(freed_count, torch.int32, 1, "freed_count")
    _check(load().kvevict_evict_random_inplace(ctypes.byref(store), _ptr(k), _ptr(v), num_requests,
                                               L, n, K, prot, seed, round_id,
                                               1 if shared_draw else 0, _ptr(kept_idx), kept_ld,
                                               _ptr(freed_pages), _ptr(freed_count), _ptr(errors),
                                               _stream(stream)),
           "kvevict_evict_random_inplace")


def kvevict_evict_pages_random(page_table, pt_ld, page_size, num_requests, L, n, K, prot, seed,
                               round_id, kept_pages=None, kept_ld=0, freed_pages=None,
                               freed_count=None, stream=None):
    groups = num_requests * L
    P, Kp = n // page_size if page_size > 0 else 0, K // page_size if page_size > 0 else 0
    _need(page_table, torch.int32, _rows(groups, pt_ld, P), "page_table")
    _need(kept_pages, torch.int32, _rows(groups, kept_ld, Kp), "kept_pages")
    _need(freed_pages, torch.int32, groups * (P - Kp), "freed_pages")
    _need(freed_count, torch.int32, 1, "freed_count")
    _check(load().kvevict_evict_pages_random(_ptr(page_table), pt_ld, page_size, num_requests, L,
                                             n, K, prot, seed, round_id, _ptr(kept_pages), kept_ld,
                                             _ptr(freed_pages), _ptr(freed_count),
                                             _stream(stream)),
           "kvevict_evict_pages_random")


def kvevict_select_random(kept_idx, kept_ld, num_requests, L, H, n, K, prot, seed, round_id,
                          shared_draw, stream=None):
    lists = num_requests * L * (1 if shared_draw else H)
    _need(kept_idx, torch.int32, _rows(lists, kept_ld, K), "kept_idx")
    _check(load().kvevict_select_random(_ptr(kept_idx), kept_ld, num_requests, L, H, n, K, prot,
                                        seed, round_id, 1 if shared_draw else 0, _stream(stream)),
           "kvevict_select_random")
