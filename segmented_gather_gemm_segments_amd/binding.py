"""Thin ctypes binding over ``liblora_sgmv.so`` -- argument marshalling only.

Functions carry the C names of ``include/lora_sgmv.h``.  Every step of the
delta path runs in the library's kernels; PyTorch supplies device memory and
the current HIP stream.  The library must have been built
(``python -m segmented_gather_gemm_segments_amd.build``); if it is missing this
module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

LORA_OK, LORA_EINVAL, LORA_ERANGE, LORA_EUNSUPPORTED, LORA_ENOMEM, LORA_EHIP = 0, -1, -2, -3, -4, -5
LORA_F32, LORA_BF16 = 0, 1
LORA_WFMT_PLAIN, LORA_WFMT_FP8_E4M3, LORA_WFMT_INT4 = 0, 1, 2
LORA_CACHE_HOST_ONLY = 1
LORA_NO_ADAPTER = -1
LORA_MAX_RANK = 128
LORA_PHASE_SHRINK, LORA_PHASE_EXPAND = 0, 1
LORA_PATH_AUTO, LORA_PATH_GATHER, LORA_PATH_MFMA = 0, 1, 2
LORA_BGMV_AUTO, LORA_BGMV_TOKEN_MAJOR, LORA_BGMV_ADAPTER_MAJOR = 0, 1, 2
LORA_DEFAULT_MFMA_MIN_TOKENS = 16
LORA_SHRINK_GATHER_TOKENS, LORA_SHRINK_GATHER_ROWS, LORA_SHRINK_MFMA_TOKENS = 4, 4, 16
LORA_EXPAND_GATHER_TOKENS, LORA_EXPAND_MFMA_TOKENS = 4, 128
LORA_EXPAND_LONG_TILE_MIN_ITEMS = 256
LORA_EXPAND_GATHER_COLS, LORA_EXPAND_MFMA_COLS = 2048, 256
LORA_PATH_TILE = 3
LORA_SHRINK_TILE_TOKENS, LORA_SHRINK_TILE_K, LORA_SHRINK_TILE_ITEM_BYTES = 64, 64, 262144
LORA_DEFAULT_TILE_MIN_TOKENS, LORA_TILE_MIN_RANK_SHORT, LORA_MAX_K_SPLITS = 16, 32, 64
LORA_TILE_PAYS_BYTES = 24 << 20


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


class lora_item(ctypes.Structure):
    _fields_ = [("perm_begin", ctypes.c_int32), ("adapter", ctypes.c_int32),
                ("count_path", ctypes.c_int32), ("block", ctypes.c_int32)]


class lora_weights(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("num_adapters", ctypes.c_int32), ("r_max", ctypes.c_int32),
                ("page_rows", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages_a", ctypes.c_int32), ("num_pages_b", ctypes.c_int32),
                ("weight_format", ctypes.c_int32),
                ("a_pages", ctypes.c_void_p), ("b_pages", ctypes.c_void_p),
                ("rank", ctypes.c_void_p), ("a_page_table", ctypes.c_void_p),
                ("b_page_table", ctypes.c_void_p), ("host_rank", ctypes.c_void_p),
                ("a_scales", ctypes.c_void_p), ("b_scales", ctypes.c_void_p)]


class lora_cache_stats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("evictions", ctypes.c_int64), ("bytes_uploaded", ctypes.c_int64),
                ("resident", ctypes.c_int32), ("scattered", ctypes.c_int32),
                ("free_pages_a", ctypes.c_int32), ("free_pages_b", ctypes.c_int32)]


_lib = None
_P, _I32, _U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64

EXPORTS = {
    "lora_abi_version": ([], _I32),
    "lora_last_error": ([], ctypes.c_char_p),
    "lora_status_name": ([_I32], ctypes.c_char_p),
    "lora_segments_build": ([_P, _I32, _I32, _P, _P, _P, _P], _I32),
    "lora_sgmv_plan": ([_I32, _P, _P, _I32, _I32, _P, _I32, _I32, _I32, _P, _I32, _P], _I32),
    "lora_sgmv_plan_tile": ([_I32, _P, _P, _I32, _I32, _P, _I32, _I32, _I32, _I32, _P, _I32, _P], _I32),
    "lora_sgmv_shrink": ([_P, _P, _I32, _P, _I32, _I32, _P, _P, _P], _I32),
    "lora_sgmv_expand": ([_P, _P, _I32, _P, _I32, _I32, _P, _P, _P], _I32),
    "lora_sgmv_plan_tiled": ([_P, _P, _I32, _I32, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P, _P],
                             _I32),
    "lora_sgmv_shrink_tiled_workspace": ([_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int64)], _I32),
    "lora_sgmv_tiled_pays": ([_P, _P, _I32, _I32, _P, _I32, _I32, _I32, _I32, _I32, _P], _I32),
    "lora_sgmv_shrink_tiled": ([_P, _P, _I32, _P, _I32, _I32, _I32, _P, _P, _P, ctypes.c_int64, _P], _I32),
    "lora_bgmv_shrink": ([_P, _P, _I32, _I32, _P, _P, _P], _I32),
    "lora_bgmv_expand": ([_P, _P, _I32, _I32, _P, _P, _P], _I32),
    "lora_bgmv_fused": ([_P, _P, _I32, _P, _I32, _I32, _P, _P, _P, _P], _I32),
    "lora_bgmv_fused_multi": ([_P, _I32, _P, _I32, _P, _I32, _P, _P, _P, _P], _I32),
    "lora_pool_create": ([_I32, _I32, _I32, _I32, _I32, _P, _P, _U64, _P], _I32),
    "lora_pool_alloc": ([_P, _I32, _P], _I32),
    "lora_pool_free": ([_P, _P, _I32], _I32),
    "lora_pool_num_free": ([_P, _P], _I32),
    "lora_pool_write_rows": ([_P, _P, _I32, _P, _P, _P], _I32),
    "lora_pool_destroy": ([_P], None),
    "lora_pool_info": ([_P, _P, _P, _P, _P, _P], _I32),
    "lora_cache_create": ([_P, _P, _I32, _I32, _P, _P, _P, _I32, _P], _I32),
    "lora_cache_register": ([_P, _I32, _I32, _P, _P, _P, _P], _I32),
    "lora_cache_prepare": ([_P, _P, _I32, _P], _I32),
    "lora_cache_get_stats": ([_P, _P], _I32),
    "lora_cache_pages": ([_P, _I32, _P, _P, _P], _I32),
    "lora_cache_destroy": ([_P], None),
    "lora_base_gemm": ([_I32, _I32, _I32, _I32, _P, _P, _P, _P, ctypes.c_int64, _P], _I32),
    "lora_base_gemm_workspace": ([_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int64)], _I32),
    "lora_base_gemm_noalloc": ([_I32, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "lora_probe_stream_read": ([_P, ctypes.c_int64, _I32, _I32, _I32, _P, _P], _I32),
    "lora_probe_release": ([_I32, _I32, _P, _P, _P, _P], _I32),
    "lora_debug_flags": ([_P, _I32], _I32),
}
LORA_DEBUG_BAD_PAGE, LORA_DEBUG_BAD_ADAPTER, LORA_DEBUG_BAD_RANK = 1, 2, 4
LORA_DEBUG_BAD_TOKEN, LORA_DEBUG_BAD_ITEM = 8, 16


_debug = False
_loaded = {}


def lib_path() -> str:
    return _build.DEBUG_LIB if _debug else _build.LIB


def select_library(debug: bool) -> None:
    """Route every call of this module to the debug build of the library
    (kernels record bad device-side values, read by lora_debug_flags) or back
    to the release build."""
    global _debug, _lib
    _debug = bool(debug)
    _lib = None


def lib():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if path not in _loaded:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is missing: build it with "
                                   "`python -m segmented_gather_gemm_segments_amd.build`")
            h = ctypes.CDLL(path)
            for name, (args, res) in EXPORTS.items():
                f = getattr(h, name)
                f.argtypes = args
                f.restype = res
            _loaded[path] = h
        _lib = _loaded[path]
    return _lib


def lora_debug_flags(clear: bool = False) -> int:
    """The debug build's error word (LORA_DEBUG_* bits); waits for the device."""
    out = ctypes.c_uint32(0)
    _check(lib().lora_debug_flags(ctypes.byref(out), int(clear)))
    return int(out.value)


def status_name(status: int) -> str:
    return lib().lora_status_name(status).decode()


def lora_last_error() -> str:
    return lib().lora_last_error().decode()


def _check(status: int):
    if status != LORA_OK:
        raise LoraError(status, lora_last_error())


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# ---------------------------------------------------------------- host calls
def lora_segments_build(token_adapter, num_adapters: int):
    """Host segment build.  Returns (token_perm, seg_starts, seg_adapter)."""
    ids = _i32(token_adapter)
    t = ids.size
    perm = np.empty(max(t, 1), np.int32)
    starts = np.empty(t + 1, np.int32)
    adapters = np.empty(max(t, 1), np.int32)
    s = ctypes.c_int32(0)
    _check(lib().lora_segments_build(_np_ptr(ids), t, num_adapters, _np_ptr(perm), _np_ptr(starts),
                                     _np_ptr(adapters), ctypes.byref(s)))
    s = s.value
    return perm[: starts[s]].copy(), starts[: s + 1].copy(), adapters[:s].copy()


def lora_sgmv_plan(phase: int, seg_starts, seg_adapter, num_adapters: int, dim: int,
                   path_policy: int = LORA_PATH_AUTO,
                   mfma_min_tokens: int = LORA_DEFAULT_MFMA_MIN_TOKENS,
                   host_rank=None, expand_tile_tokens: int = 0) -> np.ndarray:
    """Work plan as an int32 array [num_items, 4] (perm_begin, adapter, count|path<<16, block).
    dim: r_max for a shrink plan, d_out for an expand plan.  expand_tile_tokens:
    0 = the library's width table (lora_sgmv_plan), 64 or 128 = that MFMA
    expand tile (lora_sgmv_plan_tile)."""
    starts, adapters = _i32(seg_starts), _i32(seg_adapter)
    ranks = None if host_rank is None else _i32(host_rank)
    s = adapters.size
    n = ctypes.c_int32(0)
    head = (phase, _np_ptr(starts), _np_ptr(adapters), s, num_adapters, _np_ptr(ranks), dim, path_policy,
            mfma_min_tokens)
    if expand_tile_tokens:
        call = lambda *tail: lib().lora_sgmv_plan_tile(*head, int(expand_tile_tokens), *tail)
    else:
        call = lambda *tail: lib().lora_sgmv_plan(*head, *tail)
    _check(call(None, 0, ctypes.byref(n)))
    items = np.zeros((max(n.value, 1), 4), np.int32)
    _check(call(_np_ptr(items), n.value, ctypes.byref(n)))
    return items[: n.value]


def lora_sgmv_plan_tiled(seg_starts, seg_adapter, num_adapters: int, r_max: int, d_in: int,
                         path_policy: int = LORA_PATH_AUTO, tile_min_tokens: int = 0,
                         max_splits: int = 0, host_rank=None):
    """Tiled shrink plan: (int32 items [num_items, 4], k_splits)."""
    starts, adapters = _i32(seg_starts), _i32(seg_adapter)
    ranks = None if host_rank is None else _i32(host_rank)
    n, ks = ctypes.c_int32(0), ctypes.c_int32(0)
    args = (_np_ptr(starts), _np_ptr(adapters), adapters.size, num_adapters, _np_ptr(ranks), r_max, d_in,
            path_policy, tile_min_tokens, max_splits)
    _check(lib().lora_sgmv_plan_tiled(*args, None, 0, ctypes.byref(n), ctypes.byref(ks)))
    items = np.zeros((max(n.value, 1), 4), np.int32)
    _check(lib().lora_sgmv_plan_tiled(*args, _np_ptr(items), n.value, ctypes.byref(n), ctypes.byref(ks)))
    return items[: n.value], int(ks.value)


def lora_sgmv_tiled_pays(seg_starts, seg_adapter, num_adapters: int, r_max: int, d_in: int, dtype: int,
                         weight_format: int = LORA_WFMT_PLAIN, tile_min_tokens: int = 0, host_rank=None) -> bool:
    """Whether the library prefers the tiled shrink for this batch."""
    starts, adapters = _i32(seg_starts), _i32(seg_adapter)
    ranks = None if host_rank is None else _i32(host_rank)
    out = ctypes.c_int32(0)
    _check(lib().lora_sgmv_tiled_pays(_np_ptr(starts), _np_ptr(adapters), adapters.size, num_adapters,
                                      _np_ptr(ranks), r_max, d_in, dtype, weight_format, tile_min_tokens,
                                      ctypes.byref(out)))
    return bool(out.value)


def lora_sgmv_shrink_tiled_workspace(num_perm: int, r_max: int, k_splits: int) -> int:
    out = ctypes.c_int64(0)
    _check(lib().lora_sgmv_shrink_tiled_workspace(num_perm, r_max, k_splits, ctypes.byref(out)))
    return int(out.value)


# ---------------------------------------------------------------- device helpers
def _torch():
    import torch
    return torch


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Weights:
    """Device-resident adapter weights plus the lora_weights descriptor.

    ``a_pages`` [num_pages_a, page_rows, ...] and ``b_pages`` [num_pages_b,
    page_rows, ...] are torch tensors: bf16 or fp32 rows of d_in / d_out
    elements, or, for a quantized ``weight_format``, uint8 rows of the stored
    codes with fp32 row scales ``a_scales`` [num_pages_a * page_rows] and
    ``b_scales``; ``rank`` int32 [N] on device; page tables int32 [N,
    max_pages] on device or None (dense stack: page a = adapter a)."""
    dtype: int
    d_in: int
    d_out: int
    r_max: int
    page_rows: int
    a_pages: object
    b_pages: object
    rank: object
    host_rank: np.ndarray
    a_page_table: object = None
    b_page_table: object = None
    max_pages: int = 1
    weight_format: int = LORA_WFMT_PLAIN
    a_scales: object = None
    b_scales: object = None

    @property
    def num_adapters(self) -> int:
        return int(self.host_rank.size)

    def desc(self) -> lora_weights:
        self._host_rank_c = _i32(self.host_rank)
        hr = self._host_rank_c.ctypes.data if getattr(self, "host_rank_valid", True) else None
        return lora_weights(
            self.dtype, self.d_in, self.d_out, self.num_adapters, self.r_max, self.page_rows,
            self.max_pages, int(self.a_pages.shape[0]), int(self.b_pages.shape[0]),
            self.weight_format, _dptr(self.a_pages), _dptr(self.b_pages), _dptr(self.rank),
            _dptr(self.a_page_table), _dptr(self.b_page_table), hr,
            _dptr(self.a_scales), _dptr(self.b_scales))


def lora_sgmv_shrink(w: Weights, token_perm, items, x, v, num_tokens: Optional[int] = None,
                     stream=None):
    d = w.desc()
    n_tok = x.shape[0] if num_tokens is None else num_tokens
    _check(lib().lora_sgmv_shrink(ctypes.byref(d), _dptr(token_perm), int(token_perm.numel()),
                                  _dptr(items), int(items.shape[0]), n_tok, _dptr(x), _dptr(v),
                                  _stream(stream)))


def lora_sgmv_expand(w: Weights, token_perm, items, v, y, num_tokens: Optional[int] = None,
                     stream=None):
    d = w.desc()
    n_tok = y.shape[0] if num_tokens is None else num_tokens
    _check(lib().lora_sgmv_expand(ctypes.byref(d), _dptr(token_perm), int(token_perm.numel()),
                                  _dptr(items), int(items.shape[0]), n_tok, _dptr(v), _dptr(y),
                                  _stream(stream)))


def _ws_args(workspace):
    return (_dptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size())


def lora_sgmv_shrink_tiled(w: Weights, token_perm, items, k_splits: int, x, v, workspace=None,
                           num_tokens: Optional[int] = None, stream=None):
    d = w.desc()
    n = int(x.shape[0]) if num_tokens is None else num_tokens
    wp, wb = _ws_args(workspace)
    _check(lib().lora_sgmv_shrink_tiled(ctypes.byref(d), _dptr(token_perm), int(token_perm.numel()),
                                        _dptr(items), int(items.shape[0]), n, int(k_splits), _dptr(x),
                                        _dptr(v), wp, wb, _stream(stream)))


def lora_bgmv_shrink(w: Weights, token_adapter, x, v, order: int = LORA_BGMV_AUTO, stream=None):
    d = w.desc()
    _check(lib().lora_bgmv_shrink(ctypes.byref(d), _dptr(token_adapter), int(token_adapter.numel()),
                                  order, _dptr(x), _dptr(v), _stream(stream)))


def lora_bgmv_expand(w: Weights, token_adapter, v, y, order: int = LORA_BGMV_AUTO, stream=None):
    d = w.desc()
    _check(lib().lora_bgmv_expand(ctypes.byref(d), _dptr(token_adapter), int(token_adapter.numel()),
                                  order, _dptr(v), _dptr(y), _stream(stream)))


def lora_bgmv_fused(w: Weights, token_adapter, x, y, v=None, order: int = LORA_BGMV_AUTO,
                    stream=None, token_order=None):
    """token_order: optional device int32 placement order (e.g. the segment
    permutation of the batch)."""
    d = w.desc()
    n_ord = 0 if token_order is None else int(token_order.numel())
    _check(lib().lora_bgmv_fused(ctypes.byref(d), _dptr(token_adapter), int(token_adapter.numel()),
                                 _dptr(token_order), n_ord, order, _dptr(x), _dptr(v), _dptr(y),
                                 _stream(stream)))


def _multi_args(ws, ys, vs):
    descs = [w.desc() for w in ws]
    n = len(descs)
    warr = (ctypes.POINTER(lora_weights) * n)(*[ctypes.pointer(d) for d in descs])
    yarr = (ctypes.c_void_p * n)(*[_dptr(y) for y in ys])
    varr = None if vs is None else (ctypes.c_void_p * n)(*[_dptr(v) for v in vs])
    return descs, warr, yarr, varr


def lora_bgmv_fused_multi(ws, token_adapter, x, ys, vs=None, stream=None, token_order=None):
    """Fused per-token deltas of several projections sharing x, one launch."""
    descs, warr, yarr, varr = _multi_args(ws, ys, vs)
    n_ord = 0 if token_order is None else int(token_order.numel())
    _check(lib().lora_bgmv_fused_multi(warr, len(ws), _dptr(token_adapter), int(token_adapter.numel()),
                                       _dptr(token_order), n_ord, _dptr(x), varr, yarr,
                                       _stream(stream)))


def prepare_bgmv_fused_multi(ws, token_adapter, x, ys, vs=None, stream=None, token_order=None):
    descs, warr, yarr, varr = _multi_args(ws, ys, vs)
    n_ord = 0 if token_order is None else int(token_order.numel())
    keep = (descs, warr, yarr, varr, ws, token_adapter, x, ys, vs, token_order)
    return Prepared("lora_bgmv_fused_multi", (warr, len(ws), _dptr(token_adapter),
                                              int(token_adapter.numel()), _dptr(token_order), n_ord,
                                              _dptr(x), varr, yarr, _stream(stream)), keep)


def base_gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    """Workspace bytes with which lora_base_gemm splits k (0: no split)."""
    out = ctypes.c_int64(0)
    _check(lib().lora_base_gemm_workspace(m, n, k, ctypes.byref(out)))
    return int(out.value)


def base_gemm_workspace(m: int, n: int, k: int, device="cuda"):
    """A workspace tensor for lora_base_gemm on this shape, or None."""
    nbytes = base_gemm_workspace_bytes(m, n, k)
    if nbytes == 0:
        return None
    return _torch().empty((nbytes + 3) // 4, dtype=_torch().float32, device=device)


def _ws(workspace):
    return (_dptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size())


def lora_base_gemm(x, w, y, workspace=None, stream=None):
    m, k = x.shape
    n = w.shape[0]
    wp, wb = _ws(workspace)
    _check(lib().lora_base_gemm(LORA_BF16, m, n, k, _dptr(x), _dptr(w), _dptr(y), wp, wb,
                                _stream(stream)))


def lora_base_gemm_noalloc(x, w, y, stream=None):
    """lora_base_gemm without a workspace argument: split-k partials go to the
    library's own device scratch (allocates nothing)."""
    m, k = x.shape
    n = w.shape[0]
    _check(lib().lora_base_gemm_noalloc(LORA_BF16, m, n, k, _dptr(x), _dptr(w), _dptr(y),
                                        _stream(stream)))


class Pool:
    """lora_pool over caller-owned device storage: a torch tensor [num_pages,
    page_rows, row_width] of bf16 or fp32, or for a quantized weight_format a
    uint8 tensor [num_pages, page_rows, row_bytes] with fp32 row scales
    ``scales`` [num_pages * page_rows]."""

    def __init__(self, storage, page_rows: int, shuffle_seed: int = 0,
                 weight_format: int = LORA_WFMT_PLAIN, scales=None):
        self.storage = storage
        self.scales = scales
        num_pages, pr, width = storage.shape
        assert pr == page_rows
        torch = _torch()
        if weight_format == LORA_WFMT_PLAIN:
            dtype = LORA_BF16 if storage.dtype == torch.bfloat16 else LORA_F32
        else:
            dtype = LORA_BF16
            width = width * 2 if weight_format == LORA_WFMT_INT4 else width
        self.page_rows = page_rows
        h = ctypes.c_void_p()
        _check(lib().lora_pool_create(num_pages, page_rows, width, dtype, weight_format,
                                      _dptr(storage), _dptr(scales), shuffle_seed,
                                      ctypes.byref(h)))
        self._h = h

    def alloc(self, rows: int) -> np.ndarray:
        ids = np.empty((rows + self.page_rows - 1) // self.page_rows, np.int32)
        _check(lib().lora_pool_alloc(self._h, rows, _np_ptr(ids)))
        return ids

    def free(self, page_ids):
        ids = _i32(page_ids)
        _check(lib().lora_pool_free(self._h, _np_ptr(ids), ids.size))

    def num_free(self) -> int:
        n = ctypes.c_int32(0)
        _check(lib().lora_pool_num_free(self._h, ctypes.byref(n)))
        return n.value

    def write_rows(self, page_ids, src, src_scales=None, stream=None):
        """src: torch tensor [rows, row] on device (or pinned host); src_scales
        fp32 [rows] for a quantized pool."""
        ids = _i32(page_ids)
        _check(lib().lora_pool_write_rows(self._h, _np_ptr(ids), int(src.shape[0]), _dptr(src),
                                          _dptr(src_scales), _stream(stream)))

    def close(self):
        if self._h:
            lib().lora_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Cache:
    """lora_cache: LRU residency of adapters (ids 0..num_ids-1) in two pools,
    owning the device page tables and ranks (torch int32 tensors it is given,
    or none in host-only mode).  ``weights(dtype, d_in, d_out)`` is the
    descriptor the kernels read through it."""

    def __init__(self, pool_a: Pool, pool_b: Pool, num_ids: int, r_max: int, page_table_a=None,
                 page_table_b=None, rank=None, host_only: bool = False):
        self.pool_a, self.pool_b = pool_a, pool_b
        self.num_ids, self.r_max = num_ids, r_max
        self.page_rows = pool_a.page_rows
        self.max_pages = (r_max + self.page_rows - 1) // self.page_rows
        self.pt_a, self.pt_b, self.rank = page_table_a, page_table_b, rank
        self._keep = {}
        h = ctypes.c_void_p()
        _check(lib().lora_cache_create(pool_a._h, pool_b._h, num_ids, r_max, _dptr(page_table_a),
                                       _dptr(page_table_b), _dptr(rank),
                                       LORA_CACHE_HOST_ONLY if host_only else 0, ctypes.byref(h)))
        self._h = h

    def register(self, id_: int, rank: int, rows_a, rows_b, scales_a=None, scales_b=None):
        """Host rows (numpy or torch CPU, ideally pinned) kept alive by the cache."""
        self._keep[id_] = (rows_a, rows_b, scales_a, scales_b)
        ptr = lambda t: None if t is None else (t.ctypes.data if isinstance(t, np.ndarray) else t.data_ptr())
        _check(lib().lora_cache_register(self._h, id_, rank, ptr(rows_a), ptr(rows_b), ptr(scales_a),
                                         ptr(scales_b)))

    def prepare(self, ids, stream=None, host_only: bool = False):
        a = _i32(ids)
        s = None if host_only else _stream(stream)
        _check(lib().lora_cache_prepare(self._h, _np_ptr(a), a.size, s))

    def stats(self) -> dict:
        st = lora_cache_stats()
        _check(lib().lora_cache_get_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in lora_cache_stats._fields_}

    def pages(self, id_: int):
        pa = np.empty(self.max_pages, np.int32)
        pb = np.empty(self.max_pages, np.int32)
        n = ctypes.c_int32(0)
        _check(lib().lora_cache_pages(self._h, id_, _np_ptr(pa), _np_ptr(pb), ctypes.byref(n)))
        return pa[: n.value].copy(), pb[: n.value].copy()

    def weights(self, dtype: int, d_in: int, d_out: int, weight_format: int = LORA_WFMT_PLAIN) -> "Weights":
        w = Weights(dtype, d_in, d_out, self.r_max, self.page_rows, self.pool_a.storage,
                    self.pool_b.storage, self.rank, np.ones(self.num_ids, np.int32), self.pt_a,
                    self.pt_b, self.max_pages, weight_format, self.pool_a.scales, self.pool_b.scales)
        w.host_rank_valid = False
        return w

    def close(self):
        if self._h:
            lib().lora_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prepare_probe_stream_read(src, bytes_per_group: int, groups: int, threads: int, sink, stream=None,
                              nontemporal: bool = False):
    """Prepared bare streaming read (a measurement floor, not the delta path);
    nontemporal: loads with the non-temporal hint."""
    assert src.numel() * src.element_size() >= bytes_per_group * groups
    assert sink.numel() * sink.element_size() >= 4 * groups
    return Prepared("lora_probe_stream_read", (_dptr(src), int(bytes_per_group), int(groups), int(threads),
                                               int(bool(nontemporal)), _dptr(sink), _stream(stream)), (src, sink))


def prepare_probe_release(pairs: int, fence: bool, part, counters, out, stream=None):
    """Prepared release-per-workgroup probe (a measurement, not the delta path);
    counters must start at zero (every call leaves them zero)."""
    assert part.numel() * part.element_size() >= 2 * pairs * 64 * 4
    assert out.numel() * out.element_size() >= pairs * 64 * 4
    assert counters.numel() * counters.element_size() >= pairs * 4
    return Prepared("lora_probe_release", (int(pairs), int(bool(fence)), _dptr(part), _dptr(counters), _dptr(out),
                                           _stream(stream)), (part, counters, out))


# ---------------------------------------------------------------- prepared launches
class Prepared:
    """A device call with its ctypes arguments marshalled once; calling it only
    enqueues the launch (for launch-bound loops and graph capture).  Keeps the
    descriptor and every tensor it points to alive."""

    def __init__(self, fn_name: str, args: tuple, keep: tuple):
        self._fn = getattr(lib(), fn_name)
        self._args = args
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))


def prepare_bgmv(w: Weights, token_adapter, x, v, y, order: int = LORA_BGMV_AUTO, stream=None):
    """(shrink, expand) prepared BGMV launches on `stream` (default: current)."""
    d = w.desc()
    s = _stream(stream)
    n = int(token_adapter.numel())
    keep = (d, w, token_adapter, x, v, y)
    shrink = Prepared("lora_bgmv_shrink", (ctypes.byref(d), _dptr(token_adapter), n, order, _dptr(x),
                                           _dptr(v), s), keep)
    expand = Prepared("lora_bgmv_expand", (ctypes.byref(d), _dptr(token_adapter), n, order, _dptr(v),
                                           _dptr(y), s), keep)
    return shrink, expand


def prepare_sgmv(w: Weights, token_perm, shrink_items, expand_items, x, v, y, stream=None):
    """(shrink, expand) prepared SGMV launches on `stream` (default: current)."""
    d = w.desc()
    s = _stream(stream)
    keep = (d, w, token_perm, shrink_items, expand_items, x, v, y)
    npm = int(token_perm.numel())
    shrink = Prepared("lora_sgmv_shrink", (ctypes.byref(d), _dptr(token_perm), npm, _dptr(shrink_items),
                                           int(shrink_items.shape[0]), int(x.shape[0]), _dptr(x),
                                           _dptr(v), s), keep)
    expand = Prepared("lora_sgmv_expand", (ctypes.byref(d), _dptr(token_perm), npm, _dptr(expand_items),
                                           int(expand_items.shape[0]), int(y.shape[0]), _dptr(v),
                                           _dptr(y), s), keep)
    return shrink, expand


def prepare_sgmv_tiled(w: Weights, token_perm, tile_items, k_splits: int, workspace, expand_items, x, v, y,
                       stream=None):
    """(shrink, expand) prepared launches: the tiled shrink (with its reduce
    launch when k_splits > 1) and the segmented expand, on `stream`."""
    d = w.desc()
    s = _stream(stream)
    keep = (d, w, token_perm, tile_items, expand_items, x, v, y, workspace)
    npm = int(token_perm.numel())
    wp, wb = _ws_args(workspace)
    shrink = Prepared("lora_sgmv_shrink_tiled", (ctypes.byref(d), _dptr(token_perm), npm, _dptr(tile_items),
                                                 int(tile_items.shape[0]), int(x.shape[0]), int(k_splits),
                                                 _dptr(x), _dptr(v), wp, wb, s), keep)
    expand = Prepared("lora_sgmv_expand", (ctypes.byref(d), _dptr(token_perm), npm, _dptr(expand_items),
                                           int(expand_items.shape[0]), int(y.shape[0]), _dptr(v),
                                           _dptr(y), s), keep)
    return shrink, expand


def prepare_base_gemm(x, w, y, workspace=None, stream=None):
    """Prepared lora_base_gemm launch y = x w^T on `stream` (default: current)."""
    m, k = x.shape
    n = w.shape[0]
    wp, wb = _ws(workspace)
    return Prepared("lora_base_gemm", (LORA_BF16, m, n, k, _dptr(x), _dptr(w), _dptr(y), wp, wb,
                                       _stream(stream)), (x, w, y, workspace))


def prepare_bgmv_fused(w: Weights, token_adapter, x, y, v=None, order: int = LORA_BGMV_AUTO,
                       stream=None, token_order=None):
    """Prepared fused BGMV launch (shrink + expand in one kernel) on `stream`."""
    d = w.desc()
    keep = (d, w, token_adapter, x, v, y, token_order)
    n_ord = 0 if token_order is None else int(token_order.numel())
    return Prepared("lora_bgmv_fused", (ctypes.byref(d), _dptr(token_adapter),
                                        int(token_adapter.numel()), _dptr(token_order), n_ord,
                                        order, _dptr(x), _dptr(v), _dptr(y), _stream(stream)), keep)
