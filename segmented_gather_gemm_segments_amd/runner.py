"""Puts a generated batch on the GPU and drives the C ABI over it.

Data movement and bookkeeping only: tensors for x, y, v and the adapter
weights (as a dense stack or in a shuffled page pool), the host segment build,
plans, and uploads.  All arithmetic of the delta runs in the library's kernels.
Used by the GPU tests, the benchmark and the smoke check.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import binding as B
from .workloads import LoraProblem


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, dtype: str, device):
    """numpy (float32, or uint16 bf16 patterns) -> torch tensor on `device`."""
    torch = _torch()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host(t, dtype: str) -> np.ndarray:
    """torch tensor -> numpy (float32, or uint16 bf16 patterns)."""
    torch = _torch()
    if dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


class DeviceProblem:
    """A LoraProblem resident on one GPU.

    layout: "dense" -- [N, r_max, d] stacks, rows r_a..r_max-1 filled with NaN;
            "paged" -- a lora_pool of 16-row pages, shuffled, unused page rows
                       NaN, A and B^T rows sharing one pool when d_in == d_out.
    Quantized rows (p.wq "fp8" / "int4") are stored as uint8 codes with fp32
    row scales; unused rows hold FP8 NaN codes (0x7f) or INT4 7s and NaN
    scales, so a stray read shows up in the results.
    """

    def __init__(self, p: LoraProblem, device="cuda", layout: Optional[str] = None,
                 page_rows: int = 16, pool_slack: float = 2.0, pool_seed: Optional[int] = None):
        torch = _torch()
        self.p = p
        self.device = torch.device(device)
        self.layout = layout or ("paged" if p.paged else "dense")
        self.tdtype = torch.bfloat16 if p.dtype == "bf16" else torch.float32
        self.cdtype = B.LORA_BF16 if p.dtype == "bf16" else B.LORA_F32
        self.wfmt = {"": B.LORA_WFMT_PLAIN, "fp8": B.LORA_WFMT_FP8_E4M3,
                     "int4": B.LORA_WFMT_INT4}[p.wq]
        assert self.wfmt == B.LORA_WFMT_PLAIN or p.dtype == "bf16"
        self.x = to_device(p.x, p.dtype, self.device)
        self.y0 = to_device(p.y, p.dtype, self.device)
        self.ids = torch.from_numpy(p.ids).to(self.device)
        self.rank = torch.from_numpy(p.ranks.astype(np.int32)).to(self.device)
        self.r_max = p.r_max
        self._pools = []
        self.w = to_device(p.extra["w"], p.dtype, self.device) if "w" in p.extra else None
        if self.layout == "dense":
            self._dense()
        else:
            self._paged(page_rows, pool_slack, p.pool_seed if pool_seed is None else pool_seed)
        self._seg = None

    # ------------------------------------------------------------- weights
    def _row_width(self, d: int) -> int:
        """Last dimension of a stored row: d elements, or its bytes when quantized."""
        return d // 2 if self.wfmt == B.LORA_WFMT_INT4 else d

    def _empty_rows(self, shape):
        torch = _torch()
        if self.wfmt == B.LORA_WFMT_PLAIN:
            return torch.full(shape, float("nan"), dtype=self.tdtype, device=self.device)
        fill = 0x7F if self.wfmt == B.LORA_WFMT_FP8_E4M3 else 0x77
        return torch.full(shape, fill, dtype=torch.uint8, device=self.device)

    def _rows_dev(self, rows):
        torch = _torch()
        if self.wfmt == B.LORA_WFMT_PLAIN:
            return to_device(rows, self.p.dtype, self.device)
        return torch.from_numpy(np.ascontiguousarray(rows, dtype=np.uint8)).to(self.device)

    def _stack(self, rows, scales, d):
        torch = _torch()
        n = len(rows)
        st = self._empty_rows((n, self.r_max, self._row_width(d)))
        sc = None
        if self.wfmt != B.LORA_WFMT_PLAIN:
            sc = torch.full((n * self.r_max,), float("nan"), dtype=torch.float32, device=self.device)
        for a, r in enumerate(rows):
            st[a, : r.shape[0]] = self._rows_dev(r)
            if sc is not None:
                sc[a * self.r_max: a * self.r_max + r.shape[0]] = torch.from_numpy(
                    np.asarray(scales[a], np.float32)).to(self.device)
        return st, sc

    def _dense(self):
        p = self.p
        self.a_pages, a_sc = self._stack(p.a_rows, p.a_scales, p.d_in)
        self.b_pages, b_sc = self._stack(p.bt_rows, p.bt_scales, p.d_out)
        self.weights = B.Weights(self.cdtype, p.d_in, p.d_out, self.r_max, self.r_max,
                                 self.a_pages, self.b_pages, self.rank, p.ranks.astype(np.int32),
                                 weight_format=self.wfmt, a_scales=a_sc, b_scales=b_sc)

    def _paged(self, page_rows, slack, seed):
        torch = _torch()
        p = self.p
        pages_a = sum((int(r) + page_rows - 1) // page_rows for r in p.ranks)
        shared = p.d_in == p.d_out
        max_pages = (self.r_max + page_rows - 1) // page_rows

        quant = self.wfmt != B.LORA_WFMT_PLAIN

        def make_pool(n_pages, d, s):
            storage = self._empty_rows((n_pages, page_rows, self._row_width(d)))
            scales = None
            if quant:
                scales = torch.full((n_pages * page_rows,), float("nan"), dtype=torch.float32,
                                    device=self.device)
            pool = B.Pool(storage, page_rows, shuffle_seed=s, weight_format=self.wfmt,
                          scales=scales)
            self._pools.append(pool)
            return pool

        def scales_dev(lst, a):
            if not quant:
                return None
            return torch.from_numpy(np.asarray(lst[a], np.float32)).to(self.device)

        if shared:
            cap = int(np.ceil(2 * pages_a * slack))
            pool_a = pool_b = make_pool(cap, p.d_in, seed * 7919 + 1)
        else:
            cap = int(np.ceil(pages_a * slack))
            pool_a = make_pool(cap, p.d_in, seed * 7919 + 1)
            pool_b = make_pool(cap, p.d_out, seed * 7919 + 2)
        a_pt = np.full((p.num_adapters, max_pages), -1, np.int32)
        b_pt = np.full((p.num_adapters, max_pages), -1, np.int32)
        for a in range(p.num_adapters):
            r = int(p.ranks[a])
            ia = pool_a.alloc(r)
            pool_a.write_rows(ia, self._rows_dev(p.a_rows[a]), scales_dev(p.a_scales, a))
            ib = pool_b.alloc(r)
            pool_b.write_rows(ib, self._rows_dev(p.bt_rows[a]), scales_dev(p.bt_scales, a))
            a_pt[a, : ia.size] = ia
            b_pt[a, : ib.size] = ib
        torch.cuda.synchronize(self.device)
        self.host_a_pt, self.host_b_pt = a_pt, b_pt
        self.a_pages, self.b_pages = pool_a.storage, pool_b.storage
        self.weights = B.Weights(self.cdtype, p.d_in, p.d_out, self.r_max, page_rows,
                                 self.a_pages, self.b_pages, self.rank, p.ranks.astype(np.int32),
                                 torch.from_numpy(a_pt).to(self.device),
                                 torch.from_numpy(b_pt).to(self.device), max_pages,
                                 weight_format=self.wfmt, a_scales=pool_a.scales,
                                 b_scales=pool_b.scales)

    def replica(self, with_base: bool = False):
        """The same batch at other device addresses: clones of x, y0 and the
        adapter rows (and row scales), with a descriptor of their own; ids,
        ranks, page tables, segments and (unless with_base) the base weight are
        shared.  Replicas let a benchmark rotate over more bytes than the
        last-level cache holds."""
        r = object.__new__(DeviceProblem)
        r.__dict__.update(self.__dict__)
        r.x = self.x.clone()
        r.y0 = self.y0.clone()
        w = self.weights
        a = w.a_pages.clone()
        b = a if w.b_pages is w.a_pages else w.b_pages.clone()
        sa = None if w.a_scales is None else w.a_scales.clone()
        sb = sa if (w.b_scales is w.a_scales) else (None if w.b_scales is None else w.b_scales.clone())
        r.a_pages, r.b_pages = a, b
        r.weights = dataclasses.replace(w, a_pages=a, b_pages=b, a_scales=sa, b_scales=sb)
        if with_base and self.w is not None:
            r.w = self.w.clone()
        r._pools = []
        return r

    # ------------------------------------------------------------- segments, plans
    def segments(self):
        if self._seg is None:
            torch = _torch()
            perm, starts, adapters = B.lora_segments_build(self.p.ids, self.p.num_adapters)
            self._seg = (perm, starts, adapters,
                         torch.from_numpy(np.ascontiguousarray(perm)).to(self.device))
        return self._seg

    def plan(self, phase: int, policy: int = B.LORA_PATH_AUTO,
             mfma_min_tokens: int = B.LORA_DEFAULT_MFMA_MIN_TOKENS, expand_tile_tokens: int = 0):
        torch = _torch()
        _, starts, adapters, _ = self.segments()
        dim = self.r_max if phase == B.LORA_PHASE_SHRINK else self.p.d_out
        items = B.lora_sgmv_plan(phase, starts, adapters, self.p.num_adapters, dim, policy,
                                 mfma_min_tokens, host_rank=self.p.ranks.astype(np.int32),
                                 expand_tile_tokens=expand_tile_tokens)
        return torch.from_numpy(np.ascontiguousarray(items)).to(self.device)

    def tiled_pays(self, tile_min_tokens: int = 0) -> bool:
        """The library's choice between the tiled and the one-launch shrink
        for this batch (lora_sgmv_tiled_pays)."""
        _, starts, adapters, _ = self.segments()
        return B.lora_sgmv_tiled_pays(starts, adapters, self.p.num_adapters, self.r_max, self.p.d_in, self.cdtype,
                                      self.wfmt, tile_min_tokens, host_rank=self.p.ranks.astype(np.int32))

    def plan_tiled(self, policy: int = B.LORA_PATH_AUTO, tile_min_tokens: int = 0, max_splits: int = 0):
        """Tiled shrink plan on the device: (items, k_splits, workspace or None)."""
        torch = _torch()
        _, starts, adapters, _ = self.segments()
        items, ks = B.lora_sgmv_plan_tiled(starts, adapters, self.p.num_adapters, self.r_max, self.p.d_in,
                                           policy, tile_min_tokens, max_splits,
                                           host_rank=self.p.ranks.astype(np.int32))
        nbytes = B.lora_sgmv_shrink_tiled_workspace(int(starts[-1]), self.r_max, ks)
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device=self.device) if nbytes else None
        return torch.from_numpy(np.ascontiguousarray(items)).to(self.device), ks, ws

    # ------------------------------------------------------------- runs
    def new_v(self):
        torch = _torch()
        return torch.zeros((self.p.num_tokens, max(self.r_max, 1)), dtype=torch.float32,
                           device=self.device)

    def run_sgmv(self, policy: int = B.LORA_PATH_AUTO,
                 mfma_min_tokens: int = B.LORA_DEFAULT_MFMA_MIN_TOKENS, y=None, v=None,
                 tiled: bool = False, tile_min_tokens: int = 0, max_splits: int = 0,
                 expand_tile_tokens: int = 0):
        """shrink then expand over the segmented batch; returns (y, v).
        tiled: the tiled shrink (its own plan, threshold and workspace);
        expand_tile_tokens: the expand plan's MFMA token tile (0: the library's)."""
        _, _, _, perm_d = self.segments()
        ep = self.plan(B.LORA_PHASE_EXPAND, policy, mfma_min_tokens, expand_tile_tokens)
        y = self.y0.clone() if y is None else y
        v = self.new_v() if v is None else v
        if tiled:
            items, ks, ws = self.plan_tiled(policy, tile_min_tokens, max_splits)
            B.lora_sgmv_shrink_tiled(self.weights, perm_d, items, ks, self.x, v, ws)
        else:
            sp = self.plan(B.LORA_PHASE_SHRINK, policy, mfma_min_tokens)
            B.lora_sgmv_shrink(self.weights, perm_d, sp, self.x, v)
        B.lora_sgmv_expand(self.weights, perm_d, ep, v, y)
        return y, v

    def run_bgmv(self, order: int = B.LORA_BGMV_AUTO, y=None, v=None):
        y = self.y0.clone() if y is None else y
        v = self.new_v() if v is None else v
        B.lora_bgmv_shrink(self.weights, self.ids, self.x, v, order)
        B.lora_bgmv_expand(self.weights, self.ids, v, y, order)
        return y, v

    def run_bgmv_fused(self, order: int = B.LORA_BGMV_AUTO, y=None, v=None, grouped: bool = False,
                       token_order=None):
        """Fused per-token delta (one launch); returns (y, v).  grouped: place
        the tokens in the batch's segment order (tokens of an adapter together);
        token_order: an explicit device placement order instead."""
        y = self.y0.clone() if y is None else y
        v = self.new_v() if v is None else v
        if grouped:
            token_order = self.segments()[3]
        B.lora_bgmv_fused(self.weights, self.ids, self.x, y, v, order, token_order=token_order)
        return y, v

    def run_base(self, y=None):
        """Base projection y = x W^T (bf16, through lora_base_gemm); returns y."""
        torch = _torch()
        assert self.w is not None, "problem has no base weight"
        if y is None:
            y = torch.empty((self.p.num_tokens, self.p.d_out), dtype=self.tdtype, device=self.device)
        B.lora_base_gemm(self.x, self.w, y, workspace=self.base_workspace())
        return y

    def base_workspace(self):
        """The split-k workspace of this problem's base GEMM (None if it does
        not split), allocated once."""
        if not hasattr(self, "_base_ws"):
            self._base_ws = B.base_gemm_workspace(self.p.num_tokens, self.p.d_out, self.p.d_in,
                                                  device=self.device)
        return self._base_ws

    def serial_calls(self, y, v, stream=None, policy: int = B.LORA_PATH_AUTO):
        """Adapter-serial comparator: one (shrink, expand) pair of prepared
        launches per segment -- each adapter's tokens as a separate sub-batch,
        through the same kernels -- instead of one launch per phase for all of
        them.  Returns the list of pairs (plans kept alive on the object)."""
        torch = _torch()
        perm, starts, adapters, perm_d = self.segments()
        ranks = self.p.ranks.astype(np.int32)
        pairs, keep = [], []
        for sgi in range(adapters.size):
            st = starts[sgi:sgi + 2]
            ad = adapters[sgi:sgi + 1]
            sp = B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, st, ad, self.p.num_adapters, self.r_max,
                                  policy, host_rank=ranks)
            ep = B.lora_sgmv_plan(B.LORA_PHASE_EXPAND, st, ad, self.p.num_adapters, self.p.d_out,
                                  policy)
            spd = torch.from_numpy(np.ascontiguousarray(sp)).to(self.device)
            epd = torch.from_numpy(np.ascontiguousarray(ep)).to(self.device)
            keep += [spd, epd]
            pairs.append(B.prepare_sgmv(self.weights, perm_d, spd, epd, self.x, v, y, stream=stream))
        self._serial_keep = keep
        return pairs
