"""fp64 CPU oracle for the multi-LoRA delta path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links, loads
or calls it, and this package imports nothing from the product package.

The arithmetic lives in ``sgmv_oracle.c`` (plain C, fp64, sequential sums,
compiled with gcc -O2 and without -ffast-math); this module only builds it and
marshals numpy arrays.  What each function computes, and the passage of the
source pages it follows, is stated beside the C function:

* ``segments``          -- group tokens by adapter (comparison sort + run-length
                           encoding).  Pinned by the worked examples in
                           ``tests/golden/`` and by property tests.
* ``shrink``            -- v = A_{a(t)} x_t.
* ``expand``            -- y_t + B_{a(t)} v_t.
* ``apply``             -- y_t + B_{a(t)} (A_{a(t)} x_t), token by token (optionally
                           with the tokens spread over OpenMP threads).
* ``apply_segmented``   -- the same, walked segment by segment.
* ``apply_sampled``     -- ``apply`` restricted to sampled (token, column) pairs.
* ``base_sampled``      -- W x at sampled (token, column) pairs.
* ``dequant_rows``      -- code * per-row scale for FP8 E4M3 / INT4 adapter rows.

Pins (tests/test_oracle_pins.py): the merge identity Wx + B(Ax) = (W + BA)x
with BA materialised by numpy, zero adapters leave y bit-unchanged, token-order
invariance, the single-adapter batch against a numpy matmul, rank-1 unit
adapters, rank splitting (linearity), exact bf16 widening of fixed bit
patterns, exact FP8 E4M3 and INT4 decoding of fixed patterns, and the worked
segment examples.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgmv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsgmv_oracle.so")

F32, BF16, F64, FP8_E4M3, INT4 = 0, 1, 2, 3, 4

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
             "-fPIC", _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, I = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    lib.oracle_widen.argtypes = [P, I, I64, P]
    lib.oracle_dequant_rows.argtypes = [P, I, P, I64, I64, P]
    lib.oracle_segments.argtypes = [P, I32, I32, P, P, P, P]
    lib.oracle_segments.restype = I
    lib.oracle_shrink.argtypes = [I32, I32, I32, P, P, P, P, I, P, I, P]
    lib.oracle_expand.argtypes = [I32, I32, I32, P, P, P, P, P, I, P, I, P]
    lib.oracle_apply.argtypes = [I32, I32, I32, P, P, P, P, I, P, P, I, P, I, P]
    lib.oracle_apply_threads.argtypes = [I32, I32, I32, P, P, P, P, I, P, P, I, P, I, P, I]
    lib.oracle_apply_threads.restype = I
    lib.oracle_apply_segmented.argtypes = [I32, I32, I32, P, P, P, I32, P, P, P, I, P, P, I, P,
                                           I, P]
    lib.oracle_base_sampled.argtypes = [I32, P, I, P, I, I32, P, P, P]
    lib.oracle_apply_sampled.argtypes = [I32, I32, P, P, P, P, I, P, P, I, I32, P, P, P, P]
    for f in ("oracle_widen", "oracle_dequant_rows", "oracle_shrink", "oracle_expand", "oracle_apply",
              "oracle_apply_segmented", "oracle_base_sampled", "oracle_apply_sampled"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    """fp32 -> 0; raw bf16 bit patterns (uint16) -> 1; fp64 -> 2."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs must be float32, uint16 (bf16 bits) or float64, got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


@dataclass
class Adapters:
    """Adapters given densely: adapter a owns rows [row_off[a], row_off[a]+rank[a])
    of ``a_rows`` ([*, d_in], rows of A) and of ``bt_rows`` ([*, d_out], rows of
    B transposed).  Element type: float32, uint16 (bf16 bits) or float64."""
    rank: np.ndarray      # int32 [N]
    row_off: np.ndarray   # int64 [N]
    a_rows: np.ndarray    # [R, d_in]
    bt_rows: np.ndarray   # [R, d_out]

    @staticmethod
    def from_stacks(a_list, bt_list) -> "Adapters":
        """Concatenate per-adapter A ([r_a, d_in]) and B^T ([r_a, d_out]) arrays."""
        rank = np.array([a.shape[0] for a in a_list], dtype=np.int32)
        off = np.zeros(len(a_list), dtype=np.int64)
        if len(a_list) > 1:
            off[1:] = np.cumsum(rank[:-1].astype(np.int64))
        return Adapters(rank, off, _c(np.concatenate(a_list, 0)), _c(np.concatenate(bt_list, 0)))

    @staticmethod
    def from_quantized(kind: str, a_codes, a_scales, bt_codes, bt_scales) -> "Adapters":
        """Per-adapter quantised rows (codes + per-row scales), dequantised
        exactly into fp64 rows."""
        a = [dequant_rows(c, kind, s) for c, s in zip(a_codes, a_scales)]
        bt = [dequant_rows(c, kind, s) for c, s in zip(bt_codes, bt_scales)]
        return Adapters.from_stacks(a, bt)

    @staticmethod
    def uniform(a: np.ndarray, bt: np.ndarray) -> "Adapters":
        """From dense stacks a [N, r, d_in], bt [N, r, d_out]."""
        n, r = a.shape[0], a.shape[1]
        return Adapters(np.full(n, r, dtype=np.int32), np.arange(n, dtype=np.int64) * r,
                        _c(a.reshape(n * r, a.shape[2])), _c(bt.reshape(n * r, bt.shape[2])))


def dequant_rows(codes: np.ndarray, kind: str, scales: np.ndarray) -> np.ndarray:
    """Dequantised adapter rows [rows, width] in fp64: code * per-row scale.
    kind "fp8" (OCP E4M3 bytes, [rows, width] uint8) or "int4" (packed nibbles,
    [rows, width // 2] uint8, even element in the low nibble)."""
    codes = _c(np.asarray(codes, dtype=np.uint8))
    scales = _c(np.asarray(scales, dtype=np.float32))
    rows = codes.shape[0]
    width = codes.shape[1] * (2 if kind == "int4" else 1)
    assert scales.shape == (rows,)
    out = np.empty((rows, width), dtype=np.float64)
    _load().oracle_dequant_rows(_p(codes), FP8_E4M3 if kind == "fp8" else INT4, _p(scales), rows,
                                width, _p(out))
    return out


def widen_codes(codes: np.ndarray, kind: str) -> np.ndarray:
    """The values of FP8 E4M3 bytes or packed INT4 nibbles, as fp64 (flat)."""
    codes = _c(np.asarray(codes, dtype=np.uint8))
    n = codes.size * (2 if kind == "int4" else 1)
    out = np.empty(n, dtype=np.float64)
    _load().oracle_widen(_p(codes), FP8_E4M3 if kind == "fp8" else INT4, n, _p(out))
    return out


def widen(a: np.ndarray) -> np.ndarray:
    a = _c(a)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_widen(_p(a), _dtype_code(a), a.size, _p(out))
    return out


def segments(ids: np.ndarray, num_adapters: int):
    """Returns (perm, starts, adapters) or raises ValueError on an out-of-range id."""
    ids = _c(np.asarray(ids, dtype=np.int32))
    t = ids.size
    perm = np.empty(max(t, 1), dtype=np.int32)
    starts = np.empty(t + 1, dtype=np.int32)
    adapters = np.empty(max(t, 1), dtype=np.int32)
    s = ctypes.c_int32(0)
    rc = _load().oracle_segments(_p(ids), t, num_adapters, _p(perm), _p(starts), _p(adapters),
                                 ctypes.byref(s))
    if rc != 0:
        raise ValueError("adapter id out of range")
    s = s.value
    return perm[: starts[s]].copy(), starts[: s + 1].copy(), adapters[:s].copy()


def _check_common(x, ids, ad: Adapters):
    ids = _c(np.asarray(ids, dtype=np.int32))
    assert ad.rank.dtype == np.int32 and ad.row_off.dtype == np.int64
    if ids.size and ids.max() >= ad.rank.size:
        raise ValueError("adapter id out of range")
    assert ad.a_rows.dtype == ad.bt_rows.dtype
    return ids


def shrink(x: np.ndarray, ids, ad: Adapters, r_max: int) -> np.ndarray:
    x = _c(x)
    ids = _check_common(x, ids, ad)
    t, d_in = x.shape
    v = np.empty((t, r_max), dtype=np.float64)
    _load().oracle_shrink(t, d_in, r_max, _p(ids), _p(ad.rank), _p(ad.row_off), _p(x),
                          _dtype_code(x), _p(ad.a_rows), _dtype_code(ad.a_rows), _p(v))
    return v


def expand(v: np.ndarray, y_in: np.ndarray, ids, ad: Adapters) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float64))
    y_in = _c(y_in)
    ids = _check_common(y_in, ids, ad)
    t, d_out = y_in.shape
    out = np.empty((t, d_out), dtype=np.float64)
    _load().oracle_expand(t, d_out, v.shape[1], _p(ids), _p(ad.rank), _p(ad.row_off), _p(v),
                          _p(ad.bt_rows), _dtype_code(ad.bt_rows), _p(y_in), _dtype_code(y_in),
                          _p(out))
    return out


def apply(x: np.ndarray, y_in: np.ndarray, ids, ad: Adapters, threads: int = 1) -> np.ndarray:
    """y_in + B(Ax) per token; threads > 1 spreads the tokens over that many
    OpenMP threads (same per-token arithmetic, bit-identical output)."""
    return apply_counted(x, y_in, ids, ad, threads)[0]


def apply_counted(x: np.ndarray, y_in: np.ndarray, ids, ad: Adapters, threads: int = 1):
    """``apply``, returning (y_out, threads that ran)."""
    x, y_in = _c(x), _c(y_in)
    ids = _check_common(x, ids, ad)
    t, d_in = x.shape
    d_out = y_in.shape[1]
    out = np.empty((t, d_out), dtype=np.float64)
    args = (t, d_in, d_out, _p(ids), _p(ad.rank), _p(ad.row_off), _p(x), _dtype_code(x),
            _p(ad.a_rows), _p(ad.bt_rows), _dtype_code(ad.a_rows), _p(y_in), _dtype_code(y_in),
            _p(out))
    if threads <= 1:
        _load().oracle_apply(*args)
        return out, 1
    used = _load().oracle_apply_threads(*args, int(threads))
    return out, int(used)


def apply_segmented(x, y_in, perm, starts, adapters, ad: Adapters) -> np.ndarray:
    x, y_in = _c(x), _c(y_in)
    perm = _c(np.asarray(perm, dtype=np.int32))
    starts = _c(np.asarray(starts, dtype=np.int32))
    adapters = _c(np.asarray(adapters, dtype=np.int32))
    t, d_in = x.shape
    d_out = y_in.shape[1]
    out = np.empty((t, d_out), dtype=np.float64)
    _load().oracle_apply_segmented(t, d_in, d_out, _p(perm), _p(starts), _p(adapters),
                                   adapters.size, _p(ad.rank), _p(ad.row_off), _p(x),
                                   _dtype_code(x), _p(ad.a_rows), _p(ad.bt_rows),
                                   _dtype_code(ad.a_rows), _p(y_in), _dtype_code(y_in), _p(out))
    return out


def apply_sampled(x, ids, ad: Adapters, d_out: int, tok, col, y_base) -> np.ndarray:
    x = _c(x)
    ids = _check_common(x, ids, ad)
    tok = _c(np.asarray(tok, dtype=np.int32))
    col = _c(np.asarray(col, dtype=np.int32))
    y_base = _c(np.asarray(y_base, dtype=np.float64))
    out = np.empty(tok.size, dtype=np.float64)
    _load().oracle_apply_sampled(x.shape[1], d_out, _p(ids), _p(ad.rank), _p(ad.row_off), _p(x),
                                 _dtype_code(x), _p(ad.a_rows), _p(ad.bt_rows),
                                 _dtype_code(ad.a_rows), tok.size, _p(tok), _p(col), _p(y_base),
                                 _p(out))
    return out


def base_sampled(x, w, tok, col) -> np.ndarray:
    x, w = _c(x), _c(w)
    tok = _c(np.asarray(tok, dtype=np.int32))
    col = _c(np.asarray(col, dtype=np.int32))
    out = np.empty(tok.size, dtype=np.float64)
    _load().oracle_base_sampled(x.shape[1], _p(x), _dtype_code(x), _p(w), _dtype_code(w),
                                tok.size, _p(tok), _p(col), _p(out))
    return out
