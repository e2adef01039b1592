"""Algorithmic byte and flop counts of the delta path (what the method must
move, each distinct item counted once), used by the benchmark's roofline.

Per adapted matrix, the adapter's own weight bytes are
``(d_in * r + r * d_out) * b`` for element size b ("Multi-LoRA serving: the
single translator with a thousand glossaries", section "The maths that
matters", bytes-per-matrix equation and the Llama-3-70B rank-16 table).

Per launch:
  shrink bytes = T_a*d_in*s + sum_{a used} r_a*d_in*s + sum_t r_{a(t)}*4
  expand bytes = sum_t r_{a(t)}*4 + sum_{a used} r_a*d_out*s + 2*T_a*d_out*s
  fused bytes  = T_a*d_in*s + sum_{a used} r_a*(d_in + d_out)*s + 2*T_a*d_out*s
  shrink flops = 2*d_in*sum_t r_{a(t)};  expand flops = 2*d_out*sum_t r_{a(t)}
where T_a counts tokens that carry an adapter, s is the activation/weight
element size and v is fp32.  With quantized adapter rows the weight terms use
the stored size w per element (1 byte for FP8 E4M3, 1/2 for INT4) plus 4 bytes
of fp32 scale per stored row: r_a*(d*w + 4) per matrix.  Token ids, segments, plans and page tables are
metadata (< 0.1 %) and are not counted.  Re-reads of an adapter's rows by
several tokens are cache traffic, not algorithmic bytes.
"""
from __future__ import annotations

import numpy as np


def adapter_matrix_bytes(d_in: int, d_out: int, r: int, elem_bytes: int = 2) -> int:
    """Bytes of one adapted matrix's A and B."""
    return (d_in * r + r * d_out) * elem_bytes


def adapter_layer_bytes(shapes, r: int, elem_bytes: int = 2) -> int:
    """Sum of ``adapter_matrix_bytes`` over (d_in, d_out) shapes of one layer."""
    return sum(adapter_matrix_bytes(di, do, r, elem_bytes) for di, do in shapes)


def _usage(ids: np.ndarray, ranks: np.ndarray):
    ids = np.asarray(ids)
    used_tok = ids[ids >= 0]
    t_a = int(used_tok.size)
    sum_r_tok = int(np.asarray(ranks, dtype=np.int64)[used_tok].sum()) if t_a else 0
    distinct = np.unique(used_tok)
    sum_r_distinct = int(np.asarray(ranks, dtype=np.int64)[distinct].sum()) if t_a else 0
    return t_a, sum_r_tok, sum_r_distinct


def _row_bytes(d: int, elem_bytes: int, wq: str) -> int:
    """Bytes of one stored adapter row of d elements, its scale included."""
    if wq == "fp8":
        return d + 4
    if wq == "int4":
        return d // 2 + 4
    return d * elem_bytes


def shrink_bytes(ids, ranks, d_in: int, elem_bytes: int, wq: str = "") -> int:
    t_a, sum_r_tok, sum_r_distinct = _usage(ids, ranks)
    return (t_a * d_in * elem_bytes + sum_r_distinct * _row_bytes(d_in, elem_bytes, wq)
            + sum_r_tok * 4)


def expand_bytes(ids, ranks, d_out: int, elem_bytes: int, wq: str = "") -> int:
    t_a, sum_r_tok, sum_r_distinct = _usage(ids, ranks)
    return (sum_r_tok * 4 + sum_r_distinct * _row_bytes(d_out, elem_bytes, wq)
            + 2 * t_a * d_out * elem_bytes)


def fused_bytes(ids, ranks, d_in: int, d_out: int, elem_bytes: int, wq: str = "") -> int:
    """One-launch delta (shrink and expand fused, v kept on chip): x, each used
    adapter's A and B rows, y read and written."""
    t_a, _, sum_r_distinct = _usage(ids, ranks)
    return (t_a * d_in * elem_bytes
            + sum_r_distinct * (_row_bytes(d_in, elem_bytes, wq) + _row_bytes(d_out, elem_bytes, wq))
            + 2 * t_a * d_out * elem_bytes)


def shrink_flops(ids, ranks, d_in: int) -> int:
    return 2 * d_in * _usage(ids, ranks)[1]


def expand_flops(ids, ranks, d_out: int) -> int:
    return 2 * d_out * _usage(ids, ranks)[1]


def base_gemm_flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k


def base_gemm_bytes(m: int, n: int, k: int, elem_bytes: int = 2) -> int:
    return (m * k + n * k + m * n) * elem_bytes
