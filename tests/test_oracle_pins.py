"""Pins for the fp64 oracle: checks against what the pages and mathematics fix,
independent of the oracle's own formula (numpy matmuls on materialised
matrices, closed forms, invariants, worked examples).  CPU only."""
import math

import numpy as np
import pytest

import oracle
from conftest import golden_path, read_golden_examples
from segmented_gather_gemm_segments_amd import workloads as wl


def _rand_adapters(rng, ranks, d_in, d_out, dtype=np.float64):
    a = [rng.standard_normal((r, d_in)).astype(dtype) for r in ranks]
    bt = [rng.standard_normal((r, d_out)).astype(dtype) for r in ranks]
    return oracle.Adapters.from_stacks(a, bt), a, bt


# ------------------------------------------------------------------ widening
def test_bf16_widening_matches_format_definition():
    """bf16 = top half of binary32: patterns from tests/golden/bf16_patterns.txt,
    and the sign/exponent/fraction formula for every normal pattern."""
    bits, vals = [], []
    for line in open(golden_path("bf16_patterns.txt")):
        if line.startswith("#") or not line.strip():
            continue
        h, v = line.split()
        bits.append(int(h, 16))
        vals.append(float(v))
    got = oracle.widen(np.array(bits, dtype=np.uint16))
    for b, want, g in zip(bits, vals, got):
        assert g == want and math.copysign(1, g) == math.copysign(1, want), hex(b)
    allbits = np.arange(1 << 16, dtype=np.uint32)
    e = (allbits >> 7) & 0xFF
    normal = (e > 0) & (e < 255)
    b = allbits[normal]
    s = np.where(b >> 15, -1.0, 1.0)
    f = (b & 0x7F).astype(np.float64)
    expect = s * np.ldexp(1.0 + f / 128.0, (((b >> 7) & 0xFF).astype(np.int64) - 127))
    assert np.array_equal(oracle.widen(b.astype(np.uint16)), expect)


# ------------------------------------------------------------------ P1 merge identity
@pytest.mark.parametrize("dtype", [np.float64, np.float32, "bf16"])
def test_merge_identity(dtype):
    """W x + B(A x) == (W + B A) x with BA materialised (the two equations of
    the section 'The bare mechanism'), A in R^{r x d_in}, B in R^{d_out x r}."""
    rng = np.random.default_rng(11)
    t, d_in, d_out, r = 5, 7, 6, 3
    w = rng.standard_normal((d_out, d_in))
    a = rng.standard_normal((r, d_in))
    b = rng.standard_normal((d_out, r))
    x = rng.standard_normal((t, d_in))
    if dtype == "bf16":
        cast = lambda m: wl.bf16_bits(m.astype(np.float32))
        back = lambda m: wl.bf16_to_f32(m).astype(np.float64)
    else:
        cast = lambda m: m.astype(dtype)
        back = lambda m: m.astype(np.float64)
    a_c, bt_c, x_c = cast(a), cast(np.ascontiguousarray(b.T)), cast(x)
    a64, b64, x64 = back(a_c), back(bt_c).T, back(x_c)
    y_in = x64 @ w.T                                  # base term, fp64
    ad = oracle.Adapters.from_stacks([a_c], [bt_c])
    got = oracle.apply(x_c, y_in, np.zeros(t, np.int32), ad)
    merged = w + b64 @ a64                            # W' = W + BA, materialised
    want = x64 @ merged.T
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


# ------------------------------------------------------------------ P2 zero adapter
@pytest.mark.parametrize("which", ["A", "B"])
def test_zero_adapter_leaves_y_bit_unchanged(which):
    rng = np.random.default_rng(3)
    t, d_in, d_out, r = 9, 40, 24, 8
    x = wl.bf16_bits(rng.standard_normal((t, d_in)).astype(np.float32))
    y = wl.bf16_bits(rng.standard_normal((t, d_out)).astype(np.float32))
    a = wl.bf16_bits(rng.standard_normal((r, d_in)).astype(np.float32))
    bt = wl.bf16_bits(rng.standard_normal((r, d_out)).astype(np.float32))
    if which == "A":
        a[:] = 0
    else:
        bt[:] = 0
    out = oracle.apply(x, y, np.zeros(t, np.int32), oracle.Adapters.from_stacks([a], [bt]))
    assert np.array_equal(out, wl.bf16_to_f32(y).astype(np.float64))


def test_no_adapter_tokens_unchanged():
    rng = np.random.default_rng(4)
    ad, _, _ = _rand_adapters(rng, [4, 4], 10, 12)
    x = rng.standard_normal((6, 10))
    y = rng.standard_normal((6, 12))
    ids = np.array([-1, 0, -1, 1, 1, -1], np.int32)
    out = oracle.apply(x, y, ids, ad)
    assert np.array_equal(out[ids < 0], y[ids < 0])
    assert not np.array_equal(out[ids >= 0], y[ids >= 0])


# ------------------------------------------------------------------ P3 token order
def test_token_order_invariance():
    rng = np.random.default_rng(5)
    ranks = [3, 5, 2, 4]
    ad, _, _ = _rand_adapters(rng, ranks, 17, 13)
    t = 31
    ids = rng.integers(-1, len(ranks), size=t).astype(np.int32)
    x = rng.standard_normal((t, 17))
    y = rng.standard_normal((t, 13))
    base = oracle.apply(x, y, ids, ad)
    for _ in range(3):
        p = rng.permutation(t)
        out = oracle.apply(x[p], y[p], ids[p], ad)
        assert np.array_equal(out, base[p])


# ------------------------------------------------------------------ P4 special cases
def test_single_adapter_batch_is_one_matmul():
    """All tokens on one adapter: the delta is Y + (X A^T) B^T... i.e. one dense
    product, computed here with numpy's matmul on the materialised matrices."""
    rng = np.random.default_rng(6)
    t, d_in, d_out, r = 40, 64, 48, 16
    ad, a, bt = _rand_adapters(rng, [r], d_in, d_out)
    x = rng.standard_normal((t, d_in))
    y = rng.standard_normal((t, d_out))
    got = oracle.apply(x, y, np.zeros(t, np.int32), ad)
    want = y + (x @ a[0].T) @ bt[0]
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_mixed_ranks_against_numpy_per_token():
    rng = np.random.default_rng(7)
    ranks = [8, 16, 32, 64, 1]
    d_in, d_out, t = 96, 80, 50
    ad, a, bt = _rand_adapters(rng, ranks, d_in, d_out)
    ids = rng.integers(-1, len(ranks), size=t).astype(np.int32)
    x = rng.standard_normal((t, d_in))
    y = rng.standard_normal((t, d_out))
    got = oracle.apply(x, y, ids, ad)
    want = y.copy()
    for i in range(len(ranks)):
        m = ids == i
        want[m] += (x[m] @ a[i].T) @ bt[i]
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_threaded_apply_is_bit_identical_and_pinned():
    """The all-cores leg (tokens spread over OpenMP threads) gives the same bits
    as the one-thread oracle, reports the threads that ran, and is pinned to
    per-adapter numpy products like the one-thread oracle."""
    rng = np.random.default_rng(17)
    ranks = [8, 16, 32, 64, 3]
    d_in, d_out, t = 120, 88, 203
    ad, a, bt = _rand_adapters(rng, ranks, d_in, d_out)
    ids = rng.integers(-1, len(ranks), size=t).astype(np.int32)
    x = rng.standard_normal((t, d_in))
    y = rng.standard_normal((t, d_out))
    one = oracle.apply(x, y, ids, ad)
    many, used = oracle.apply_counted(x, y, ids, ad, threads=4)
    assert used == 4
    assert np.array_equal(one, many)
    want = y.copy()
    for i in range(len(ranks)):
        m = ids == i
        want[m] += (x[m] @ a[i].T) @ bt[i]
    assert np.max(np.abs(many - want)) <= 1e-12 * np.max(np.abs(want))


def test_rank1_unit_adapter_is_exact_copy():
    """A = e_k^T and B = e_i: the delta at (t, i) is exactly x[t, k], zero elsewhere."""
    rng = np.random.default_rng(8)
    d_in, d_out, t, k, i = 12, 9, 5, 7, 4
    a = np.zeros((1, d_in), np.float32)
    a[0, k] = 1
    bt = np.zeros((1, d_out), np.float32)
    bt[0, i] = 1
    x = rng.standard_normal((t, d_in)).astype(np.float32)
    y = np.zeros((t, d_out), np.float32)
    out = oracle.apply(x, y, np.zeros(t, np.int32), oracle.Adapters.from_stacks([a], [bt]))
    want = np.zeros((t, d_out))
    want[:, i] = x[:, k]
    assert np.array_equal(out, want)


def test_rank_split_linearity():
    """A rank-2r adapter equals its two rank-r halves applied one after the other."""
    rng = np.random.default_rng(9)
    d_in, d_out, t, r = 33, 21, 7, 4
    a = rng.standard_normal((2 * r, d_in))
    bt = rng.standard_normal((2 * r, d_out))
    x = rng.standard_normal((t, d_in))
    y = rng.standard_normal((t, d_out))
    ids = np.zeros(t, np.int32)
    full = oracle.apply(x, y, ids, oracle.Adapters.from_stacks([a], [bt]))
    half = oracle.apply(x, y, ids, oracle.Adapters.from_stacks([a[:r]], [bt[:r]]))
    both = oracle.apply(x, half, ids, oracle.Adapters.from_stacks([a[r:]], [bt[r:]]))
    assert np.max(np.abs(full - both)) <= 1e-12 * np.max(np.abs(full))


def test_phases_compose_to_apply():
    """shrink then expand (the two phases of the SGMV section) equals the whole
    delta; and shrink alone equals A x by numpy."""
    rng = np.random.default_rng(10)
    ranks = [8, 16, 4]
    ad, a, bt = _rand_adapters(rng, ranks, 50, 30)
    t = 20
    ids = rng.integers(-1, 3, size=t).astype(np.int32)
    x = rng.standard_normal((t, 50))
    y = rng.standard_normal((t, 30))
    v = oracle.shrink(x, ids, ad, 16)
    for tt in range(t):
        if ids[tt] >= 0:
            r = ranks[ids[tt]]
            assert np.allclose(v[tt, :r], a[ids[tt]] @ x[tt], rtol=0, atol=1e-12)
            assert np.all(v[tt, r:] == 0)
    assert np.array_equal(oracle.expand(v, y, ids, ad), oracle.apply(x, y, ids, ad))


def test_segmented_walk_equals_token_walk():
    rng = np.random.default_rng(12)
    ranks = [2, 6, 3, 5, 4]
    ad, _, _ = _rand_adapters(rng, ranks, 19, 11)
    t = 40
    ids = rng.integers(-1, 5, size=t).astype(np.int32)
    x = rng.standard_normal((t, 19))
    y = rng.standard_normal((t, 11))
    perm, starts, adapters = oracle.segments(ids, 5)
    assert np.array_equal(oracle.apply_segmented(x, y, perm, starts, adapters, ad),
                          oracle.apply(x, y, ids, ad))


def test_sampled_equals_full():
    rng = np.random.default_rng(13)
    ad, _, _ = _rand_adapters(rng, [4, 8], 24, 16, np.float32)
    t = 10
    ids = np.array([0, 1, -1, 1, 0, 0, 1, -1, 0, 1], np.int32)
    x = rng.standard_normal((t, 24)).astype(np.float32)
    y = rng.standard_normal((t, 16)).astype(np.float32)
    full = oracle.apply(x, y, ids, ad)
    tok = rng.integers(0, t, 25)
    col = rng.integers(0, 16, 25)
    got = oracle.apply_sampled(x, ids, ad, 16, tok, col, y[tok, col].astype(np.float64))
    assert np.array_equal(got, full[tok, col])


def test_base_sampled():
    rng = np.random.default_rng(14)
    x = wl.bf16_bits(rng.standard_normal((6, 40)).astype(np.float32))
    w = wl.bf16_bits(rng.standard_normal((30, 40)).astype(np.float32))
    tok = rng.integers(0, 6, 50)
    col = rng.integers(0, 30, 50)
    got = oracle.base_sampled(x, w, tok, col)
    want = (wl.bf16_to_f32(x).astype(np.float64) @ wl.bf16_to_f32(w).astype(np.float64).T)[tok, col]
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # identity weight returns x exactly
    eye = np.eye(40, dtype=np.float32)
    xf = rng.standard_normal((3, 40)).astype(np.float32)
    tk, cl = np.repeat(np.arange(3), 40), np.tile(np.arange(40), 3)
    assert np.array_equal(oracle.base_sampled(xf, eye, tk, cl), xf[tk, cl].astype(np.float64))


# ------------------------------------------------------------------ P5 segments
@pytest.mark.parametrize("ex", read_golden_examples("segments_worked_examples.txt"),
                         ids=lambda e: e["name"])
def test_segments_worked_examples(ex):
    ids = np.array(ex["ids"].split(), np.int32)
    perm, starts, adapters = oracle.segments(ids, int(ex["num_adapters"]))
    assert perm.tolist() == [int(v) for v in ex["token_perm"].split()]
    assert starts.tolist() == [int(v) for v in ex["seg_starts"].split()]
    assert adapters.tolist() == [int(v) for v in ex["seg_adapter"].split()]


def test_segments_properties_random():
    rng = np.random.default_rng(15)
    for trial in range(200):
        n = int(rng.integers(1, 20))
        t = int(rng.integers(0, 60))
        ids = rng.integers(-1, n, size=t).astype(np.int32)
        perm, starts, adapters = oracle.segments(ids, n)
        kept = np.flatnonzero(ids >= 0)
        assert sorted(perm.tolist()) == kept.tolist()
        assert starts[0] == 0 and starts[-1] == kept.size
        assert np.all(np.diff(starts) > 0)
        assert np.all(np.diff(adapters) > 0)
        for s in range(adapters.size):
            seg = perm[starts[s]:starts[s + 1]]
            assert np.all(ids[seg] == adapters[s])
            assert np.all(np.diff(seg) > 0)          # stable: original order


def test_segments_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.segments(np.array([0, 3, 1], np.int32), 3)
    with pytest.raises(ValueError):
        oracle.segments(np.array([0, -2], np.int32), 3)


# ------------------------------------------------------------------ planted mistakes
MUTATIONS = {
    # a dropped term of the shrink sum
    "drop_last_k": ("for (int32_t k = 0; k < d_in; ++k)\n      s += elem(a_rows",
                    "for (int32_t k = 0; k < d_in - 1; ++k)\n      s += elem(a_rows"),
    # a wrong sign on the delta
    "wrong_sign": ("      y += s;\n    }\n    y_out[(int64_t)t * d_out + i] = y;\n  }\n}",
                   "      y -= s;\n    }\n    y_out[(int64_t)t * d_out + i] = y;\n  }\n}"),
    # B read untransposed (index of j and i swapped within the row block)
    "transposed_b": ("s += elem(bt_rows, w_dtype, (row_off[a] + j) * (int64_t)d_out + i) * v[j];",
                     "s += elem(bt_rows, w_dtype, (row_off[a] + (i % (r > 0 ? r : 1))) * (int64_t)d_out + j) * v[j];"),
    # FP8 exponent bias off by one
    "fp8_bias": ("for (int i = 0; i < e - 7; ++i) p *= 2.0;\n  for (int i = 0; i < 7 - e; ++i) p /= 2.0;",
                 "for (int i = 0; i < e - 8; ++i) p *= 2.0;\n  for (int i = 0; i < 8 - e; ++i) p /= 2.0;"),
    # INT4 nibbles in the wrong order
    "int4_nibbles": ("(base[i >> 1] >> ((i & 1) * 4)) & 15", "(base[i >> 1] >> (((i + 1) & 1) * 4)) & 15"),
    # wrong adapter row offset (adapter a reads adapter 0's rows)
    "wrong_adapter": ("int64_t arow = (row_off[a] + j) * (int64_t)d_in;\n    for (int32_t k = 0; k < d_in; ++k)\n      s += elem(a_rows, w_dtype, arow + k) * elem(x, x_dtype, (int64_t)t * d_in + k);\n    v[j] = s;",
                      "int64_t arow = (row_off[0] + j) * (int64_t)d_in;\n    for (int32_t k = 0; k < d_in; ++k)\n      s += elem(a_rows, w_dtype, arow + k) * elem(x, x_dtype, (int64_t)t * d_in + k);\n    v[j] = s;"),
}


def _pin_suite_passes():
    try:
        test_merge_identity(np.float64)
        test_single_adapter_batch_is_one_matmul()
        test_mixed_ranks_against_numpy_per_token()
        test_rank1_unit_adapter_is_exact_copy()
        test_zero_adapter_leaves_y_bit_unchanged("B")
        test_fp8_e4m3_decoding_matches_format_definition()
        test_int4_decoding_matches_twos_complement()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    """Compile the oracle with one plausible mistake planted (on the CPU) and
    check that the pins above reject it."""
    import ctypes
    import subprocess
    src = open(oracle._SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(mutated), "-o",
                           str(so)])
    real = oracle._load()
    assert _pin_suite_passes()
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "_SRC", str(mutated))
    oracle._load()
    assert not _pin_suite_passes(), f"planted mistake {name} went unnoticed"
    monkeypatch.setattr(oracle, "_lib", real)


# ------------------------------------------------------------------ low-precision adapter rows
def test_fp8_e4m3_decoding_matches_format_definition():
    """Bytes from tests/golden/fp8_e4m3_patterns.txt decode to the printed values
    (OCP E4M3), sign of zero included; NaN patterns decode to NaN."""
    for line in open(golden_path("fp8_e4m3_patterns.txt")):
        if line.startswith("#") or not line.strip():
            continue
        h, v = line.split()
        got = oracle.widen_codes(np.array([int(h, 16)], np.uint8), "fp8")[0]
        want = float(v)
        if math.isnan(want):
            assert math.isnan(got), h
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), h


def test_int4_decoding_matches_twos_complement():
    for line in open(golden_path("int4_patterns.txt")):
        if line.startswith("#") or not line.strip():
            continue
        h, e0, e1 = line.split()
        got = oracle.widen_codes(np.array([int(h, 16)], np.uint8), "int4")
        assert got.tolist() == [float(e0), float(e1)], h


def test_fp8_codes_ordered_and_rne_quantizer():
    """Non-negative FP8 codes 0x00..0x7E are strictly increasing in value (the
    quantizer relies on it); the generator's round-to-nearest-even lands on a
    neighbouring code of every input, with ties to the even code."""
    vals = oracle.widen_codes(np.arange(127, dtype=np.uint8), "fp8")
    assert np.all(np.diff(vals) > 0)
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((6, 64)).astype(np.float32)
    codes, scales = wl.quantize_rows(rows, "fp8")
    deq = oracle.dequant_rows(codes, "fp8", scales)
    q = rows.astype(np.float64) / scales.astype(np.float64)[:, None]
    mags = np.minimum(np.abs(q), 448.0)   # the quantizer clamps to the largest finite code
    for r in range(rows.shape[0]):
        assert np.max(np.abs(deq[r])) == pytest.approx(np.max(np.abs(rows[r])), rel=1e-6)
        for c in range(rows.shape[1]):
            got = abs(deq[r, c]) / scales[r]
            lo = vals[vals <= mags[r, c]].max()
            hi = vals[vals >= mags[r, c]].min()
            assert got in (lo, hi)
            if abs(mags[r, c] - lo) != abs(hi - mags[r, c]):
                assert got == (lo if abs(mags[r, c] - lo) < abs(hi - mags[r, c]) else hi)
    # an exact tie: halfway between 1.0 (0x38, even) and 1.125 (0x39) rounds to 1.0
    c, s = wl.quantize_rows(np.array([[448.0, 1.0625]], np.float32), "fp8")
    assert s[0] == 1.0 and c[0, 1] == 0x38


def test_quantized_rank1_adapter_is_exact():
    """FP8 and INT4 rank-1 adapters with unit codes and power-of-two scales move
    x[t, k] * s_A * s_B exactly into y[t, i] (dequantisation multiplies, it does
    not round)."""
    t, d_in, d_out, k, i = 4, 16, 24, 5, 17
    rng = np.random.default_rng(8)
    x = rng.standard_normal((t, d_in))
    y = rng.standard_normal((t, d_out))
    for kind, one in (("fp8", 0x38), ("int4", 1)):
        if kind == "fp8":
            a = np.zeros((1, d_in), np.uint8); a[0, k] = one
            b = np.zeros((1, d_out), np.uint8); b[0, i] = one
        else:
            a = np.zeros((1, d_in // 2), np.uint8); a[0, k // 2] = one << (4 * (k % 2))
            b = np.zeros((1, d_out // 2), np.uint8); b[0, i // 2] = one << (4 * (i % 2))
        ad = oracle.Adapters.from_quantized(kind, [a], [np.array([0.25], np.float32)], [b],
                                            [np.array([8.0], np.float32)])
        out = oracle.apply(x, y, np.zeros(t, np.int32), ad)
        want = y.copy()
        want[:, i] += x[:, k] * 2.0
        assert np.array_equal(out, want), kind


def test_int4_quantizer_rounds_and_clamps():
    rows = np.array([[7.0, -7.0, 3.5, 2.5, -0.5, 0.0, 6.9, -3.49]], np.float32)
    codes, scales = wl.quantize_rows(rows, "int4")
    assert scales[0] == 1.0
    vals = oracle.widen_codes(codes, "int4")
    assert vals.tolist() == [7, -7, 4, 2, -0.0, 0, 7, -3]
