"""Host half of the C ABI, exercised without a GPU: symbol exports, the segment
build (bit-exact against the oracle's different algorithm), the planner's
coverage, the page pool's bookkeeping and the error conventions."""
import ctypes
import types
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT, read_golden_examples
from segmented_gather_gemm_segments_amd import binding as B
from segmented_gather_gemm_segments_amd import build as lbuild


@pytest.fixture(scope="module", autouse=True)
def built_lib():
    if not lbuild.up_to_date():
        lbuild.build()
    return B.lib()


def header_functions():
    """Every function declared in include/*.h."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 15
    h = ctypes.CDLL(B.lib_path())
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(B.EXPORTS), "binding and header disagree"
    assert B.lib().lora_abi_version() == 2


# ------------------------------------------------------------------ segments
@pytest.mark.parametrize("ex", read_golden_examples("segments_worked_examples.txt"),
                         ids=lambda e: e["name"])
def test_segments_worked_examples(ex):
    ids = np.array(ex["ids"].split(), np.int32)
    perm, starts, adapters = B.lora_segments_build(ids, int(ex["num_adapters"]))
    assert perm.tolist() == [int(v) for v in ex["token_perm"].split()]
    assert starts.tolist() == [int(v) for v in ex["seg_starts"].split()]
    assert adapters.tolist() == [int(v) for v in ex["seg_adapter"].split()]


def test_segments_bit_exact_vs_oracle_random():
    rng = np.random.default_rng(21)
    for trial in range(300):
        n = int(rng.integers(1, 300))
        t = int(rng.integers(0, 2000))
        p_none = rng.random() * 0.3
        ids = rng.integers(0, n, size=t).astype(np.int32)
        ids[rng.random(t) < p_none] = -1
        got = B.lora_segments_build(ids, n)
        want = oracle.segments(ids, n)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_segments_full_size_workloads():
    from segmented_gather_gemm_segments_amd import workloads as wl
    for ids, n in [(wl.sgmv_prefill().ids, 64), (wl.layer_batch_ids(), 256),
                   (wl.hetero_paged().ids, 64)]:
        got = B.lora_segments_build(ids, n)
        want = oracle.segments(ids, n)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_segments_edge_cases():
    perm, starts, adapters = B.lora_segments_build(np.zeros(0, np.int32), 5)
    assert perm.size == 0 and starts.tolist() == [0] and adapters.size == 0
    perm, starts, adapters = B.lora_segments_build(np.full(7, -1, np.int32), 5)
    assert perm.size == 0 and starts.tolist() == [0]
    perm, starts, adapters = B.lora_segments_build(np.full(9, 3, np.int32), 5)
    assert perm.tolist() == list(range(9)) and starts.tolist() == [0, 9] and adapters.tolist() == [3]
    with pytest.raises(B.LoraError) as e:
        B.lora_segments_build(np.array([0, 5], np.int32), 5)
    assert e.value.status == B.LORA_ERANGE
    with pytest.raises(B.LoraError) as e:
        B.lora_segments_build(np.array([-2], np.int32), 5)
    assert e.value.status == B.LORA_ERANGE


# ------------------------------------------------------------------ planner
def _coverage(items, starts, adapters, ranks, dim, phase):
    """Count how often each (perm position, output unit) is covered: rows of v
    for a shrink plan, 8-column chunks of y for an expand plan."""
    n_tok = int(starts[-1])
    width = dim if phase == B.LORA_PHASE_SHRINK else dim // 8
    cov = np.zeros((n_tok, width), np.int32)
    seg_of = np.repeat(np.arange(starts.size - 1), np.diff(starts))
    for pb, a, cp, blk in items:
        cnt, path = cp & 0xFFFF, cp >> 16
        assert 1 <= cnt and path in (B.LORA_PATH_GATHER, B.LORA_PATH_MFMA)
        assert len(set(seg_of[pb:pb + cnt])) == 1        # one segment per item
        if phase == B.LORA_PHASE_SHRINK:
            r = int(ranks[a])
            if path == B.LORA_PATH_MFMA:
                assert cnt <= B.LORA_SHRINK_MFMA_TOKENS and blk == 0
                j0, j1 = 0, r
            else:
                assert cnt <= B.LORA_SHRINK_GATHER_TOKENS
                j0 = blk * B.LORA_SHRINK_GATHER_ROWS
                j1 = min(r, j0 + B.LORA_SHRINK_GATHER_ROWS)
                assert j0 < r                                # no empty row group is planned
            cov[pb:pb + cnt, j0:j1] += 1
        else:
            assert cnt <= (B.LORA_EXPAND_MFMA_TOKENS if path == B.LORA_PATH_MFMA else B.LORA_EXPAND_GATHER_TOKENS)
            cols = B.LORA_EXPAND_MFMA_COLS if path == B.LORA_PATH_MFMA else B.LORA_EXPAND_GATHER_COLS
            c0, c1 = blk * cols, min(dim, (blk + 1) * cols)
            assert c0 < dim
            cov[pb:pb + cnt, c0 // 8:c1 // 8] += 1
    return cov


@pytest.mark.parametrize("policy", [B.LORA_PATH_AUTO, B.LORA_PATH_GATHER, B.LORA_PATH_MFMA])
def test_plan_covers_every_output_once(policy):
    rng = np.random.default_rng(31)
    for trial in range(40):
        n = int(rng.integers(1, 40))
        t = int(rng.integers(1, 600))
        ids = rng.integers(-1, n, size=t).astype(np.int32)
        perm, starts, adapters = B.lora_segments_build(ids, n)
        if adapters.size == 0:
            continue
        ranks = rng.integers(1, 65, size=n).astype(np.int32)
        r_max = int(ranks.max())
        d_out = int(rng.integers(1, 600)) * 8
        for phase, dim in ((B.LORA_PHASE_SHRINK, r_max), (B.LORA_PHASE_EXPAND, d_out)):
            items = B.lora_sgmv_plan(phase, starts, adapters, n, dim, policy, host_rank=ranks)
            cov = _coverage(items, starts, adapters, ranks, dim, phase)
            seg_of = np.repeat(np.arange(adapters.size), np.diff(starts))
            if phase == B.LORA_PHASE_SHRINK:
                want = (np.arange(r_max)[None, :] < ranks[adapters[seg_of]][:, None]).astype(np.int32)
                assert np.array_equal(cov, want)
            else:
                assert np.all(cov == 1)
            # adapter of each item is its segment's adapter
            assert np.all(adapters[seg_of[items[:, 0]]] == items[:, 1])
        # without host ranks every adapter is planned at r_max
        items = B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, starts, adapters, n, r_max, policy)
        cov = _coverage(items, starts, adapters, np.full(n, r_max, np.int32), r_max,
                        B.LORA_PHASE_SHRINK)
        assert np.all(cov == 1)


def test_plan_path_choice_and_order():
    starts = np.array([0, 1, 16, 116], np.int32)     # lengths 1, 15, 100
    adapters = np.array([0, 1, 2], np.int32)
    items = B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, starts, adapters, 3, 16)
    paths = {int(a): int(cp >> 16) for _, a, cp, _ in items}
    assert paths == {0: B.LORA_PATH_GATHER, 1: B.LORA_PATH_GATHER, 2: B.LORA_PATH_MFMA}
    items = B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, starts, adapters, 3, 16, mfma_min_tokens=1)
    assert all((cp >> 16) == B.LORA_PATH_MFMA for _, _, cp, _ in items)
    # heaviest first: expand items ordered by the bytes they move (y read and
    # written per token, plus the adapter's B^T rows over the item's columns:
    # 16 rows assumed when no ranks are given)
    items = B.lora_sgmv_plan(B.LORA_PHASE_EXPAND, starts, adapters, 3, 4096)
    cols = np.where((items[:, 2] >> 16) == B.LORA_PATH_MFMA, B.LORA_EXPAND_MFMA_COLS,
                    B.LORA_EXPAND_GATHER_COLS)
    weight = cols * (4 * (items[:, 2] & 0xFFFF) + 32)
    assert np.all(np.diff(weight) <= 0)
    # a rank-8 adapter on the gather path needs two row groups, a rank-16 one four
    items = B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, starts, adapters, 3, 16, B.LORA_PATH_GATHER,
                             host_rank=np.array([8, 16, 16], np.int32))
    assert sorted(int(b) for _, a, _, b in items if a == 0) == [0, 1]


def test_expand_mfma_token_tile():
    """MFMA expand items take 128 tokens for output widths nearest 8192 of the
    measured widths (1024, 4096, 8192, 14336, 28672) while the plan then still
    holds >= 256 MFMA items, else 64; every (token, column) stays covered once
    either way."""
    def plan(lens, d_out):
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        adapters = np.arange(len(lens), dtype=np.int32)
        items = B.lora_sgmv_plan(B.LORA_PHASE_EXPAND, starts, adapters, len(lens), d_out)
        cov = _coverage(items, starts, adapters, np.full(len(lens), 16), d_out, B.LORA_PHASE_EXPAND)
        assert np.all(cov == 1)
        m = items[(items[:, 2] >> 16) == B.LORA_PATH_MFMA]
        return int((m[:, 2] & 0xFFFF).max()), len(m)
    # the 70B layer's batch: 255 one-token requests and one of 1025 tokens
    lens = [1] * 255 + [1025]
    assert plan(lens, 8192) == (128, 9 * 32)     # q, o, down
    assert plan(lens, 1024) == (64, 17 * 4)      # k, v: 9 x 4 = 36 long items would not fill the device
    assert plan(lens, 28672) == (64, 17 * 112)   # gate, up
    assert plan(lens, 4096) == (64, 17 * 16)
    assert plan(lens, 14336) == (64, 17 * 56)
    assert plan(lens, 10240) == (128, 9 * 40)    # nearest measured width 8192
    assert plan(lens, 12288) == (64, 17 * 48)    # nearest 14336
    # the item threshold: 8 x 32 = 256 long items, 7 x 32 = 224
    assert plan([1024], 8192) == (128, 256)
    assert plan([1000], 8192) == (128, 256)
    assert plan([896], 8192) == (64, 14 * 32)
    assert plan([896, 100], 8192)[0] == 128     # (7 + 1) x 32


@pytest.mark.parametrize("tile", [64, 128])
def test_expand_tile_forced(tile):
    """lora_sgmv_plan_tile with a given MFMA expand tile: every MFMA item of a
    long segment but its last holds exactly `tile` tokens, the coverage holds,
    a shrink plan is unchanged, and other tiles are rejected."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        n = int(rng.integers(1, 12))
        ids = rng.integers(-1, n, size=int(rng.integers(1, 900))).astype(np.int32)
        perm, starts, adapters = B.lora_segments_build(ids, n)
        if adapters.size == 0:
            continue
        ranks = rng.integers(1, 65, size=n).astype(np.int32)
        d_out = int(rng.integers(1, 300)) * 8
        items = B.lora_sgmv_plan(B.LORA_PHASE_EXPAND, starts, adapters, n, d_out, expand_tile_tokens=tile)
        assert np.all(_coverage(items, starts, adapters, ranks, d_out, B.LORA_PHASE_EXPAND) == 1)
        for pb, a, cp, blk in items:
            cnt, path = cp & 0xFFFF, cp >> 16
            if path == B.LORA_PATH_MFMA:
                s = int(np.searchsorted(starts, pb, side="right")) - 1
                assert cnt == min(tile, int(starts[s + 1]) - pb) and (pb - int(starts[s])) % tile == 0
        sh = B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, starts, adapters, n, int(ranks.max()), host_rank=ranks,
                              expand_tile_tokens=tile)
        assert np.array_equal(sh, B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, starts, adapters, n, int(ranks.max()),
                                                   host_rank=ranks))
    for bad in (32, 96, 256, -64):
        with pytest.raises(B.LoraError) as e:
            B.lora_sgmv_plan(B.LORA_PHASE_EXPAND, np.array([0, 300], np.int32), np.array([0], np.int32), 1, 1024,
                             expand_tile_tokens=bad)
        assert e.value.status == B.LORA_EINVAL


def test_plan_errors():
    with pytest.raises(B.LoraError) as e:
        B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, np.array([0, 2], np.int32), np.array([7], np.int32), 3, 16)
    assert e.value.status == B.LORA_ERANGE
    with pytest.raises(B.LoraError) as e:
        B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, np.array([0, 2, 2], np.int32), np.array([0, 1], np.int32), 3, 16)
    assert e.value.status == B.LORA_EINVAL
    with pytest.raises(B.LoraError) as e:
        B.lora_sgmv_plan(B.LORA_PHASE_EXPAND, np.array([0, 2], np.int32), np.array([0], np.int32), 3, 12)
    assert e.value.status == B.LORA_EUNSUPPORTED
    with pytest.raises(B.LoraError):
        B.lora_sgmv_plan(7, np.array([0, 2], np.int32), np.array([0], np.int32), 3, 64)
    # capacity too small -> ENOMEM, count still reported
    lib = B.lib()
    st = np.array([0, 40], np.int32)
    ad = np.array([0], np.int32)
    n = ctypes.c_int32(0)
    items = np.zeros((1, 4), np.int32)
    rc = lib.lora_sgmv_plan(0, st.ctypes.data, ad.ctypes.data, 1, 1, None, 16, 0, 16,
                            items.ctypes.data, 1, ctypes.byref(n))
    assert rc == B.LORA_ENOMEM and n.value == 3
    # an empty batch plans to nothing
    assert B.lora_sgmv_plan(0, np.array([0], np.int32), np.zeros(0, np.int32), 3, 16).shape == (0, 4)
    # r_max out of range for a shrink plan; a rank above r_max
    with pytest.raises(B.LoraError) as e:
        B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, np.array([0, 2], np.int32), np.array([0], np.int32), 3, 129)
    assert e.value.status == B.LORA_EUNSUPPORTED
    with pytest.raises(B.LoraError) as e:
        B.lora_sgmv_plan(B.LORA_PHASE_SHRINK, np.array([0, 2], np.int32), np.array([0], np.int32), 3, 16,
                         host_rank=np.array([32, 8, 8], np.int32))
    assert e.value.status == B.LORA_ERANGE


# ------------------------------------------------------------------ pool
class _FakeStorage:
    """Host-only stand-in for a device tensor: the pool's bookkeeping never
    dereferences storage except in write_rows (GPU-tier)."""

    def __init__(self, n, pr, w):
        self.shape = (n, pr, w)
        self.buf = np.zeros(1, np.uint8)
        import torch
        self.dtype = torch.bfloat16

    def data_ptr(self):
        return self.buf.ctypes.data


def test_pool_alloc_free_and_shuffle():
    s = _FakeStorage(64, 16, 128)
    p = B.Pool(s, 16, shuffle_seed=1234)
    assert p.num_free() == 64
    got = [p.alloc(r) for r in (8, 16, 17, 64, 1)]
    assert [g.size for g in got] == [1, 1, 2, 4, 1]
    flat = np.concatenate(got)
    assert len(set(flat.tolist())) == flat.size and flat.min() >= 0 and flat.max() < 64
    assert p.num_free() == 64 - 9
    assert flat.tolist() != sorted(flat.tolist())            # shuffled order
    q = B.Pool(_FakeStorage(64, 16, 128), 16, shuffle_seed=1234)
    assert np.array_equal(np.concatenate([q.alloc(r) for r in (8, 16, 17, 64, 1)]), flat)
    z = B.Pool(_FakeStorage(8, 16, 128), 16, shuffle_seed=0)
    assert z.alloc(48).tolist() == [0, 1, 2]                  # seed 0: in order
    p.free(got[2])
    assert p.num_free() == 64 - 7
    with pytest.raises(B.LoraError) as e:
        p.free(got[2])                                       # double free
    assert e.value.status == B.LORA_EINVAL
    with pytest.raises(B.LoraError) as e:
        p.alloc(16 * 100)
    assert e.value.status == B.LORA_ENOMEM
    assert p.num_free() == 64 - 7                             # nothing taken on failure
    rest = p.alloc(16 * p.num_free())
    assert p.num_free() == 0 and rest.size == 57


def test_pool_formats():
    """Quantized pools need row scales (and bf16), plain pools take none; the
    bookkeeping is the same for every format."""
    lib, h = B.lib(), ctypes.c_void_p()
    buf = np.zeros(4, np.float32)
    sc = buf.ctypes.data
    assert lib.lora_pool_create(8, 16, 64, B.LORA_BF16, B.LORA_WFMT_FP8_E4M3, 16, None, 0,
                                ctypes.byref(h)) == B.LORA_EINVAL
    assert lib.lora_pool_create(8, 16, 64, B.LORA_BF16, B.LORA_WFMT_PLAIN, 16, sc, 0,
                                ctypes.byref(h)) == B.LORA_EINVAL
    assert lib.lora_pool_create(8, 16, 64, B.LORA_F32, B.LORA_WFMT_INT4, 16, sc, 0,
                                ctypes.byref(h)) == B.LORA_EUNSUPPORTED
    assert lib.lora_pool_create(8, 16, 63, B.LORA_BF16, B.LORA_WFMT_INT4, 16, sc, 0,
                                ctypes.byref(h)) == B.LORA_EINVAL
    assert lib.lora_pool_create(8, 16, 64, B.LORA_BF16, 7, 16, sc, 0,
                                ctypes.byref(h)) == B.LORA_EUNSUPPORTED
    s = _FakeStorage(8, 16, 32)
    p = B.Pool(s, 16, shuffle_seed=3, weight_format=B.LORA_WFMT_INT4, scales=_FakeStorage(1, 1, 1))
    ids = p.alloc(20)
    assert ids.size == 2 and p.num_free() == 6
    with pytest.raises(B.LoraError) as e:   # a quantized pool needs the rows' scales
        p.write_rows(ids, _FakeStorage(20, 1, 32), stream=types.SimpleNamespace(cuda_stream=0))
    assert e.value.status == B.LORA_EINVAL
    p.free(ids)
    assert p.num_free() == 8


# ------------------------------------------------------------------ ABI errors
def _desc(**kw):
    base = dict(dtype=1, d_in=64, d_out=64, num_adapters=2, r_max=16, page_rows=16, max_pages=1,
                num_pages_a=2, num_pages_b=2, weight_format=0, a_pages=16, b_pages=16, rank=16,
                a_page_table=None, b_page_table=None, host_rank=None, a_scales=None,
                b_scales=None)
    base.update(kw)
    return B.lora_weights(*[base[f] for f, _ in B.lora_weights._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), B.LORA_EUNSUPPORTED),
    (dict(d_in=60), B.LORA_EUNSUPPORTED),
    (dict(d_out=0), B.LORA_EUNSUPPORTED),
    (dict(r_max=200), B.LORA_EUNSUPPORTED),
    (dict(r_max=0), B.LORA_EUNSUPPORTED),
    (dict(a_pages=None), B.LORA_EINVAL),
    (dict(a_pages=18), B.LORA_EINVAL),            # misaligned
    (dict(page_rows=8), B.LORA_EINVAL),           # dense stack needs page_rows >= r_max
    (dict(weight_format=3), B.LORA_EUNSUPPORTED),
    (dict(weight_format=-1), B.LORA_EUNSUPPORTED),
    (dict(weight_format=1, dtype=0, a_scales=16, b_scales=16), B.LORA_EUNSUPPORTED),  # fp32 + FP8
    (dict(weight_format=1), B.LORA_EINVAL),                                 # no row scales
    (dict(weight_format=2, a_scales=16), B.LORA_EINVAL),                    # one scale array
    (dict(weight_format=2, a_scales=18, b_scales=16), B.LORA_EINVAL),       # misaligned scales
    (dict(a_page_table=64), B.LORA_EINVAL),       # one table without the other
    # stored-row numbers must fit 32 bits: 2^27 pages of 16 rows is 2^31 rows
    (dict(a_page_table=64, b_page_table=64, num_pages_a=1 << 27), B.LORA_EINVAL),
    (dict(a_page_table=64, b_page_table=64, num_pages_b=(1 << 27) + 5), B.LORA_EINVAL),
])
def test_weight_validation_errors(kw, status):
    d = _desc(**kw)
    rc = B.lib().lora_sgmv_shrink(ctypes.byref(d), 16, 1, 16, 1, 1, 16, 16, None)
    assert rc == status, B.lora_last_error()
    assert B.lora_last_error()


def test_largest_pool_within_32_bit_rows_is_accepted():
    """(2^31 - 1) // 16 pages of 16 rows pass validation (zero items: a
    validated no-op, no GPU needed)."""
    d = _desc(a_page_table=64, b_page_table=64, num_pages_a=(2**31 - 1) // 16,
              num_pages_b=(2**31 - 1) // 16)
    rc = B.lib().lora_sgmv_shrink(ctypes.byref(d), 16, 1, 16, 0, 1, 16, 16, None)
    assert rc == B.LORA_OK, B.lora_last_error()


def test_host_rank_validation():
    hr = np.array([16, 17], np.int32)
    d = _desc(host_rank=hr.ctypes.data)
    rc = B.lib().lora_bgmv_expand(ctypes.byref(d), 16, 1, 0, 16, 16, None)
    assert rc == B.LORA_ERANGE


def test_empty_batches_are_noops():
    d = _desc()
    lib = B.lib()
    assert lib.lora_sgmv_shrink(ctypes.byref(d), None, 0, None, 0, 0, None, None, None) == B.LORA_OK
    assert lib.lora_sgmv_expand(ctypes.byref(d), 16, 4, 16, 0, 8, 16, 16, None) == B.LORA_OK
    assert lib.lora_bgmv_shrink(ctypes.byref(d), None, 0, 0, None, None, None) == B.LORA_OK
    fused = lib.lora_bgmv_fused
    assert fused(ctypes.byref(d), None, 0, None, 0, 0, None, None, None, None) == B.LORA_OK
    assert fused(ctypes.byref(d), 16, 1, None, 0, 0, None, None, 16, None) == B.LORA_EINVAL
    assert fused(ctypes.byref(d), 16, 1, None, 0, 0, 16, 20, 16, None) == B.LORA_EINVAL  # misaligned v
    assert fused(ctypes.byref(d), 16, -1, None, 0, 0, 16, None, 16, None) == B.LORA_EINVAL
    assert fused(ctypes.byref(d), 16, 1, None, 0, 7, 16, None, 16, None) == B.LORA_EINVAL  # order
    assert fused(ctypes.byref(d), 16, 4, 16, 5, 0, 16, None, 16, None) == B.LORA_EINVAL  # order too long
    assert fused(ctypes.byref(d), 16, 4, 16, -1, 0, 16, None, 16, None) == B.LORA_EINVAL
    assert fused(ctypes.byref(d), 16, 4, 16, 0, 0, 16, None, 16, None) == B.LORA_OK      # empty order
    assert lib.lora_bgmv_expand(ctypes.byref(d), 16, 1, 9, 16, 16, None) == B.LORA_EINVAL  # bad order
    assert lib.lora_sgmv_shrink(ctypes.byref(d), None, 4, 16, 2, 8, 16, 16, None) == B.LORA_EINVAL


def test_base_gemm_workspace_rule():
    """The base GEMM's split-k rule, through the host-only size query (no GPU
    here: the library then assumes MI355X's 256 compute units, 768 slots of
    three workgroups): k is split 2 or 4 ways only for grids of at most half
    the slots, and only while every slice keeps 4 k-steps of 64; the
    workspace holds one fp32 partial output per slice."""
    def ws(m, n, k):
        return B.base_gemm_workspace_bytes(m, n, k)

    out = lambda s, m, n: s * m * n * 4
    assert ws(1280, 1024, 8192) == out(4, 1280, 1024)   # 80 tiles: the 70B k/v projections
    assert ws(1280, 2048, 8192) == out(4, 1280, 2048)   # 160 tiles
    assert ws(1280, 4096, 8192) == out(2, 1280, 4096)   # 320 tiles: 4 slices would overfill
    assert ws(1280, 8192, 8192) == 0                    # 640 tiles: more than half the slots
    assert ws(1280, 28672, 8192) == 0
    assert ws(77, 264, 520) == out(2, 77, 264)          # k of 520: 2 slices keep 4 steps each
    assert ws(200, 136, 1032) == out(4, 200, 136)
    assert ws(129, 128, 64) == 0                        # too short to split
    assert ws(0, 8, 8) == 0
    with pytest.raises(B.LoraError):
        ws(-1, 8, 8)
    with pytest.raises(B.LoraError):
        ws(8, 0, 8)


# ------------------------------------------------------------------ tiled shrink plan
def _tile_slice_len(d_in, ks):
    even = -(-d_in // ks)
    return -(-even // B.LORA_SHRINK_TILE_K) * B.LORA_SHRINK_TILE_K


@pytest.mark.parametrize("policy", [B.LORA_PATH_AUTO, B.LORA_PATH_GATHER, B.LORA_PATH_MFMA])
def test_tiled_plan_covers_every_output_once(policy):
    """Every (token, row of its adapter, d_in slice) is covered exactly once:
    tile items cover (tokens x all rows x one slice), gather items (tokens x
    row group x all of d_in)."""
    rng = np.random.default_rng(40 + policy)
    for trial in range(20):
        nseg = int(rng.integers(1, 12))
        lens = rng.integers(1, 200, size=nseg)
        ranks = rng.choice([1, 8, 13, 16, 32, 50, 64], size=6).astype(np.int32)
        seg_ad = rng.integers(0, 6, size=nseg).astype(np.int32)
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        d_in = int(rng.choice([64, 512, 4096, 8192, 28672]))
        items, ks = B.lora_sgmv_plan_tiled(starts, seg_ad, 6, 64, d_in, policy, 0, 0, host_rank=ranks)
        assert 1 <= ks <= B.LORA_MAX_K_SPLITS
        sl = _tile_slice_len(d_in, ks)
        assert (ks - 1) * sl < d_in  # no empty slice
        n = int(starts[-1])
        cover = np.zeros((n, 64, ks), np.int32)
        for pb, a, cp, blk in items:
            cnt, path = cp & 0xFFFF, cp >> 16
            seg = int(np.searchsorted(starts, pb, side="right") - 1)
            assert seg_ad[seg] == a and pb + cnt <= starts[seg + 1]
            r = int(ranks[a])
            if path == B.LORA_PATH_TILE:
                assert cnt <= B.LORA_SHRINK_TILE_TOKENS and 0 <= blk < ks
                assert policy != B.LORA_PATH_GATHER
                cover[pb:pb + cnt, :r, blk] += 1
            else:
                assert path == B.LORA_PATH_GATHER and policy != B.LORA_PATH_MFMA
                assert cnt <= B.LORA_SHRINK_GATHER_TOKENS
                j0 = blk * B.LORA_SHRINK_GATHER_ROWS
                cover[pb:pb + cnt, j0:min(r, j0 + B.LORA_SHRINK_GATHER_ROWS), :] += 1
        for s in range(nseg):
            r = int(ranks[seg_ad[s]])
            blk = cover[starts[s]:starts[s + 1]]
            assert np.all(blk[:, :r, :] == 1) and np.all(blk[:, r:, :] == 0)
            tiled = policy == B.LORA_PATH_MFMA or (policy == B.LORA_PATH_AUTO and (lens[s] >= 16 or r >= 32))
            is_tile = [it for it in items if it[0] >= starts[s] and it[0] < starts[s + 1]]
            assert all((it[2] >> 16 == B.LORA_PATH_TILE) == tiled for it in is_tile)


def test_tiled_slices_and_workspace():
    # heaviest item (64 + 64) x 8192 x 2 bytes = 2 MiB -> 8 slices of 1024
    items, ks = B.lora_sgmv_plan_tiled([0, 100], [0], 1, 64, 8192, host_rank=[64])
    assert ks == 8 and _tile_slice_len(8192, 8) == 1024
    assert sum(1 for it in items if it[2] >> 16 == B.LORA_PATH_TILE) == 2 * 8
    # max_splits bounds it
    assert B.lora_sgmv_plan_tiled([0, 100], [0], 1, 64, 8192, max_splits=3, host_rank=[64])[1] == 3
    # rank 16, 1024 tokens on 8192: (64 + 16) x 16 KiB = 1.25 MiB -> 5 slices of 1664 (the last 1536)
    items, ks = B.lora_sgmv_plan_tiled([0, 1024], [0], 1, 16, 8192, host_rank=[16])
    assert ks == 5 and _tile_slice_len(8192, 5) == 1664 and 4 * 1664 < 8192
    assert B.lora_sgmv_shrink_tiled_workspace(1280, 16, 5) == 5 * 1280 * 16 * 4
    assert B.lora_sgmv_shrink_tiled_workspace(1280, 16, 1) == 0
    # no tiled segment (short, rank 16): one slice; a short rank-32 segment is tiled
    assert B.lora_sgmv_plan_tiled([0, 3, 4], [0, 0], 1, 16, 8192, host_rank=[16])[1] == 1
    items, ks = B.lora_sgmv_plan_tiled([0, 3], [0], 1, 32, 8192, host_rank=[32])
    assert ks == 3 and all(it[2] >> 16 == B.LORA_PATH_TILE for it in items)  # (3 + 32) x 16 KiB


def test_tiled_plan_validation():
    lib = B.lib()
    n, ks = ctypes.c_int32(0), ctypes.c_int32(0)
    starts = np.array([0, 10], np.int32)
    ad = np.array([0], np.int32)
    sp, ap = starts.ctypes.data_as(ctypes.c_void_p), ad.ctypes.data_as(ctypes.c_void_p)
    call = lambda d_in, r_max, ms=0: lib.lora_sgmv_plan_tiled(sp, ap, 1, 1, None, r_max, d_in, 0, 0, ms, None, 0,
                                                               ctypes.byref(n), ctypes.byref(ks))
    assert call(4096, 16) == B.LORA_OK
    assert call(4104, 16) == B.LORA_EUNSUPPORTED      # not a multiple of 64
    assert call(0, 16) == B.LORA_EUNSUPPORTED
    assert call(4096, 65) == B.LORA_EUNSUPPORTED      # r_max above 64
    assert call(4096, 16, 65) == B.LORA_EINVAL        # max_splits above the bound
    assert lib.lora_sgmv_plan_tiled(sp, ap, 1, 1, None, 16, 4096, 0, 0, 0, None, 0, None,
                                    ctypes.byref(ks)) == B.LORA_EINVAL
    out = ctypes.c_int64(0)
    assert lib.lora_sgmv_shrink_tiled_workspace(10, 16, 0, ctypes.byref(out)) == B.LORA_EINVAL
    assert lib.lora_sgmv_shrink_tiled_workspace(10, 65, 2, ctypes.byref(out)) == B.LORA_EINVAL
    assert lib.lora_sgmv_shrink_tiled_workspace(-1, 16, 2, ctypes.byref(out)) == B.LORA_EINVAL


def test_tiled_pays_choice():
    """The library prefers the tiled shrink where its tile items save at least
    24 MiB of compute-unit reads: the prefill and heterogeneous batches (bf16,
    FP8 or INT4 rows) and the 70B layer's down projection (d_in 28672), not
    the layer's q projection (d_in 8192: 768 A rows x 16 KiB = 12 MiB saved);
    never for fp32 activations, r_max above 64 or d_in not a multiple of 64."""
    from segmented_gather_gemm_segments_amd import workloads as wl

    def pays(p, dtype=B.LORA_BF16, wfmt=B.LORA_WFMT_PLAIN, d_in=None):
        _, st, ad = B.lora_segments_build(p.ids, p.num_adapters)
        return B.lora_sgmv_tiled_pays(st, ad, p.num_adapters, p.r_max, d_in or p.d_in, dtype, wfmt,
                                      host_rank=p.ranks.astype(np.int32))
    pre = wl.sgmv_prefill()
    het = wl.hetero_paged()
    lay = wl.layer_projection("q", with_base=False)
    down = wl.layer_projection("down", with_base=False)
    assert pays(pre) and pays(het) and not pays(lay) and pays(down)
    assert not pays(het, dtype=B.LORA_F32)
    assert pays(het, wfmt=B.LORA_WFMT_FP8_E4M3) and pays(het, wfmt=B.LORA_WFMT_INT4)
    assert not pays(het, d_in=8200)
    # the byte rule: 64 one-token rank-64 segments on d_in 8192 save 64 x (16 - 1) rows x 16 KiB = 15 MiB
    # (no), 128 of them 30 MiB (yes); rank 16 saves nothing on one token (x read 4x vs 1x: 3 rows each)
    st64 = np.arange(65, dtype=np.int32)
    st128 = np.arange(129, dtype=np.int32)
    assert not B.lora_sgmv_tiled_pays(st64, np.arange(64), 64, 64, 8192, B.LORA_BF16, host_rank=[64] * 64)
    assert B.lora_sgmv_tiled_pays(st128, np.arange(128), 128, 64, 8192, B.LORA_BF16, host_rank=[64] * 128)
    assert not B.lora_sgmv_tiled_pays(st128, np.arange(128), 128, 16, 8192, B.LORA_BF16, host_rank=[16] * 128)
    assert not B.lora_sgmv_tiled_pays([0, 1], [0], 1, 80, 4096, B.LORA_BF16, host_rank=[80])
