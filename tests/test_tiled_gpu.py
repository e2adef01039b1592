"""GPU parity of the tiled segmented shrink (lora_sgmv_shrink_tiled: 64-token
tiles of x and A streamed through LDS, d_in cut into slices whose partial
products a second launch adds in slice order) through the C ABI, against the
fp64 oracle: v within 1e-4 normwise per token (bf16 inputs, fp32
accumulation), and y after the usual expand within 2e-2 normwise and one bf16
rounding per element.  Covers one and several slices, every rank class
(16/32/64 row tiles, ranks not a multiple of 16), partial token tiles, the
three path policies, dense and paged pools, repeat-run bit identity, and the
heterogeneous and prefill batches at full size."""
import numpy as np
import pytest

import oracle
from segmented_gather_gemm_segments_amd import binding as B
from segmented_gather_gemm_segments_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return True


def say(msg):
    print(f"[case] {msg}", flush=True)


def runner():
    from segmented_gather_gemm_segments_amd import runner as R
    return R


def _threads():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def ad_of(p):
    """The problem's adapters in fp64 (quantized rows dequantized exactly)."""
    if p.wq:
        return oracle.Adapters.from_quantized(p.wq, p.a_rows, p.a_scales, p.bt_rows, p.bt_scales)
    return oracle.Adapters.from_stacks(p.a_rows, p.bt_rows)


def check(dp, y, v, label, want_y=None):
    p = dp.p
    ad = ad_of(p)
    want_v = oracle.shrink(p.x, p.ids, ad, dp.r_max)
    got_v = v.cpu().numpy().astype(np.float64)
    rows = np.flatnonzero(p.ids >= 0)
    for t in rows:
        got_v[t, p.ranks[p.ids[t]]:] = 0.0
    den = np.max(np.abs(want_v[rows]), axis=1)
    den[den == 0] = 1.0
    err_v = float(np.max(np.max(np.abs(got_v[rows] - want_v[rows]), axis=1) / den)) if rows.size else 0.0
    say(f"{label}: v error {err_v:.3e}")
    assert err_v <= 1e-4, label
    if want_y is None:
        want_y = oracle.apply(p.x, p.y, p.ids, ad, threads=_threads())
    got = wl.bf16_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    scale = np.max(np.abs(want_y), axis=1, keepdims=True)
    scale[scale == 0] = 1.0
    err = float(np.max(np.max(np.abs(got - want_y), axis=1, keepdims=True) / scale))
    say(f"{label}: y error {err:.3e}")
    assert err <= 2e-2, label
    assert np.all(np.abs(got - want_y) <= np.abs(want_y) * 2.0**-8 + 1e-4 * scale), label
    none = p.ids < 0
    if none.any():
        y0 = wl.bf16_to_f32(dp.y0.view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.array_equal(got[none], y0[none].astype(np.float64)), label


POLICIES = [("auto", B.LORA_PATH_AUTO), ("gather", B.LORA_PATH_GATHER), ("tile", B.LORA_PATH_MFMA)]


def mixed(seed=21, d_in=4096, d_out=768, ranks=(8, 16, 24, 32, 40, 64)):
    """Segments of 1 to 200 tokens (partial 64-token tiles, one-token
    segments), ranks of every row-tile count and some not a multiple of 16."""
    lens = [200, 1, 64, 65, 17, 3, 130, 16, 15, 90]
    ids = [i % len(ranks) for i in range(len(lens))]
    return wl.make_problem(f"tiled_mixed_{seed}", lens, ids, list(ranks), d_in, d_out, "bf16", seed)


@pytest.mark.parametrize("max_splits", [1, 3, 0])
@pytest.mark.parametrize("name,policy", POLICIES)
def test_tiled_mixed(name, policy, max_splits):
    R = runner()
    p = mixed()
    dp = R.DeviceProblem(p)
    items, ks, ws = dp.plan_tiled(policy, 0, max_splits)
    say(f"tiled mixed policy={name} max_splits={max_splits}: k_splits={ks}, items={items.shape[0]}")
    if max_splits == 1:
        assert ks == 1 and ws is None
    elif name != "gather":
        # heaviest tile item: 64 tokens + rank 32 over 8 KiB rows = 768 KiB
        assert ks == 3, ks
    y, v = dp.run_sgmv(policy, tiled=True, max_splits=max_splits)
    torch.cuda.synchronize()
    check(dp, y, v, f"mixed/{name}/{max_splits}")


@pytest.mark.parametrize("layout", ["dense", "paged"])
def test_tiled_r_max_classes(layout):
    """r_max 16, 32 and 64 select the three LDS sizes of the kernel."""
    R = runner()
    for rmax, ranks in ((16, (16, 8, 12)), (32, (32, 16, 20)), (64, (64, 48, 8))):
        p = wl.make_problem(f"tiled_r{rmax}", [70, 40, 5, 128], [0, 1, 2, 0], list(ranks), 2048, 520, "bf16",
                            30 + rmax)
        dp = R.DeviceProblem(p, layout=layout)
        for ms in (1, 0):
            y, v = dp.run_sgmv(tiled=True, tile_min_tokens=2, max_splits=ms)
            torch.cuda.synchronize()
            check(dp, y, v, f"r_max {rmax}/{layout}/splits {ms}")


def test_tiled_paged_equals_dense_and_repeats_bit_identical():
    R = runner()
    p = wl.hetero_paged(num_tokens=900, num_segments=14, d=1024, seed=12)
    dense = R.DeviceProblem(p, layout="dense")
    paged = R.DeviceProblem(p, layout="paged")
    say("tiled: paged vs dense, repeats")
    outs = []
    for dp in (dense, paged, dense):
        y, v = dp.run_sgmv(tiled=True)
        outs.append((y.view(torch.int16).clone(), v.clone()))
    torch.cuda.synchronize()
    for y, v in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(v, outs[0][1])
    check(dense, *dense.run_sgmv(tiled=True), "hetero 900")


def test_tiled_none_ids_and_unused_adapters():
    R = runner()
    rng = np.random.default_rng(8)
    ids = rng.integers(-1, 3, size=300).astype(np.int32)
    p = wl.make_problem("tiled_none", None, None, [16, 64, 32, 8], 256, 264, "bf16", 13, ids=ids)
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv(tiled=True, tile_min_tokens=1)
    torch.cuda.synchronize()
    check(dp, y, v, "none ids")


@pytest.mark.parametrize("layout", ["dense", "paged"])
@pytest.mark.parametrize("wq", ["fp8", "int4"])
def test_tiled_quantized_rows(wq, layout):
    """FP8 E4M3 and INT4 rows (dequantised from LDS, row scale on the sums):
    a mixed batch with every rank class and ranks not a multiple of 16, one
    and several slices, every policy."""
    R = runner()
    lens = [150, 1, 64, 17, 3, 90, 33]
    p = wl.make_problem(f"tiled_{wq}", lens, [i % 5 for i in range(len(lens))], [8, 24, 40, 64, 13], 2048, 520,
                        "bf16", 60, wq=wq, paged=layout == "paged", page_rows=16)
    dp = R.DeviceProblem(p, layout=layout)
    for name, pol in POLICIES:
        for ms in (1, 0):
            y, v = dp.run_sgmv(pol, tiled=True, max_splits=ms)
            torch.cuda.synchronize()
            check(dp, y, v, f"{wq}/{layout}/{name}/splits {ms}")


@pytest.mark.parametrize("wq", ["fp8", "int4"])
def test_tiled_hetero_quantized_full_size(wq):
    """The heterogeneous paged batch with FP8 or INT4 rows, every row and v."""
    R = runner()
    p = wl.hetero_paged(wq=wq)
    dp = R.DeviceProblem(p)
    assert dp.tiled_pays()
    say(f"tiled hetero full size, {wq} rows")
    y, v = dp.run_sgmv(tiled=True)
    torch.cuda.synchronize()
    check(dp, y, v, f"hetero tiled {wq}")


def test_tiled_errors():
    R = runner()
    lib = B.lib()
    p = mixed(d_in=1024)
    dp = R.DeviceProblem(p)
    items, ks, _ = dp.plan_tiled(max_splits=1)
    ws = torch.zeros(4, dtype=torch.float32, device="cuda")
    _, _, _, perm_d = dp.segments()
    v = dp.new_v()
    d = dp.weights.desc()
    import ctypes
    args = (ctypes.byref(d), B._dptr(perm_d), int(perm_d.numel()), B._dptr(items), int(items.shape[0]),
            p.num_tokens)
    assert ks == 1
    # two slices without a workspace, or with a short one; k_splits out of range
    assert lib.lora_sgmv_shrink_tiled(*args, 2, B._dptr(dp.x), B._dptr(v), None, 0, None) == B.LORA_EINVAL
    assert lib.lora_sgmv_shrink_tiled(*args, 2, B._dptr(dp.x), B._dptr(v), B._dptr(ws), 16, None) == B.LORA_EINVAL
    assert lib.lora_sgmv_shrink_tiled(*args, 0, B._dptr(dp.x), B._dptr(v), None, 0, None) == B.LORA_EINVAL
    assert lib.lora_sgmv_shrink_tiled(*args, 65, B._dptr(dp.x), B._dptr(v), None, 0, None) == B.LORA_EINVAL
    # 1024 / 64 = 16 units: 17 slices would leave one empty
    assert lib.lora_sgmv_shrink_tiled(*args, 17, B._dptr(dp.x), B._dptr(v), None, 0, None) == B.LORA_EINVAL
    # fp32 activations are not supported by the tiled shrink (quantized rows are)
    pf = wl.make_problem("tiled_f32", [20], [0], [16], 256, 256, "f32", 3)
    df = R.DeviceProblem(pf)
    it_f, ks_f, _ = df.plan_tiled()
    _, _, _, perm_f = df.segments()
    vf = df.new_v()
    with pytest.raises(B.LoraError):
        B.lora_sgmv_shrink_tiled(df.weights, perm_f, it_f, ks_f, df.x, vf, None)


@pytest.mark.parametrize("shape", ["q", "up"])
def test_tiled_prefill_full_size(shape):
    """The prefill batch as benchmarked (8192 tokens, 32 Zipf requests), every
    row and every token's v."""
    R = runner()
    p = wl.sgmv_prefill(shape=shape)
    dp = R.DeviceProblem(p)
    say(f"tiled prefill full size {shape}")
    y, v = dp.run_sgmv(tiled=True)
    torch.cuda.synchronize()
    check(dp, y, v, f"prefill {shape} tiled")


def test_tiled_hetero_full_size():
    """The heterogeneous paged batch as benchmarked, every row and v."""
    R = runner()
    p = wl.hetero_paged()
    dp = R.DeviceProblem(p)
    items, ks, _ = dp.plan_tiled()
    say(f"tiled hetero full size: k_splits {ks}, items {items.shape[0]}")
    y, v = dp.run_sgmv(tiled=True)
    torch.cuda.synchronize()
    check(dp, y, v, "hetero tiled")


def test_tiled_layer_projection():
    """The 70B layer's q projection delta (256 one-token decode segments on
    gather items, the 1024-token prefill on tile items), every row and v."""
    R = runner()
    p = wl.layer_projection("q", with_base=False)
    dp = R.DeviceProblem(p)
    say("tiled layer q")
    y, v = dp.run_sgmv(tiled=True)
    torch.cuda.synchronize()
    check(dp, y, v, "layer q tiled")
