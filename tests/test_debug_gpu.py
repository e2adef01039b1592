"""The debug build of the library (liblora_sgmv_debug.so, LORA_DEBUG): its
kernels record bad device-side values -- a page id outside the pool, an
adapter id outside {-1} U [0, N), a used adapter's rank outside 1..r_max, a
token_perm entry outside the batch, a malformed plan item -- in an error word
read back by lora_debug_flags, while every kernel still skips such values
and exits normally (the device synchronises without error, and the tokens the
bad value does not touch keep their bits).  A clean run leaves the word 0."""
import numpy as np
import pytest

from segmented_gather_gemm_segments_amd import binding as B
from segmented_gather_gemm_segments_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def debug_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.select_library(True)
    B.lib()
    yield
    B.select_library(False)


def say(msg):
    print(f"[case] {msg}", flush=True)


def runner():
    from segmented_gather_gemm_segments_amd import runner as R
    return R


def _problem(layout):
    R = runner()
    p = wl.make_problem(f"debug_{layout}", [40, 3, 1, 25, 7], [0, 3, 1, 2, 4], [16, 8, 32, 16, 24],
                        512, 768, "bf16", 77)
    return p, R.DeviceProblem(p, layout=layout)


def _flags():
    torch.cuda.synchronize()      # every kernel ended normally
    return B.lora_debug_flags(clear=True)


def test_release_library_has_no_debug_word():
    B.select_library(False)
    try:
        with pytest.raises(B.LoraError) as e:
            B.lora_debug_flags()
        assert e.value.status == B.LORA_EUNSUPPORTED
    finally:
        B.select_library(True)


def test_clean_runs_leave_the_word_zero():
    B.lora_debug_flags(clear=True)
    for layout in ("dense", "paged"):
        p, dp = _problem(layout)
        say(f"debug clean {layout}")
        for pol in (B.LORA_PATH_AUTO, B.LORA_PATH_GATHER, B.LORA_PATH_MFMA):
            dp.run_sgmv(pol)
        for order in (B.LORA_BGMV_TOKEN_MAJOR, B.LORA_BGMV_ADAPTER_MAJOR):
            dp.run_bgmv(order)
            dp.run_bgmv_fused(order)
        dp.run_bgmv_fused(grouped=True)
        assert _flags() == 0


def test_bad_page_id_is_reported():
    p, dp = _problem("paged")
    say("debug bad page")
    B.lora_debug_flags(clear=True)
    y_ok, _ = dp.run_sgmv(B.LORA_PATH_AUTO)
    assert _flags() == 0
    a = 3                                     # the 3-token request
    dp.weights.a_page_table[a, 0] = dp.a_pages.shape[0] + 5
    dp.weights.b_page_table[a, 0] = -7
    for pol in (B.LORA_PATH_AUTO, B.LORA_PATH_GATHER, B.LORA_PATH_MFMA):
        y, _ = dp.run_sgmv(pol)
        assert _flags() & B.LORA_DEBUG_BAD_PAGE
        other = torch.from_numpy(np.flatnonzero(p.ids != a)).cuda()
        if pol == B.LORA_PATH_AUTO:
            assert torch.equal(y[other].view(torch.int16), y_ok[other].view(torch.int16))
    y, _ = dp.run_bgmv_fused()
    assert _flags() & B.LORA_DEBUG_BAD_PAGE


def test_bad_adapter_id_and_rank_are_reported():
    p, dp = _problem("dense")
    say("debug bad adapter id and rank")
    B.lora_debug_flags(clear=True)
    y_ok, _ = dp.run_bgmv_fused()
    assert _flags() == 0
    t_bad = 5
    dp.ids[t_bad] = p.num_adapters + 9
    for order in (B.LORA_BGMV_TOKEN_MAJOR, B.LORA_BGMV_ADAPTER_MAJOR):
        dp.run_bgmv(order)
        assert _flags() & B.LORA_DEBUG_BAD_ADAPTER
    y, _ = dp.run_bgmv_fused()
    assert _flags() == B.LORA_DEBUG_BAD_ADAPTER
    other = torch.from_numpy(np.delete(np.arange(p.num_tokens), t_bad)).cuda()
    assert torch.equal(y[other].view(torch.int16), y_ok[other].view(torch.int16))
    assert torch.equal(y[t_bad].view(torch.int16), dp.y0[t_bad].view(torch.int16))
    dp.ids[t_bad] = int(p.ids[t_bad])
    dp.rank[4] = dp.r_max + 5                 # clamped to r_max by the kernels
    dp.run_bgmv_fused()
    assert _flags() & B.LORA_DEBUG_BAD_RANK
    dp.run_sgmv(B.LORA_PATH_AUTO)
    assert _flags() & B.LORA_DEBUG_BAD_RANK


def test_bad_token_and_plan_item_are_reported():
    p, dp = _problem("dense")
    say("debug bad token and item")
    B.lora_debug_flags(clear=True)
    _, _, _, perm_d = dp.segments()
    sp = dp.plan(B.LORA_PHASE_SHRINK)
    ep = dp.plan(B.LORA_PHASE_EXPAND)
    y, v = dp.y0.clone(), dp.new_v()
    bad_perm = perm_d.clone()
    bad_perm[0] = p.num_tokens + 3
    B.lora_sgmv_shrink(dp.weights, bad_perm, sp, dp.x, v)
    B.lora_sgmv_expand(dp.weights, bad_perm, ep, v, y)
    assert _flags() == B.LORA_DEBUG_BAD_TOKEN
    bad_items = sp.clone()
    bad_items[0, 1] = p.num_adapters           # adapter outside [0, N)
    B.lora_sgmv_shrink(dp.weights, perm_d, bad_items, dp.x, v)
    assert _flags() == B.LORA_DEBUG_BAD_ITEM


def test_tiled_shrink_reports_bad_values():
    """The tiled shrink (tile items, its gather items and the slice reduction)
    records a bad page, token or plan item like the one-launch kernels, and
    the rows the bad value does not touch keep their bits."""
    R = runner()
    p = wl.make_problem("debug_tiled", [70, 3, 1, 25, 7], [0, 3, 1, 2, 4], [16, 8, 32, 16, 24], 2048, 512,
                        "bf16", 78)
    dp = R.DeviceProblem(p, layout="paged")
    say("debug tiled shrink")
    B.lora_debug_flags(clear=True)
    items, ks, ws = dp.plan_tiled(tile_min_tokens=2)
    host_items = items.cpu().numpy()
    tile = np.flatnonzero((host_items[:, 2] >> 16) == B.LORA_PATH_TILE)
    assert ks > 1 and tile.size > 0
    _, _, _, perm_d = dp.segments()

    def shrink(perm, its):
        v = dp.new_v()
        B.lora_sgmv_shrink_tiled(dp.weights, perm, its, ks, dp.x, v, ws)
        return v

    v_ok = shrink(perm_d, items)
    assert _flags() == 0
    a = 0                                     # the 70-token request: tile items
    saved = int(dp.weights.a_page_table[a, 0])
    dp.weights.a_page_table[a, 0] = dp.a_pages.shape[0] + 5
    v = shrink(perm_d, items)
    assert _flags() == B.LORA_DEBUG_BAD_PAGE
    other = torch.from_numpy(np.flatnonzero(p.ids != a)).cuda()
    assert torch.equal(v[other].view(torch.int32), v_ok[other].view(torch.int32))
    dp.weights.a_page_table[a, 0] = saved
    assert torch.equal(shrink(perm_d, items).view(torch.int32), v_ok.view(torch.int32))
    assert _flags() == 0
    bad_perm = perm_d.clone()
    bad_perm[0] = p.num_tokens + 3
    shrink(bad_perm, items)
    assert _flags() == B.LORA_DEBUG_BAD_TOKEN
    bad_items = items.clone()
    bad_items[int(tile[0]), 3] = ks            # a d_in slice past the last
    shrink(perm_d, bad_items)
    assert _flags() == B.LORA_DEBUG_BAD_ITEM
