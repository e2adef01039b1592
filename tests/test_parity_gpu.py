"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Tolerances (normwise per token row, max_t max_i
|g - o| / max_i |o_t|): 2e-2 for bf16 I/O with fp32 accumulation and 1e-5 for
fp32 I/O, as the workloads fix them; tighter internal bounds are derived in
the design notes and checked too (v in fp32: 1e-4 for bf16 inputs; y for bf16:
each element within one bf16 rounding of the exact value plus 1e-4 of the
row's scale).  Integer work (segments) and the zero-adapter case are
bit-exact.
"""
import numpy as np
import pytest

import oracle
from segmented_gather_gemm_segments_amd import binding as B
from segmented_gather_gemm_segments_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
V_TOL = {"bf16": 1e-4, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # raises if the library is missing
    return True


def say(msg):
    print(f"[case] {msg}", flush=True)


def runner():
    from segmented_gather_gemm_segments_amd import runner as R
    return R


def host_y(dp, y):
    R = runner()
    a = R.to_host(y, dp.p.dtype)
    return wl.bf16_to_f32(a).astype(np.float64) if dp.p.dtype == "bf16" else a.astype(np.float64)


def normwise(got, want, rows=None):
    if rows is not None:
        got, want = got[rows], want[rows]
    if got.size == 0:
        return 0.0
    denom = np.max(np.abs(want), axis=1)
    denom[denom == 0] = 1.0
    return float(np.max(np.max(np.abs(got - want), axis=1) / denom))


def check_y(dp, y_gpu, want, label):
    got = host_y(dp, y_gpu)
    err = normwise(got, want)
    say(f"{label}: normwise y error {err:.3e}")
    assert err <= TOL[dp.p.dtype], f"{label}: {err}"
    if dp.p.dtype == "bf16":
        # each element within one bf16 rounding (2^-8 relative) of the exact value,
        # plus the fp32 accumulation slack
        scale = np.max(np.abs(want), axis=1, keepdims=True)
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0**-8 + 1e-4 * scale), label
    # tokens without an adapter are bit-unchanged
    none = dp.p.ids < 0
    if none.any():
        y0 = host_y(dp, dp.y0)
        assert np.array_equal(got[none], y0[none]), label
    return err


def check_v(dp, v_gpu, label):
    p = dp.p
    want = oracle.shrink(p.x, p.ids, oracle_adapters(p), dp.r_max)
    got = v_gpu.cpu().numpy().astype(np.float64)
    rows = p.ids >= 0
    mask = np.zeros_like(got, dtype=bool)
    for t in np.flatnonzero(rows):
        mask[t, : p.ranks[p.ids[t]]] = True
    got = np.where(mask, got, 0.0)
    err = normwise(got, want, rows)
    say(f"{label}: normwise v error {err:.3e}")
    assert err <= V_TOL[p.dtype], f"{label}: v {err}"


def oracle_adapters(p):
    """The problem's adapters in fp64 (quantized rows dequantized exactly)."""
    if p.wq:
        return oracle.Adapters.from_quantized(p.wq, p.a_rows, p.a_scales, p.bt_rows, p.bt_scales)
    return oracle.Adapters.from_stacks(p.a_rows, p.bt_rows)


def _threads():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_y(p):
    return oracle.apply(p.x, p.y, p.ids, oracle_adapters(p), threads=_threads())


POLICIES = [("auto", B.LORA_PATH_AUTO), ("gather", B.LORA_PATH_GATHER), ("mfma", B.LORA_PATH_MFMA)]


# ------------------------------------------------------------------ config 1: tiny fp32
@pytest.mark.parametrize("name,policy", POLICIES)
def test_tiny_sgmv_fp32(name, policy):
    R = runner()
    p = wl.tiny_sgmv()
    say(f"tiny fp32 sgmv policy={name}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv(policy)
    torch.cuda.synchronize()
    check_v(dp, v, f"tiny/{name}")
    check_y(dp, y, oracle_y(p), f"tiny/{name}")


# ------------------------------------------------------------------ config 2: decode
@pytest.mark.parametrize("order", [B.LORA_BGMV_TOKEN_MAJOR, B.LORA_BGMV_ADAPTER_MAJOR, B.LORA_BGMV_AUTO])
def test_bgmv_decode_full_size(order):
    R = runner()
    p = wl.bgmv_decode()
    say(f"bgmv decode full size order={order}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_bgmv(order)
    torch.cuda.synchronize()
    check_v(dp, v, f"bgmv/{order}")
    check_y(dp, y, oracle_y(p), f"bgmv/{order}")


def test_bgmv_fused_decode_full_size():
    """The one-launch per-token delta on the decode batch, and its agreement
    with the two-launch path (different summation orders: within rounding)."""
    R = runner()
    p = wl.bgmv_decode()
    say("bgmv fused decode full size")
    dp = R.DeviceProblem(p)
    y, v = dp.run_bgmv_fused(B.LORA_BGMV_ADAPTER_MAJOR)
    y2, v2 = dp.run_bgmv()
    y3, _ = dp.run_bgmv_fused(B.LORA_BGMV_ADAPTER_MAJOR)
    y4, v4 = dp.run_bgmv_fused(B.LORA_BGMV_TOKEN_MAJOR)
    torch.cuda.synchronize()
    check_v(dp, v, "fused")
    check_y(dp, y, oracle_y(p), "fused")
    assert torch.equal(y.view(torch.int16), y3.view(torch.int16))      # run-to-run identical
    assert torch.equal(y.view(torch.int16), y4.view(torch.int16))      # both orders, same bits
    assert torch.equal(v, v4)
    assert normwise(host_y(dp, y), host_y(dp, y2)) <= 2e-2


def test_bgmv_fused_token_order():
    """Placement order of the fused kernel: the segment order (tokens of an
    adapter together) and an arbitrary partial order give the same bits for
    every listed token as index order; unlisted and out-of-range entries are
    skipped (y unchanged)."""
    R = runner()
    p = wl.bgmv_decode()
    say("bgmv fused token order")
    dp = R.DeviceProblem(p)
    y0, v0 = dp.run_bgmv_fused()
    yg, vg = dp.run_bgmv_fused(grouped=True)
    rng = np.random.default_rng(7)
    listed = rng.permutation(p.num_tokens)[: p.num_tokens // 2]
    order = np.concatenate([listed, [-1, p.num_tokens, 10**6]]).astype(np.int32)
    rng.shuffle(order)
    yp, vp = dp.run_bgmv_fused(token_order=torch.from_numpy(order).cuda())
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), yg.view(torch.int16))
    assert torch.equal(v0, vg)
    lt = torch.from_numpy(np.sort(listed)).cuda()
    unl = np.setdiff1d(np.arange(p.num_tokens), listed)
    ut = torch.from_numpy(unl).cuda()
    assert torch.equal(yp[lt].view(torch.int16), y0[lt].view(torch.int16))
    assert torch.equal(vp[lt], v0[lt])
    assert torch.equal(yp[ut].view(torch.int16), dp.y0[ut].view(torch.int16))
    check_y(dp, yg, oracle_y(p), "fused grouped")


def test_bgmv_orders_bit_identical_and_sgmv_gather_agrees():
    """Per-token results do not depend on grouping: token-major and
    adapter-major give the same bits.  The segmented gather path splits d_in
    over twice as many waves, so its v agrees to fp32 rounding and its y
    within the bf16 bound."""
    R = runner()
    p = wl.bgmv_decode(num_tokens=200, num_adapters=32, d_in=1024, d_out=1536, seed=7)
    say("bgmv orders bit identity; sgmv-gather agreement")
    dp = R.DeviceProblem(p)
    y1, v1 = dp.run_bgmv(B.LORA_BGMV_TOKEN_MAJOR)
    y2, v2 = dp.run_bgmv(B.LORA_BGMV_ADAPTER_MAJOR)
    y3, v3 = dp.run_sgmv(B.LORA_PATH_GATHER)
    torch.cuda.synchronize()
    assert torch.equal(v1, v2)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    rel = float((v3 - v1).abs().max() / v1.abs().max())
    assert rel <= 1e-5, rel
    check_y(dp, y3, oracle_y(p), "sgmv gather")


# ------------------------------------------------------------------ config 3: prefill (reduced)
@pytest.mark.parametrize("name,policy", POLICIES)
def test_sgmv_prefill_reduced(name, policy):
    """Zipf request lengths over several MFMA tiles with ragged tails."""
    R = runner()
    p = wl.make_problem("prefill_reduced", wl.zipf_lengths(np.random.default_rng(3), 1200, 10),
                        np.arange(10, dtype=np.int32) * 3, [16] * 32, 1024, 1536, "bf16", 33)
    say(f"prefill reduced policy={name}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv(policy)
    torch.cuda.synchronize()
    check_v(dp, v, f"prefill/{name}")
    check_y(dp, y, oracle_y(p), f"prefill/{name}")


# ------------------------------------------------------------------ config 4: hetero paged (reduced)
@pytest.mark.parametrize("name,policy", POLICIES)
def test_hetero_paged_reduced(name, policy):
    R = runner()
    p = wl.hetero_paged(num_tokens=700, num_segments=16, d=1024)
    say(f"hetero paged reduced policy={name} ranks={p.ranks.tolist()}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv(policy)
    torch.cuda.synchronize()
    check_v(dp, v, f"hetero/{name}")
    check_y(dp, y, oracle_y(p), f"hetero/{name}")


def test_paged_equals_dense_bit_identical():
    R = runner()
    p = wl.hetero_paged(num_tokens=500, num_segments=12, d=768, seed=9)
    say("paged vs dense")
    dense = R.DeviceProblem(p, layout="dense")
    paged = R.DeviceProblem(p, layout="paged")
    for pol in (B.LORA_PATH_GATHER, B.LORA_PATH_MFMA):
        y1, v1 = dense.run_sgmv(pol)
        y2, v2 = paged.run_sgmv(pol)
        torch.cuda.synchronize()
        assert torch.equal(v1, v2)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        assert torch.isfinite(y2.float()).all()          # NaN-filled unused rows never read


def test_figure_heterogeneous_batch():
    """Four requests -> A12, A12, A47, A89 with ranks 16, 8, 32 (the page's
    figure), one token each plus a few more tokens per request."""
    R = runner()
    ranks = np.full(100, 8, np.int32)
    ranks[12], ranks[47], ranks[89] = 16, 8, 32
    p = wl.make_problem("figure", [5, 3, 1, 7], [12, 12, 47, 89], ranks, 256, 384, "bf16", 125)
    say("figure batch")
    for layout in ("dense", "paged"):
        dp = R.DeviceProblem(p, layout=layout)
        for name, pol in POLICIES:
            y, v = dp.run_sgmv(pol, mfma_min_tokens=4)
            torch.cuda.synchronize()
            check_v(dp, v, f"figure/{layout}/{name}")
            check_y(dp, y, oracle_y(p), f"figure/{layout}/{name}")


# ------------------------------------------------------------------ invariants and edges
def test_zero_adapter_leaves_y_bit_unchanged():
    R = runner()
    p = wl.make_problem("zero", [20, 3, 40], [0, 1, 2], [16, 16, 16], 512, 512, "bf16", 5)
    p.bt_rows = [np.zeros_like(b) for b in p.bt_rows]
    say("zero adapter")
    dp = R.DeviceProblem(p)
    for _, pol in POLICIES:
        y, _ = dp.run_sgmv(pol)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), dp.y0.view(torch.int16))
    y, _ = dp.run_bgmv()
    assert torch.equal(y.view(torch.int16), dp.y0.view(torch.int16))
    y, _ = dp.run_bgmv_fused()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), dp.y0.view(torch.int16))


def test_token_permutation_invariance():
    R = runner()
    p = wl.make_problem("perm", [30, 2, 50, 1, 17], [3, 0, 1, 2, 4], [16, 8, 32, 16, 64], 512, 768,
                        "bf16", 6)
    say("token permutation")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv()
    pi = np.random.default_rng(1).permutation(p.num_tokens)
    q = wl.LoraProblem("perm2", p.dtype, p.ids[pi].copy(), p.x[pi].copy(), p.y[pi].copy(), p.a_rows,
                       p.bt_rows, p.ranks)
    dq = R.DeviceProblem(q)
    y2, v2 = dq.run_sgmv()
    torch.cuda.synchronize()
    a, b = host_y(dp, y)[pi], host_y(dq, y2)
    say(f"permutation: bit-identical={np.array_equal(a, b)} max diff={np.max(np.abs(a - b)):.3e}")
    assert normwise(a, b) <= 1e-6
    check_y(dq, y2, oracle_y(q), "perm")


def test_repeat_runs_bit_identical():
    R = runner()
    p = wl.hetero_paged(num_tokens=600, num_segments=10, d=512, seed=11)
    say("repeat determinism")
    dp = R.DeviceProblem(p)
    outs = [dp.run_sgmv()[0].view(torch.int16).clone() for _ in range(3)]
    outs += [dp.run_bgmv()[0].view(torch.int16).clone() for _ in range(2)]
    outs += [dp.run_bgmv_fused()[0].view(torch.int16).clone() for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert torch.equal(outs[3], outs[4])
    assert torch.equal(outs[5], outs[6])


@pytest.mark.parametrize("layout", ["dense", "paged"])
@pytest.mark.parametrize("dtype,wq", [("bf16", ""), ("bf16", "fp8"), ("f32", "")])
def test_expand_tiles_bit_identical(layout, dtype, wq):
    """MFMA expand items of 64 and of 128 tokens (two passes per workgroup)
    give every token the same bits, and both match the oracle: segments of
    1..300 tokens (several 128-token items, ragged last ones), ranks 8..72
    (one- and two-chunk ranks), d_out ragged against the 256-column blocks."""
    R = runner()
    lens = [300, 1, 128, 129, 64, 65, 17, 3, 200, 16]
    p = wl.make_problem(f"exp_tiles_{dtype}{wq}_{layout}", lens, [i % 5 for i in range(len(lens))],
                        [8, 16, 40, 64, 72], 512, 1288, dtype, 61, paged=layout == "paged", page_rows=16, wq=wq)
    dp = R.DeviceProblem(p, layout=layout)
    say(f"expand tiles 64 / 128 {dtype}{wq} {layout}")
    _, _, _, perm_d = dp.segments()
    v = dp.new_v()
    B.lora_sgmv_shrink(dp.weights, perm_d, dp.plan(B.LORA_PHASE_SHRINK), dp.x, v)
    ys = {}
    for tile in (64, 128):
        ep = dp.plan(B.LORA_PHASE_EXPAND, expand_tile_tokens=tile)
        cnt = (ep[:, 2] & 0xFFFF)[(ep[:, 2] >> 16) == B.LORA_PATH_MFMA]
        assert int(cnt.max()) == tile
        ys[tile] = dp.y0.clone()
        B.lora_sgmv_expand(dp.weights, perm_d, ep, v, ys[tile])
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(ys[64].view(bits), ys[128].view(bits))
    check_y(dp, ys[128], oracle_y(p), f"expand tile 128 {dtype}{wq} {layout}")


@pytest.mark.parametrize("case", ["one_token", "all_single", "one_segment", "ragged_d", "none_ids",
                                  "unused_adapters", "rank128", "odd_ranks"])
def test_edge_cases(case):
    R = runner()
    rng = np.random.default_rng(17)
    if case == "one_token":
        p = wl.make_problem(case, [1], [0], [16], 512, 512, "bf16", 1)
    elif case == "all_single":
        p = wl.make_problem(case, [1] * 40, np.arange(40), [16] * 40, 256, 264, "bf16", 2)
    elif case == "one_segment":
        p = wl.make_problem(case, [333], [1], [16, 32], 520, 1000, "bf16", 3)
    elif case == "ragged_d":
        p = wl.make_problem(case, [37, 5], [0, 1], [16, 8], 8 * 37, 8 * 101, "bf16", 4)
    elif case == "none_ids":
        ids = rng.integers(-1, 4, size=90).astype(np.int32)
        p = wl.make_problem(case, None, None, [16, 32, 8, 64], 384, 256, "bf16", 5, ids=ids)
    elif case == "unused_adapters":
        p = wl.make_problem(case, [20, 4], [7, 2], [16] * 10, 256, 256, "bf16", 6)
    elif case == "rank128":
        p = wl.make_problem(case, [40, 3], [0, 1], [128, 100], 256, 512, "bf16", 7)
    else:
        p = wl.make_problem(case, [19, 2, 33], [0, 1, 2], [3, 13, 24], 128, 136, "f32", 8)
    say(f"edge {case}")
    want = oracle_y(p)
    for layout in ("dense", "paged"):
        dp = R.DeviceProblem(p, layout=layout)
        for name, pol in POLICIES:
            y, v = dp.run_sgmv(pol)
            torch.cuda.synchronize()
            check_v(dp, v, f"{case}/{layout}/{name}")
            check_y(dp, y, want, f"{case}/{layout}/{name}")
        for order in (B.LORA_BGMV_TOKEN_MAJOR, B.LORA_BGMV_ADAPTER_MAJOR):
            y, v = dp.run_bgmv(order)
            torch.cuda.synchronize()
            check_y(dp, y, want, f"{case}/{layout}/bgmv{order}")
        for order in (B.LORA_BGMV_TOKEN_MAJOR, B.LORA_BGMV_ADAPTER_MAJOR):
            y, v = dp.run_bgmv_fused(order)
            torch.cuda.synchronize()
            check_v(dp, v, f"{case}/{layout}/fused{order}")
            check_y(dp, y, want, f"{case}/{layout}/fused{order}")


def test_empty_batch_noop():
    R = runner()
    p = wl.make_problem("empty", None, None, [16, 16], 256, 256, "bf16", 9,
                        ids=np.full(12, -1, np.int32))
    dp = R.DeviceProblem(p)
    y, _ = dp.run_sgmv()
    y2, _ = dp.run_bgmv()
    y3, _ = dp.run_bgmv_fused()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), dp.y0.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), dp.y0.view(torch.int16))
    assert torch.equal(y3.view(torch.int16), dp.y0.view(torch.int16))


@pytest.mark.parametrize("workload", ["hetero_reduced", "decode"])
def test_adapter_serial_comparator(workload):
    """The adapter-serial comparator (one shrink + expand launch per adapter
    sub-batch, through the same kernels) against the oracle on every row and
    every token's v, and bit-identical to the one-launch plan (it runs the same
    work items)."""
    R = runner()
    if workload == "decode":
        p = wl.bgmv_decode()
        p.mode = "sgmv"
    else:
        p = wl.hetero_paged(num_tokens=500, num_segments=12, d=768, seed=21)
    say(f"adapter-serial comparator {workload}")
    dp = R.DeviceProblem(p)
    y1, v1 = dp.run_sgmv()
    y2, v2 = dp.y0.clone(), dp.new_v()
    for shrink, expand in dp.serial_calls(y2, v2):
        shrink()
        expand()
    torch.cuda.synchronize()
    check_v(dp, v2, f"serial {workload}")
    check_y(dp, y2, oracle_y(p), f"serial {workload}")
    assert torch.equal(v1, v2)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------------------ quantized adapter rows
WQ = ["fp8", "int4"]


@pytest.mark.parametrize("layout", ["dense", "paged"])
@pytest.mark.parametrize("name,policy", POLICIES)
@pytest.mark.parametrize("wq", WQ)
def test_quant_sgmv_mixed(wq, name, policy, layout):
    """FP8 E4M3 / INT4 rows with per-row scales on both SGMV paths, dense and
    paged, against the oracle on the exactly dequantized rows."""
    R = runner()
    p = wl.quant_mixed(wq, paged=layout == "paged")
    say(f"quant sgmv {wq} policy={name} layout={layout}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv(policy)
    torch.cuda.synchronize()
    check_v(dp, v, f"quant/{wq}/{name}/{layout}")
    check_y(dp, y, oracle_y(p), f"quant/{wq}/{name}/{layout}")


@pytest.mark.parametrize("wq", WQ)
def test_quant_bgmv_mixed(wq):
    """Per-token paths (two-launch in both orders, fused in both orders) on the
    mixed quantized batch, paged."""
    R = runner()
    p = wl.quant_mixed(wq, paged=True)
    dp = R.DeviceProblem(p)
    want = oracle_y(p)
    for label, run in [("bgmv-tm", lambda: dp.run_bgmv(B.LORA_BGMV_TOKEN_MAJOR)),
                       ("bgmv-am", lambda: dp.run_bgmv(B.LORA_BGMV_ADAPTER_MAJOR)),
                       ("fused-tm", lambda: dp.run_bgmv_fused(B.LORA_BGMV_TOKEN_MAJOR)),
                       ("fused-am", lambda: dp.run_bgmv_fused(B.LORA_BGMV_ADAPTER_MAJOR))]:
        say(f"quant bgmv {wq} {label}")
        y, v = run()
        torch.cuda.synchronize()
        check_v(dp, v, f"quant/{wq}/{label}")
        check_y(dp, y, want, f"quant/{wq}/{label}")


@pytest.mark.parametrize("wq", WQ)
def test_quant_bgmv_decode_full_size(wq):
    """The decode batch (256 tokens, 128 rank-16 adapters, 4096 -> 4096) with
    quantized rows: fused (the default decode path) and two-launch."""
    R = runner()
    p = wl.bgmv_decode(wq=wq)
    say(f"quant bgmv decode full size {wq}")
    dp = R.DeviceProblem(p)
    want = oracle_y(p)
    y, v = dp.run_bgmv_fused()
    y2, v2 = dp.run_bgmv()
    torch.cuda.synchronize()
    check_v(dp, v, f"quant-decode/{wq}/fused")
    check_y(dp, y, want, f"quant-decode/{wq}/fused")
    check_v(dp, v2, f"quant-decode/{wq}/two")
    check_y(dp, y2, want, f"quant-decode/{wq}/two")


@pytest.mark.parametrize("wq", WQ)
def test_quant_hetero_paged_full_size(wq):
    """The heterogeneous paged batch (4096 tokens, 64 requests, ranks 8..64,
    8192 -> 8192) with quantized rows, one launch per phase."""
    R = runner()
    p = wl.hetero_paged(wq=wq)
    say(f"quant hetero paged full size {wq}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv()
    torch.cuda.synchronize()
    check_v(dp, v, f"quant-hetero/{wq}")
    check_y(dp, y, oracle_y(p), f"quant-hetero/{wq}")


# ------------------------------------------------------------------ several projections, one launch
@pytest.mark.parametrize("wq", ["", "fp8"])
def test_fused_multi_projection(wq):
    """q, k and v deltas of one batch in one launch: bit-identical to three
    single-projection fused launches (index order and segment order), and each
    within the bf16 bound of the oracle."""
    R = runner()
    shapes = [("q", 1024), ("k", 256), ("v", 264)]
    p0 = wl.bgmv_decode(num_tokens=96, num_adapters=40, d_in=1024, d_out=1024, seed=31, wq=wq)
    probs = [p0]
    for i, (_, d_out) in enumerate(shapes[1:]):
        p = wl.make_problem(f"multi_{i}", None, None, [16] * 40, 1024, d_out, "bf16", 40 + i,
                            mode="bgmv", ids=p0.ids, wq=wq)
        p.x = p0.x
        probs.append(p)
    say(f"fused multi-projection wq={wq or 'bf16'}")
    dps = [R.DeviceProblem(p) for p in probs]
    x = dps[0].x
    ids = dps[0].ids
    for grouped in (False, True):
        order = dps[0].segments()[3] if grouped else None
        ys = [dp.y0.clone() for dp in dps]
        vs = [dp.new_v() for dp in dps]
        B.lora_bgmv_fused_multi([dp.weights for dp in dps], ids, x, ys, vs, token_order=order)
        singles = [dp.run_bgmv_fused(token_order=order) for dp in dps]
        torch.cuda.synchronize()
        for (y1, v1), y, v in zip(singles, ys, vs):
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
            assert torch.equal(v, v1)
    for dp, p, y in zip(dps, probs, ys):
        check_y(dp, y, oracle_y(p), f"multi {p.name}")


# ------------------------------------------------------------------ configs 3 and 4 at full size
@pytest.mark.parametrize("shape", ["q", "up"])
def test_sgmv_prefill_full_size(shape):
    """The prefill batch as benchmarked: 8192 tokens in 32 Zipf-length requests,
    automatic path policy, dense stacks; EVERY output row and every token's v
    against the oracle."""
    R = runner()
    p = wl.sgmv_prefill(shape=shape)
    say(f"prefill full size {shape}: {p.num_tokens} tokens, {p.d_in} -> {p.d_out}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv()
    torch.cuda.synchronize()
    check_v(dp, v, f"prefill {shape}")
    want = oracle.apply(p.x, p.y, p.ids, oracle_adapters(p), threads=_threads())
    check_y(dp, y, want, f"prefill {shape}, all {p.num_tokens} rows")


def test_hetero_paged_full_size():
    """The heterogeneous paged batch as benchmarked (bf16 rows, ranks 8..64,
    shuffled 16-row pages, automatic policy), every row against the oracle."""
    R = runner()
    p = wl.hetero_paged()
    say(f"hetero paged full size: {p.num_tokens} tokens, ranks {sorted(set(p.ranks.tolist()))}")
    dp = R.DeviceProblem(p)
    y, v = dp.run_sgmv()
    torch.cuda.synchronize()
    check_v(dp, v, "hetero full")
    check_y(dp, y, oracle_y(p), "hetero full")
