"""HIP graph capture of the hot-path calls through the C ABI: each call is
captured once and the graph replayed several times, with the program's own
eager work and device synchronisations between the replays; every replay must
equal the eager call bit for bit (the kernels' reduction orders are fixed and
none of them records a memset).  Covers the fused decode launch, the segmented
shrink + expand pair and the tiled shrink + expand on the paged heterogeneous
batch, three projections' deltas forked onto three streams and joined with
events, and the base GEMM with and without its split-k workspace (two
launches per call)."""
import numpy as np
import pytest

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


def replay_and_check(stream, capture, reset, outs, wants, label, replays=3):
    """Capture `capture()` on `stream`, then replay it `replays` times, each
    after `reset()` and some unrelated eager work, comparing `outs` to `wants`."""
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        capture()
    torch.cuda.synchronize()
    for i in range(replays):
        reset()
        scratch = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
        _ = float(scratch.sum())  # eager work and a synchronisation between replays
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, wants):
            assert torch.equal(o, w), f"{label}: replay {i} differs from the eager call"
    say(f"{label}: {replays} replays equal the eager call")


def test_graph_fused_decode():
    R = runner()
    dp = R.DeviceProblem(wl.config(2))
    say("graph fused decode: 256 tokens, 128 adapters, segment order")
    y_e, _ = dp.run_bgmv_fused(grouped=True)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    y_g = dp.y0.clone()
    call = B.prepare_bgmv_fused(dp.weights, dp.ids, dp.x, y_g, None, B.LORA_BGMV_AUTO, stream=st,
                                token_order=dp.segments()[3])
    replay_and_check(st, call, lambda: y_g.copy_(dp.y0), [y_g], [y_e], "fused decode")


def test_graph_sgmv_paged_hetero():
    R = runner()
    dp = R.DeviceProblem(wl.config(4))
    say("graph sgmv: 4096 tokens, 64 segments, ranks 8..64, paged pool")
    y_e, v_e = dp.run_sgmv()
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    y_g, v_g = dp.y0.clone(), dp.new_v()
    _, _, _, perm_d = dp.segments()
    sp = dp.plan(B.LORA_PHASE_SHRINK)
    ep = dp.plan(B.LORA_PHASE_EXPAND)
    shrink, expand = B.prepare_sgmv(dp.weights, perm_d, sp, ep, dp.x, v_g, y_g, stream=st)

    def capture():
        shrink()
        expand()

    def reset():
        y_g.copy_(dp.y0)
        v_g.zero_()

    replay_and_check(st, capture, reset, [y_g, v_g], [y_e, v_e], "sgmv shrink+expand")


def test_graph_sgmv_tiled():
    """The tiled shrink (tile launch + slice reduction) and the expand."""
    R = runner()
    dp = R.DeviceProblem(wl.config(4))
    say("graph tiled sgmv: 4096 tokens, 64 segments, ranks 8..64, paged pool")
    y_e, v_e = dp.run_sgmv(tiled=True)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    y_g, v_g = dp.y0.clone(), dp.new_v()
    _, _, _, perm_d = dp.segments()
    items, ks, ws = dp.plan_tiled()
    assert ks > 1
    ep = dp.plan(B.LORA_PHASE_EXPAND)
    shrink, expand = B.prepare_sgmv_tiled(dp.weights, perm_d, items, ks, ws, ep, dp.x, v_g, y_g, stream=st)

    def capture():
        shrink()
        expand()

    def reset():
        y_g.copy_(dp.y0)
        v_g.zero_()
        ws.fill_(float("nan"))  # the partials of every replay are rewritten before they are read

    replay_and_check(st, capture, reset, [y_g, v_g], [y_e, v_e], "tiled shrink+expand")


def test_graph_layer_group_on_three_streams():
    """The q, k and v deltas of the 70B layer, each on its own stream, forked
    from and joined back to the capture stream with events (as the bench's
    layer step runs them): every replay equals the three eager calls."""
    R = runner()
    dps = [R.DeviceProblem(wl.layer_projection(n, with_base=False)) for n in ("q", "k", "v")]
    say("graph layer q|k|v on three streams")
    wants = []
    for dp in dps:
        y, v = dp.run_sgmv()
        wants += [y, v]
    torch.cuda.synchronize()
    main = torch.cuda.Stream()
    lanes = [main, torch.cuda.Stream(), torch.cuda.Stream()]
    outs, calls = [], []
    for dp, ls in zip(dps, lanes):
        y_g, v_g = dp.y0.clone(), dp.new_v()
        _, _, _, perm_d = dp.segments()
        sp, ep = dp.plan(B.LORA_PHASE_SHRINK), dp.plan(B.LORA_PHASE_EXPAND)
        calls.append(B.prepare_sgmv(dp.weights, perm_d, sp, ep, dp.x, v_g, y_g, stream=ls))
        outs += [y_g, v_g]

    def capture():
        fork = torch.cuda.Event()
        fork.record(main)
        for ls in lanes[1:]:
            ls.wait_event(fork)
        for c in calls:
            c[0]()
            c[1]()
        for ls in lanes[1:]:
            done = torch.cuda.Event()
            done.record(ls)
            main.wait_event(done)

    def reset():
        for dp, j in zip(dps, range(0, 6, 2)):
            outs[j].copy_(dp.y0)
            outs[j + 1].zero_()

    replay_and_check(main, capture, reset, outs, wants, "layer q|k|v streams")


@pytest.mark.parametrize("m,n,k,split", [(256, 1024, 4096, True), (300, 520, 4104, True),
                                         (1280, 1024, 8192, True), (256, 1024, 4096, False)])
def test_graph_base_gemm(m, n, k, split):
    rng = np.random.default_rng(m + n + k)
    x = torch.from_numpy(wl.bf16_bits(rng.standard_normal((m, k), dtype=np.float32)).view(np.int16))
    w = torch.from_numpy(wl.bf16_bits((rng.standard_normal((n, k), dtype=np.float32)
                                       * np.float32(1 / np.sqrt(k)))).view(np.int16))
    xd, wd = x.view(torch.bfloat16).cuda(), w.view(torch.bfloat16).cuda()
    ws = B.base_gemm_workspace(m, n, k) if split else None
    if split:
        assert ws is not None
    say(f"graph base gemm m={m} n={n} k={k} workspace={0 if ws is None else ws.numel() * 4}")
    y_e = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    B.lora_base_gemm(xd, wd, y_e, workspace=ws)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    y_g = torch.empty_like(y_e)
    call = B.prepare_base_gemm(xd, wd, y_g, workspace=ws, stream=st)

    def reset():
        y_g.fill_(float("nan"))
        if ws is not None:
            ws.fill_(float("nan"))

    replay_and_check(st, call, reset, [y_g], [y_e], f"base gemm {m}x{n}x{k}")
