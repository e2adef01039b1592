"""GPU parity of the base projection (lora_base_gemm) and of the 70B-shape
decoder-layer projections (base y = x W^T, then the SGMV delta added to it),
through the C ABI, against the fp64 oracle.  Normwise tolerance 2e-2 (bf16
I/O, fp32 accumulation); each sampled element also within one bf16 rounding
of the exact value plus 1e-3 of its row's scale."""
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


def bf16_host(t):
    return wl.bf16_to_f32(t.detach().view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def check_sampled(got, want, row_scale, label):
    """got/want: values at sampled pairs; row_scale: max |row| of the exact output."""
    err = float(np.max(np.abs(got - want) / row_scale))
    say(f"{label}: sampled normwise error {err:.3e}")
    assert err <= 2e-2, label
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0**-8 + 1e-3 * row_scale), label


def rand_bf16(rng, shape, std):
    return wl.bf16_bits((rng.standard_normal(shape, dtype=np.float32) * np.float32(std)))


@pytest.mark.parametrize("split", [False, True], ids=["whole_k", "split_k"])
@pytest.mark.parametrize("m,n,k", [(1, 8, 8), (77, 264, 520), (200, 136, 1032), (129, 128, 64),
                                   (256, 1024, 768), (300, 520, 4104),
                                   (256, 256, 512), (128, 1024, 4096), (384, 128, 192)])
def test_base_gemm_small_full(m, n, k, split):
    """Every output of ragged shapes (partial tiles in m, n and k), and of
    whole-tile shapes (m, n multiples of 128, k of 64: the direct-to-LDS
    kernel with a k-step of 32), without and with a workspace (with one, these
    few-tile grids split k into 2 or 4 slices, except where k is too short to
    split)."""
    rng = np.random.default_rng(m * 7 + n + k)
    x = rand_bf16(rng, (m, k), 1.0)
    w = rand_bf16(rng, (n, k), 1.0 / np.sqrt(k))
    ws = B.base_gemm_workspace(m, n, k) if split else None
    if split and k >= 512:
        assert ws is not None, "a few-tile grid with k >= 512 splits k"
    say(f"base gemm full m={m} n={n} k={k} workspace={0 if ws is None else ws.numel() * 4}")
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    yd = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    if ws is not None:
        ws.fill_(float("nan"))  # every partial the reduction reads must be written
    B.lora_base_gemm(xd, wd, yd, workspace=ws)
    torch.cuda.synchronize()
    got = bf16_host(yd)
    tok, col = np.meshgrid(np.arange(m, dtype=np.int32), np.arange(n, dtype=np.int32), indexing="ij")
    want = oracle.base_sampled(x, w, tok.ravel(), col.ravel()).reshape(m, n)
    scale = np.maximum(np.max(np.abs(want), axis=1, keepdims=True), 1e-30)
    check_sampled(got, want, np.broadcast_to(scale, want.shape), f"gemm {m}x{n}x{k}")


def test_base_gemm_large_grid_sampled():
    """A whole-tile grid of 1536 tiles (six per compute unit: the direct-to-LDS
    kernel with a k-step of 64), checked on 48 full rows."""
    m, n, k = 1536, 16384, 192
    rng = np.random.default_rng(1536)
    x = rand_bf16(rng, (m, k), 1.0)
    w = rand_bf16(rng, (n, k), 1.0 / np.sqrt(k))
    say(f"base gemm large grid m={m} n={n} k={k}")
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    yd = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    assert B.base_gemm_workspace_bytes(m, n, k) == 0
    B.lora_base_gemm(xd, wd, yd)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 127, 128, m - 1], rng.choice(m, 44, replace=False)]))
    got = bf16_host(yd)[rows]
    tok, col = np.meshgrid(rows.astype(np.int32), np.arange(n, dtype=np.int32), indexing="ij")
    want = oracle.base_sampled(x, w, tok.ravel(), col.ravel()).reshape(rows.size, n)
    scale = np.maximum(np.max(np.abs(want), axis=1, keepdims=True), 1e-30)
    check_sampled(got, want, np.broadcast_to(scale, want.shape), f"gemm {m}x{n}x{k}")


def test_base_gemm_errors():
    lib = B.lib()
    assert lib.lora_base_gemm(B.LORA_F32, 8, 8, 8, 16, 16, 16, None, 0, None) == B.LORA_EUNSUPPORTED
    assert lib.lora_base_gemm(B.LORA_BF16, 8, 12, 8, 16, 16, 16, None, 0, None) == B.LORA_EUNSUPPORTED
    assert lib.lora_base_gemm(B.LORA_BF16, 8, 8, 8, None, 16, 16, None, 0, None) == B.LORA_EINVAL
    assert lib.lora_base_gemm(B.LORA_BF16, 8, 8, 8, 18, 16, 16, None, 0, None) == B.LORA_EINVAL
    assert lib.lora_base_gemm(B.LORA_BF16, 8, 8, 8, 16, 16, 16, 24, 64, None) == B.LORA_EINVAL
    assert lib.lora_base_gemm(B.LORA_BF16, 8, 8, 8, 16, 16, 16, None, -1, None) == B.LORA_EINVAL
    assert lib.lora_base_gemm(B.LORA_BF16, 0, 8, 8, None, None, None, None, 0, None) == B.LORA_OK
    # the 70B shapes: only the 80-tile k/v projections (1280 x 1024) split, 4 ways
    assert B.base_gemm_workspace_bytes(1280, 1024, 8192) == 4 * 1280 * 1024 * 4
    assert B.base_gemm_workspace_bytes(1280, 8192, 8192) == 0
    assert B.base_gemm_workspace_bytes(1280, 28672, 8192) == 0
    assert B.base_gemm_workspace_bytes(0, 8, 8) == 0


# tokens whose full output rows are checked: decode tokens (one-token
# segments), the decode token sharing adapter 0 with the prefill request, and
# prefill tokens at the segment's start, middle and end
def _check_rows(p):
    rows = [0, 1, 77, 200, 255, 256, 257, 700, 1100, 1279]
    rows.append(int(np.flatnonzero(p.ids[:256] == 0)[0]))
    return np.array(sorted(set(rows)), dtype=np.int32)


def _rows_close(got, want, label, elementwise=True):
    scale = np.max(np.abs(want), axis=1, keepdims=True)
    err = float(np.max(np.max(np.abs(got - want), axis=1, keepdims=True) / scale))
    say(f"{label}: normwise error {err:.3e} over {want.shape[0]} full rows")
    assert err <= 2e-2, label
    if elementwise:
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0**-8 + 1e-3 * scale), label


def _threads():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("name", [n for n, _, _ in wl.LAYER_70B])
def test_layer70b_projection(name):
    """One projection of the 70B-shape layer at full size (1280 tokens: 256
    decode tokens on 256 rank-16 adapters plus a 1024-token prefill request on
    adapter 0), for each of the seven projections: the base GEMM checked on
    sampled full rows; then the SGMV delta (segmented mode, automatic path:
    one 1025-token MFMA segment, 255 gather segments) added to the GPU's base
    output, checked on EVERY row against the oracle with that same base output
    as y_in, and its v on every token; and the per-token (BGMV) delta and the
    segmented gather delta on every row too (the two shrinks split d_in over
    different numbers of waves, so they agree within one bf16 rounding, not
    bit for bit)."""
    R = runner()
    p = wl.layer_projection(name)
    say(f"layer70b {name}: {p.d_in} -> {p.d_out}")
    dp = R.DeviceProblem(p)
    y_base = dp.run_base()
    torch.cuda.synchronize()
    rows = _check_rows(p)
    yb = bf16_host(y_base)
    tok = np.repeat(rows, p.d_out).astype(np.int32)
    col = np.tile(np.arange(p.d_out, dtype=np.int32), rows.size)
    want_b = oracle.base_sampled(p.x, p.extra["w"], tok, col).reshape(rows.size, p.d_out)
    _rows_close(yb[rows], want_b, f"{name} base")
    # delta on top of the GPU's base output (the oracle takes the same y_in)
    y, v = dp.run_sgmv(B.LORA_PATH_AUTO, y=y_base.clone())
    torch.cuda.synchronize()
    got = bf16_host(y)
    ad = oracle.Adapters.from_stacks(p.a_rows, p.bt_rows)
    yb_bits = y_base.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.apply(p.x, yb_bits, p.ids, ad, threads=_threads())
    _rows_close(got, want, f"{name} base+delta, all {p.num_tokens} rows")
    want_v = oracle.shrink(p.x, p.ids, ad, dp.r_max)
    got_v = v.cpu().numpy().astype(np.float64)
    err_v = float(np.max(np.max(np.abs(got_v - want_v), axis=1) / np.max(np.abs(want_v), axis=1)))
    say(f"{name} v: normwise error {err_v:.3e} over all {p.num_tokens} tokens")
    assert err_v <= 1e-4, name
    # per-token mode and the segmented gather path on the same batch
    y2, _ = dp.run_bgmv(B.LORA_BGMV_AUTO, y=y_base.clone())
    y3, _ = dp.run_sgmv(B.LORA_PATH_GATHER, y=y_base.clone())
    torch.cuda.synchronize()
    g2, g3 = bf16_host(y2), bf16_host(y3)
    _rows_close(g2, want, f"{name} bgmv base+delta, all rows")
    _rows_close(g3, want, f"{name} sgmv gather base+delta, all rows")
    scale = np.max(np.abs(g3), axis=1, keepdims=True)
    assert np.all(np.abs(g2 - g3) <= np.abs(g3) * 2.0**-7 + 1e-4 * scale), f"{name} bgmv vs gather"
