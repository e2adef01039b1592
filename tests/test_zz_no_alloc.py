"""lora_base_gemm_noalloc (split-k partials in the library's own device
scratch, nothing allocated by the call) against lora_base_gemm with a
caller-owned workspace, through the C ABI: two calls in a row, the second on a
smaller problem, each bit-identical to the workspace entry point (same kernels,
same k split), and each checked against the fp64 oracle on sampled rows."""
import numpy as np
import pytest

import oracle
from segmented_gather_gemm_segments_amd import binding as B
from segmented_gather_gemm_segments_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, std):
    return wl.bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    return wl.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_base_gemm_noalloc_matches_workspace_entry_point():
    B.lib()
    # the 70B k projection (80 tiles: k split 4 ways, 20 MiB of partials),
    # then a smaller ragged problem (15 tiles, also split 4 ways) that reuses
    # the scratch the first call left filled
    for m, n, k in [(1280, 1024, 8192), (300, 520, 4104)]:
        print(f"[case] base gemm noalloc m={m} n={n} k={k}", flush=True)
        ws_bytes = B.base_gemm_workspace_bytes(m, n, k)
        assert ws_bytes > 0, "the case must take the split-k path"
        assert ws_bytes <= 24 << 20
        rng = np.random.default_rng(m + n + k)
        x = _bf16(rng, (m, k), 1.0)
        w = _bf16(rng, (n, k), 1.0 / np.sqrt(k))
        xd, wd = _dev(x), _dev(w)
        y_ws = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        y_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = B.base_gemm_workspace(m, n, k)
        B.lora_base_gemm(xd, wd, y_ws, workspace=ws)
        B.lora_base_gemm_noalloc(xd, wd, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), (m, n, k)
        rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 6, replace=False)])).astype(np.int32)
        tok = np.repeat(rows, n).astype(np.int32)
        col = np.tile(np.arange(n, dtype=np.int32), rows.size)
        want = oracle.base_sampled(x, w, tok, col).reshape(rows.size, n)
        got = _host(y_na)[rows]
        scale = np.max(np.abs(want), axis=1, keepdims=True)
        err = float(np.max(np.abs(got - want) / scale))
        print(f"[case] sampled normwise error {err:.3e}", flush=True)
        assert err <= 2e-2
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0**-8 + 1e-3 * scale)


@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_base_gemm_noalloc_argument_errors():
    lib = B.lib()
    assert lib.lora_base_gemm_noalloc(B.LORA_F32, 8, 8, 8, 16, 16, 16, None) == B.LORA_EUNSUPPORTED
    assert lib.lora_base_gemm_noalloc(B.LORA_BF16, 8, 12, 8, 16, 16, 16, None) == B.LORA_EUNSUPPORTED
    assert lib.lora_base_gemm_noalloc(B.LORA_BF16, 8, 8, 8, None, 16, 16, None) == B.LORA_EINVAL
    assert lib.lora_base_gemm_noalloc(B.LORA_BF16, 8, 8, 8, 18, 16, 16, None) == B.LORA_EINVAL
    assert lib.lora_base_gemm_noalloc(B.LORA_BF16, 0, 8, 8, None, None, None, None) == B.LORA_OK
