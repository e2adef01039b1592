"""Adapter residency on the GPU: a sequence of decode batches over a universe
of adapters larger than the pools, every batch enqueued behind the previous
one with no host synchronisation, so uploads (on the cache's copy stream) may
evict adapters that earlier, still queued batches read.  Every batch's result
is checked against the fp64 oracle on the host copies of the adapters, to the
bf16 tolerance (normwise 2e-2; each element within one bf16 rounding plus
1e-4 of the row's scale)."""
import numpy as np
import pytest

import oracle
from segmented_gather_gemm_segments_amd import binding as B
from segmented_gather_gemm_segments_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PAGE_ROWS = 16


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _adapters(u):
    if u.wq:
        return oracle.Adapters.from_quantized(u.wq, u.a_rows, u.a_scales, u.bt_rows, u.bt_scales)
    return oracle.Adapters.from_stacks(u.a_rows, u.bt_rows)


def _pinned(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).pin_memory()


@pytest.mark.parametrize("wq,pinned", [("", True), ("fp8", True), ("", False)])
def test_churn_sequence_matches_oracle(wq, pinned):
    """pinned: host copies in pinned memory (gathered by the upload kernel);
    otherwise pageable numpy arrays (uploaded by asynchronous copies)."""
    num_ids, d_in, d_out = 24, 512, 776
    u, seq = wl.churn(num_ids=num_ids, batches=14, tokens=10, rank_choices=(8, 16, 32), d_in=d_in,
                      d_out=d_out, seed=21, wq=wq, no_adapter=0.1)
    pages = lambda a: -(-int(u.ranks[a]) // PAGE_ROWS)
    need = max(sum(pages(a) for a in set(ids[ids >= 0].tolist())) for ids, _, _ in seq)
    n_pages = need + 2                     # far below the universe's pages: churn
    assert n_pages < sum(pages(a) for a in range(num_ids))
    print(f"[case] churn wq={wq or 'bf16'} pinned={pinned}: {n_pages} pages per pool", flush=True)
    dev = torch.device("cuda:0")
    wf = {"": B.LORA_WFMT_PLAIN, "fp8": B.LORA_WFMT_FP8_E4M3}[wq]

    def pool(d, seed):
        if wf == B.LORA_WFMT_PLAIN:
            st = torch.full((n_pages, PAGE_ROWS, d), float("nan"), dtype=torch.bfloat16, device=dev)
            return B.Pool(st, PAGE_ROWS, shuffle_seed=seed)
        st = torch.full((n_pages, PAGE_ROWS, d), 0x7F, dtype=torch.uint8, device=dev)
        sc = torch.full((n_pages * PAGE_ROWS,), float("nan"), dtype=torch.float32, device=dev)
        return B.Pool(st, PAGE_ROWS, shuffle_seed=seed, weight_format=wf, scales=sc)

    pa, pb = pool(d_in, 3), pool(d_out, 4)
    r_max = 32
    mp = r_max // PAGE_ROWS
    pt_a = torch.empty((num_ids, mp), dtype=torch.int32, device=dev)
    pt_b = torch.empty((num_ids, mp), dtype=torch.int32, device=dev)
    rank = torch.empty(num_ids, dtype=torch.int32, device=dev)
    cache = B.Cache(pa, pb, num_ids, r_max, pt_a, pt_b, rank)
    host = _pinned if pinned else np.ascontiguousarray
    for a in range(num_ids):
        sa = host(u.a_scales[a]) if wq else None
        sb = host(u.bt_scales[a]) if wq else None
        cache.register(a, int(u.ranks[a]), host(u.a_rows[a]), host(u.bt_rows[a]), sa, sb)
    w = cache.weights(B.LORA_BF16, d_in, d_out, wf)
    st = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(st):
        for k, (ids, x, y) in enumerate(seq):
            ids_d = torch.from_numpy(ids).to(dev)
            x_d = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            y_d = torch.from_numpy(y.view(np.int16)).to(dev).view(torch.bfloat16)
            cache.prepare(ids, stream=st)
            if k % 2 == 0:
                B.lora_bgmv_fused(w, ids_d, x_d, y_d, None, stream=st)
            else:
                v = torch.zeros((ids.size, r_max), dtype=torch.float32, device=dev)
                B.lora_bgmv_shrink(w, ids_d, x_d, v, stream=st)
                B.lora_bgmv_expand(w, ids_d, v, y_d, stream=st)
            outs.append(y_d)
    torch.cuda.synchronize()
    s = cache.stats()
    print(f"[case] stats {s}", flush=True)
    assert s["evictions"] > 0 and s["misses"] > num_ids // 2
    ad = _adapters(u)
    for k, (ids, x, y) in enumerate(seq):
        want = oracle.apply(x, y, ids, ad)
        got = wl.bf16_to_f32(outs[k].cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
        den = np.max(np.abs(want), axis=1)
        err = float(np.max(np.max(np.abs(got - want), axis=1) / den))
        assert err <= 2e-2, (k, err)
        scale = den[:, None]
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0**-8 + 1e-4 * scale), k
        none = ids < 0
        assert np.array_equal(got[none], wl.bf16_to_f32(y[none]).astype(np.float64)), k
    cache.close()
