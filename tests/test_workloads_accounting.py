"""Input generators (determinism, shapes, distributions) and the benchmark's
algorithmic byte counter (pinned to the page's Llama-3-70B rank-16 table).  CPU only."""
import os

import numpy as np

from conftest import golden_path
from segmented_gather_gemm_segments_amd import accounting as acc
from segmented_gather_gemm_segments_amd import workloads as wl


def _golden_table():
    rows, totals = {}, {}
    for line in open(golden_path("adapter_bytes_70b_r16.txt")):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        if len(parts) == 4:
            rows[parts[0]] = (int(parts[1]), int(parts[2]), int(parts[3]))
        else:
            totals[parts[0]] = int(parts[1])
    return rows, totals


def test_byte_counter_matches_70b_table():
    rows, totals = _golden_table()
    for name, (d_in, d_out, want) in rows.items():
        assert acc.adapter_matrix_bytes(d_in, d_out, 16, 2) == want, name
    layer = acc.adapter_layer_bytes([(di, do) for di, do, _ in rows.values()], 16, 2)
    assert layer == totals["sum_per_layer"]
    total = layer * totals["layers"]
    assert round(total / 2**20) == totals["total_mib"]
    attn = acc.adapter_layer_bytes([rows[k][:2] for k in ("Q", "O", "K", "V")], 16, 2)
    assert round(attn * totals["layers"] / 2**20) == totals["attention_only_mib"]
    # the generator's 70B layer shapes are the table's shapes
    assert sorted((di, do) for _, di, do in wl.LAYER_70B) == sorted(v[:2] for v in rows.values())


def test_byte_counter_linear_in_rank_and_8b_crosscheck():
    shapes70 = [(di, do) for _, di, do in wl.LAYER_70B]
    b16 = acc.adapter_layer_bytes(shapes70, 16)
    for r in (8, 32, 64):
        assert acc.adapter_layer_bytes(shapes70, r) * 16 == b16 * r
    shapes8 = [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336),
               (4096, 14336), (14336, 4096)]
    assert acc.adapter_layer_bytes(shapes8, 16) == 2_621_440
    assert acc.adapter_layer_bytes(shapes8, 16) * 32 == 80 * 2**20


def test_per_launch_bytes():
    ids = np.array([0, 0, 1, -1, 2], np.int32)
    ranks = np.array([8, 16, 32], np.int32)
    # 4 adapted tokens, distinct ranks 8+16+32, per-token ranks 8+8+16+32
    assert acc.shrink_bytes(ids, ranks, 100, 2) == 4 * 100 * 2 + 56 * 100 * 2 + 64 * 4
    assert acc.expand_bytes(ids, ranks, 50, 2) == 64 * 4 + 56 * 50 * 2 + 2 * 4 * 50 * 2
    assert acc.shrink_flops(ids, ranks, 100) == 2 * 100 * 64


def test_bf16_rounding_is_rne():
    f = np.array([1.0, 1.00390625, 1.01171875, -3.0e-3, 65504.0, 1e-40], np.float32)
    bits = wl.bf16_bits(f)
    back = wl.bf16_to_f32(bits)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1.0
    assert back[1] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> the even one, 1+2^-6
    assert back[2] == np.float32(1.015625)
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    b = wl.bf16_to_f32(wl.bf16_bits(x))
    assert np.all(np.abs(b - x) <= np.abs(x) * 2.0**-8)


def test_generators_are_deterministic_and_shaped():
    p1, p2 = wl.tiny_sgmv(), wl.tiny_sgmv()
    assert np.array_equal(p1.x, p2.x) and np.array_equal(p1.a_rows[2], p2.a_rows[2])
    assert p1.ids.tolist() == [2] * 16 + [0] + [1] * 31
    assert p1.x.dtype == np.float32 and p1.d_in == 512 and p1.r_max == 8
    d = wl.bgmv_decode(num_tokens=64, num_adapters=16, d_in=256, d_out=128)
    assert d.x.dtype == np.uint16 and d.ids.min() >= 0 and d.ids.max() < 16
    h = wl.hetero_paged(num_tokens=512, num_segments=16, d=256)
    assert set(h.ranks.tolist()) <= {8, 16, 32, 64}
    assert h.seg_lengths.sum() == 512 and h.seg_lengths.min() >= 1
    assert sorted(h.seg_ids.tolist()) == list(range(16))


def test_zipf_lengths():
    rng = np.random.default_rng(1)
    lens = wl.zipf_lengths(rng, 8192, 32)
    assert lens.sum() == 8192 and lens.min() >= 1 and lens.size == 32
    # the largest request is near 8192 / H(32, 1.1) = 2324
    assert 1900 < lens.max() < 2800


def test_full_size_configs_shapes():
    p = wl.sgmv_prefill(shape="q")
    assert p.num_tokens == 8192 and np.unique(p.ids).size == 32 and p.num_adapters == 64
    ids = wl.layer_batch_ids()
    assert ids.size == 1280 and np.unique(ids[:256]).size == 256 and np.all(ids[256:] == 0)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before
    touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode != 0
    assert "one GPU only" in res.stdout + res.stderr
