"""Adapter residency bookkeeping (LRU eviction, page accounting, errors) in
host-only mode: no GPU.  The device side (uploads, ordering against the
compute stream, results through the cached page tables) is tested in
test_residency_gpu.py."""
import numpy as np
import pytest

from segmented_gather_gemm_segments_amd import binding as B


class _Fake:
    """Stand-in for a device tensor: host-only caches never touch storage."""

    def __init__(self, n, pr, w):
        import torch
        self.shape = (n, pr, w)
        self.buf = np.zeros(1, np.uint8)
        self.dtype = torch.bfloat16

    def data_ptr(self):
        return self.buf.ctypes.data


def _cache(pages_a=8, pages_b=8, shared=False, num_ids=32, r_max=32, seed=5):
    pa = B.Pool(_Fake(pages_a, 16, 64), 16, shuffle_seed=seed)
    pb = pa if shared else B.Pool(_Fake(pages_b, 16, 64), 16, shuffle_seed=seed + 1)
    c = B.Cache(pa, pb, num_ids, r_max, host_only=True)
    return c, pa, pb


def _register(c, ranks):
    rows = np.zeros(1, np.uint16)
    for i, r in enumerate(ranks):
        c.register(i, int(r), rows, rows)


class LruModel:
    """The policy restated: hits refresh; misses evict the least recently used
    adapters outside the batch until the batch's pages fit."""

    def __init__(self, ranks, pages_a, pages_b, shared, page_rows=16):
        self.ranks, self.shared = ranks, shared
        self.free_a, self.free_b = pages_a, pages_b
        self.res = {}          # id -> stamp
        self.t = 0
        self.pr = page_rows
        self.hits = self.misses = self.evictions = 0

    def np_(self, a):
        return -(-int(self.ranks[a]) // self.pr)

    def fits(self, need, fa, fb):
        return need * 2 <= fa if self.shared else (need <= fa and need <= fb)

    def prepare(self, ids):
        self.t += 1
        batch = sorted(set(int(i) for i in ids if i >= 0))
        miss = [a for a in batch if a not in self.res]
        need = sum(self.np_(a) for a in miss)
        fa, fb = self.free_a, self.free_b
        victims = []
        for a, _ in sorted(((a, s) for a, s in self.res.items() if a not in batch), key=lambda q: (q[1], q[0])):
            if self.fits(need, fa, fb):
                break
            victims.append(a)
            fa += self.np_(a) * (2 if self.shared else 1)
            fb += self.np_(a)
        if not self.fits(need, fa, fb):
            return False
        for a in victims:
            del self.res[a]
        self.evictions += len(victims)
        self.free_a, self.free_b = fa - need * (2 if self.shared else 1), fb - need
        for a in batch:
            self.res[a] = self.t
        self.hits += len(batch) - len(miss)
        self.misses += len(miss)
        return True


@pytest.mark.parametrize("shared", [False, True])
def test_lru_matches_model(shared):
    rng = np.random.default_rng(11)
    ranks = rng.choice([8, 16, 24, 32], size=32)
    pages = 24
    c, pa, pb = _cache(pages, pages, shared=shared)
    _register(c, ranks)
    m = LruModel(ranks, pages, pages, shared)
    zipf = 1.0 / np.arange(1, 33) ** 1.1
    zipf /= zipf.sum()
    for step in range(300):
        ids = rng.choice(32, size=int(rng.integers(1, 10)), p=zipf)
        if rng.random() < 0.2:
            ids = np.concatenate([ids, [-1]])
        ok = m.prepare(ids)
        if ok:
            c.prepare(ids, host_only=True)
        else:
            with pytest.raises(B.LoraError) as e:
                c.prepare(ids, host_only=True)
            assert e.value.status == B.LORA_ENOMEM
        st = c.stats()
        assert st["resident"] == len(m.res)
        assert (st["hits"], st["misses"], st["evictions"]) == (m.hits, m.misses, m.evictions)
        assert st["free_pages_a"] == pa.num_free() == m.free_a
        if not shared:
            assert st["free_pages_b"] == m.free_b
        for a in range(32):
            pg_a, pg_b = c.pages(a)
            assert (pg_a.size > 0) == (a in m.res)
            if a in m.res:
                assert pg_a.size == pg_b.size == m.np_(a)
        # every resident adapter's pages are distinct across the pool(s)
        allp = np.concatenate([c.pages(a)[0] for a in m.res] + ([c.pages(a)[1] for a in m.res] if shared else [np.zeros(0, np.int32)]))
        assert len(set(allp.tolist())) == allp.size


def test_cache_errors_and_atomic_failure():
    c, pa, pb = _cache(4, 4, r_max=64)
    _register(c, [16, 32, 32, 64])
    with pytest.raises(B.LoraError) as e:
        c.prepare([5], host_only=True)           # not registered
    assert e.value.status == B.LORA_ERANGE
    with pytest.raises(B.LoraError) as e:
        c.prepare([40], host_only=True)          # outside the id space
    assert e.value.status == B.LORA_ERANGE
    c.prepare([0, 1], host_only=True)            # 1 + 2 pages
    before = c.stats()
    with pytest.raises(B.LoraError) as e:
        c.prepare([1, 2, 3], host_only=True)     # 2 + 2 + 4 pages > 4
    assert e.value.status == B.LORA_ENOMEM
    assert c.stats() == before                    # nothing changed
    c.prepare([3], host_only=True)                # evicts 0 then 1 (LRU order), takes all 4 pages
    st = c.stats()
    assert st["resident"] == 1 and st["evictions"] == 2 and st["free_pages_a"] == 0
    with pytest.raises(B.LoraError) as e:
        c.register(3, 16, np.zeros(1), np.zeros(1))   # resident adapters keep their rows
    assert e.value.status == B.LORA_EINVAL


def test_shuffled_pool_scatters_pages():
    c, pa, pb = _cache(64, 64, num_ids=16, r_max=64)
    _register(c, [64] * 16)
    c.prepare(list(range(16)), host_only=True)
    st = c.stats()
    assert st["resident"] == 16 and st["scattered"] >= 12   # churn-like placement
