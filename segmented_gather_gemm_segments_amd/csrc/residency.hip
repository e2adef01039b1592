// Adapter residency: an LRU cache of adapters over the two page pools (A rows
// and B^T rows), filled from caller-owned host copies.
//
// The tiering follows "Multi-LoRA serving: the single translator with a
// thousand glossaries" (TL;DR and section "Operational pitfalls": adapters
// paged in a shared pool, cold start, fragmentation; the figure of the typical
// stack: hot adapters in the HBM pool, warm ones in host RAM with LRU eviction
// and asynchronous host-to-device copies on use) and "Multi-LoRA Inference
// Serving: Serving Thousands of Fine-Tuned Models on One GPU" (the paragraph
// on vLLM's fixed-size adapter pool that swaps adapters in and out as
// requests arrive, and the paragraph on tiering).
//
// lora_cache_prepare(batch ids) makes every adapter of a batch resident:
//   * hits only refresh their LRU stamp;
//   * misses take pages from the pools, evicting least-recently-used adapters
//     that the batch does not use until the pages fit (or fail with nothing
//     changed) -- among them first those whose last batch has completed, so
//     that an upload rarely has to wait for a batch still in flight;
//   * uploads (rows, row scales, page-table rows, ranks) go on the cache's own
//     copy stream, so they overlap with kernels already queued on the compute
//     stream; the compute stream then waits for them with an event;
//   * pages freed by an eviction are rewritten only after the last batch that
//     used the evicted adapter has finished: each prepare records an event on
//     the compute stream (after everything queued so far, i.e. after the
//     previous batch's kernels) that becomes the last-use mark of the
//     previous batch's adapters, and the copy stream waits on the evicted
//     adapters' marks -- which, the adapters being least recently used, have
//     normally long completed, so the wait costs nothing.
// Page-table rows and ranks are written by a small kernel whose entries travel
// as kernel arguments, so no host staging buffer can change under a pending
// copy.  The rows themselves are gathered by one copy kernel per prepare that
// reads the pinned host copies directly (pinned host memory is addressable from
// the GPU) and writes every page -- one launch instead of one DMA request per
// page and pool, whose per-request cost dominated; host copies that are not
// device-addressable (pageable memory) are uploaded with plain asynchronous
// copies instead.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <memory>
#include <vector>

#include "lora_internal.h"

using namespace lora;

namespace {

constexpr int kEntryPages = 8;   // pages per table entry
constexpr int kTableBatch = 16;  // entries per update launch

struct TableEntry {
  int32_t id, rank, first, count;  // pages [first, first + count) of adapter id; rank < 0: keep
  int32_t pa[kEntryPages];
  int32_t pb[kEntryPages];
};

struct TableUpdate {
  int32_t n, max_pages;
  int32_t *pt_a, *pt_b, *rank;
  TableEntry e[kTableBatch];
};

__global__ __launch_bounds__(kTableBatch * kEntryPages) void table_update_kernel(TableUpdate u) {
  const int i = threadIdx.x / kEntryPages, p = threadIdx.x % kEntryPages;
  if (i >= u.n) return;
  const TableEntry &e = u.e[i];
  if (p < e.count) {
    const int64_t at = (int64_t)e.id * u.max_pages + e.first + p;
    u.pt_a[at] = e.pa[p];
    u.pt_b[at] = e.pb[p];
  }
  if (p == 0 && e.rank >= 0) u.rank[e.id] = e.rank;
}

// Upload jobs: `bytes` (a multiple of 4) from src (device-addressable host
// memory) to dst (a page of a pool, or its scales).  Block b of the launch
// copies slice b % kSlices of job b / kSlices.
struct CopyJob {
  const char *src;
  char *dst;
  int64_t bytes;
};
constexpr int kCopyJobs = 64;
constexpr int kSlices = 8;
struct CopyBatch {
  int32_t n;
  CopyJob j[kCopyJobs];
};

__global__ __launch_bounds__(256) void upload_kernel(CopyBatch b) {
  const int ji = blockIdx.x / kSlices, sl = blockIdx.x % kSlices;
  if (ji >= b.n) return;
  const CopyJob &j = b.j[ji];
  const bool vec = (((uintptr_t)j.src | (uintptr_t)j.dst) & 15u) == 0;
  const int64_t n16 = vec ? j.bytes >> 4 : 0;
  // 16-byte units, four in flight per thread
  const int64_t stride = (int64_t)kSlices * blockDim.x;
  int64_t i = (int64_t)sl * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = reinterpret_cast<const uint4 *>(j.src)[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) reinterpret_cast<uint4 *>(j.dst)[i + u * stride] = q[u];
  }
  for (; i < n16; i += stride) reinterpret_cast<uint4 *>(j.dst)[i] = reinterpret_cast<const uint4 *>(j.src)[i];
  // the rest (or everything, unaligned) in 4-byte words
  for (int64_t k = (n16 << 2) + (int64_t)sl * blockDim.x + threadIdx.x; k < (j.bytes >> 2); k += stride)
    reinterpret_cast<uint32_t *>(j.dst)[k] = reinterpret_cast<const uint32_t *>(j.src)[k];
}

__global__ void fill_kernel(int32_t *p, int64_t n, int32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

struct Event {
  hipEvent_t e = nullptr;
  ~Event() {
    if (e) (void)hipEventDestroy(e);
  }
};

struct Entry {
  bool registered = false, resident = false;
  bool mapped = false;                // host copies readable by the GPU (pinned)
  int32_t rank = 0;
  const void *host_a = nullptr, *host_b = nullptr;
  const float *sc_a = nullptr, *sc_b = nullptr;
  const char *dev_a = nullptr, *dev_b = nullptr, *dev_sa = nullptr, *dev_sb = nullptr;
  std::vector<int32_t> pages_a, pages_b;
  uint64_t stamp = 0;                 // LRU: last batch that used it
  std::shared_ptr<Event> last_use;    // completes after that batch's kernels
};

}  // namespace

struct lora_cache {
  lora_pool *pool_a, *pool_b;
  int32_t num_ids, r_max, page_rows, max_pages, flags;
  int64_t row_bytes_a, row_bytes_b;
  int32_t *pt_a, *pt_b, *rank;
  hipStream_t copy = nullptr;
  std::vector<Entry> ids;
  std::vector<int32_t> last_batch;    // adapters of the previous prepare
  uint64_t batch = 0;
  lora_cache_stats stats{};
  bool host_only() const { return flags & LORA_CACHE_HOST_ONLY; }
};

namespace {

int64_t pool_row_bytes(int32_t width, int32_t dtype, int32_t wf) {
  if (wf == LORA_WFMT_FP8_E4M3) return width;
  if (wf == LORA_WFMT_INT4) return width / 2;
  return (int64_t)width * (dtype == LORA_BF16 ? 2 : 4);
}

lora_status flush_updates(lora_cache *c, std::vector<TableEntry> &pending) {
  if (c->host_only()) {
    pending.clear();
    return LORA_OK;
  }
  for (size_t i0 = 0; i0 < pending.size(); i0 += kTableBatch) {
    TableUpdate u{};
    u.n = (int32_t)std::min<size_t>(kTableBatch, pending.size() - i0);
    u.max_pages = c->max_pages;
    u.pt_a = c->pt_a;
    u.pt_b = c->pt_b;
    u.rank = c->rank;
    for (int i = 0; i < u.n; ++i) u.e[i] = pending[i0 + (size_t)i];
    hipLaunchKernelGGL(table_update_kernel, dim3(1), dim3(kTableBatch * kEntryPages), 0, c->copy, u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "page-table update launch");
  }
  pending.clear();
  return LORA_OK;
}

// Table entries (rank and page ids, in groups of kEntryPages) for adapter id;
// pages of -1 for an eviction.
void table_entries(const lora_cache *c, int32_t id, int32_t rank, const std::vector<int32_t> &pa,
                   const std::vector<int32_t> &pb, bool evict, std::vector<TableEntry> &out) {
  for (int32_t first = 0; first < c->max_pages; first += kEntryPages) {
    TableEntry e{};
    e.id = id;
    e.rank = first == 0 ? rank : -1;
    e.first = first;
    e.count = std::min(kEntryPages, c->max_pages - first);
    for (int p = 0; p < e.count; ++p) {
      const size_t k = (size_t)(first + p);
      e.pa[p] = (!evict && k < pa.size()) ? pa[k] : -1;
      e.pb[p] = (!evict && k < pb.size()) ? pb[k] : -1;
    }
    out.push_back(e);
  }
}

// Device address of host memory, or nullptr when it is not device-addressable
// (pageable).  Clears the error a failed query leaves behind.
const char *device_view(const void *p) {
  if (!p) return nullptr;
  hipPointerAttribute_t at;
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type != hipMemoryTypeHost || !at.devicePointer) return nullptr;
  return (const char *)at.devicePointer;
}

lora_status flush_copies(lora_cache *c, std::vector<CopyJob> &jobs) {
  for (size_t i0 = 0; i0 < jobs.size(); i0 += kCopyJobs) {
    CopyBatch b{};
    b.n = (int32_t)std::min<size_t>(kCopyJobs, jobs.size() - i0);
    for (int i = 0; i < b.n; ++i) b.j[i] = jobs[i0 + (size_t)i];
    hipLaunchKernelGGL(upload_kernel, dim3(b.n * kSlices), dim3(256), 0, c->copy, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "upload launch");
  }
  jobs.clear();
  return LORA_OK;
}

bool consecutive(const std::vector<int32_t> &p) {
  for (size_t i = 1; i < p.size(); ++i)
    if (p[i] != p[i - 1] + 1) return false;
  return true;
}

}  // namespace

extern "C" lora_status lora_cache_create(lora_pool *pool_a, lora_pool *pool_b, int32_t num_ids,
                                         int32_t r_max, int32_t *device_page_table_a,
                                         int32_t *device_page_table_b, int32_t *device_rank,
                                         int32_t flags, lora_cache **out) {
  if (!out || !pool_a || !pool_b) return fail(LORA_EINVAL, "null argument");
  if (num_ids <= 0) return fail(LORA_EINVAL, "num_ids must be positive");
  if (r_max < 1 || r_max > LORA_MAX_RANK)
    return fail(LORA_EUNSUPPORTED, "r_max %d outside 1..%d", r_max, LORA_MAX_RANK);
  if (flags & ~LORA_CACHE_HOST_ONLY) return fail(LORA_EINVAL, "unknown flags 0x%x", flags);
  int32_t na, pra, wa, da, fa, nb, prb, wb, db, fb;
  lora_status st = lora_pool_info(pool_a, &na, &pra, &wa, &da, &fa);
  if (st != LORA_OK) return st;
  if ((st = lora_pool_info(pool_b, &nb, &prb, &wb, &db, &fb)) != LORA_OK) return st;
  if (pra != prb || da != db || fa != fb)
    return fail(LORA_EINVAL, "the two pools differ in page rows, dtype or format");
  const bool host_only = flags & LORA_CACHE_HOST_ONLY;
  if (!host_only && (!device_page_table_a || !device_page_table_b || !device_rank))
    return fail(LORA_EINVAL, "null device table");
  std::unique_ptr<lora_cache> c(new lora_cache());
  c->pool_a = pool_a;
  c->pool_b = pool_b;
  c->num_ids = num_ids;
  c->r_max = r_max;
  c->page_rows = pra;
  c->max_pages = (r_max + pra - 1) / pra;
  c->flags = flags;
  c->row_bytes_a = pool_row_bytes(wa, da, fa);
  c->row_bytes_b = pool_row_bytes(wb, db, fb);
  c->pt_a = device_page_table_a;
  c->pt_b = device_page_table_b;
  c->rank = device_rank;
  c->ids.resize((size_t)num_ids);
  if (!host_only) {
    hipError_t e = hipStreamCreateWithFlags(&c->copy, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
    const int64_t nt = (int64_t)num_ids * c->max_pages;
    hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(256), 0, c->copy, c->pt_a, nt, -1);
    hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(256), 0, c->copy, c->pt_b, nt, -1);
    hipLaunchKernelGGL(fill_kernel, dim3(64), dim3(256), 0, c->copy, c->rank, (int64_t)num_ids, 0);
    if ((e = hipGetLastError()) != hipSuccess || (e = hipStreamSynchronize(c->copy)) != hipSuccess) {
      (void)hipStreamDestroy(c->copy);
      return hip_fail(e, "page-table initialisation");
    }
  }
  *out = c.release();
  return ok();
}

extern "C" lora_status lora_cache_register(lora_cache *c, int32_t id, int32_t rank,
                                           const void *host_a_rows, const void *host_b_rows,
                                           const float *host_a_scales, const float *host_b_scales) {
  if (!c) return fail(LORA_EINVAL, "null cache");
  if (id < 0 || id >= c->num_ids) return fail(LORA_ERANGE, "adapter id %d outside [0, %d)", id, c->num_ids);
  if (rank < 1 || rank > c->r_max) return fail(LORA_ERANGE, "rank %d outside 1..%d", rank, c->r_max);
  if (!host_a_rows || !host_b_rows) return fail(LORA_EINVAL, "null rows");
  int32_t np, pr, wd, dt, wf;
  lora_pool_info(c->pool_a, &np, &pr, &wd, &dt, &wf);
  const bool quant = wf != LORA_WFMT_PLAIN;
  if (quant != (host_a_scales != nullptr) || quant != (host_b_scales != nullptr))
    return fail(LORA_EINVAL, "row scales are required for quantized pools and only for them");
  Entry &e = c->ids[(size_t)id];
  if (e.resident) return fail(LORA_EINVAL, "adapter %d is resident; it cannot be re-registered", id);
  e.registered = true;
  e.rank = rank;
  e.host_a = host_a_rows;
  e.host_b = host_b_rows;
  e.sc_a = host_a_scales;
  e.sc_b = host_b_scales;
  e.mapped = false;
  if (!c->host_only()) {
    e.dev_a = device_view(host_a_rows);
    e.dev_b = device_view(host_b_rows);
    e.dev_sa = device_view(host_a_scales);
    e.dev_sb = device_view(host_b_scales);
    e.mapped = e.dev_a && e.dev_b && (!quant || (e.dev_sa && e.dev_sb));
  }
  return ok();
}

extern "C" lora_status lora_cache_prepare(lora_cache *c, const int32_t *ids, int32_t n,
                                          hipStream_t compute) {
  if (!c) return fail(LORA_EINVAL, "null cache");
  if (n < 0 || (n > 0 && !ids)) return fail(LORA_EINVAL, "bad batch");
  // distinct adapters of the batch, validated
  const uint64_t stamp = ++c->batch;
  std::vector<int32_t> batch;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t a = ids[i];
    if (a == LORA_NO_ADAPTER) continue;
    if (a < 0 || a >= c->num_ids) return fail(LORA_ERANGE, "adapter id %d outside [0, %d)", a, c->num_ids);
    if (!c->ids[(size_t)a].registered) return fail(LORA_ERANGE, "adapter %d is not registered", a);
    batch.push_back(a);
  }
  std::sort(batch.begin(), batch.end());
  batch.erase(std::unique(batch.begin(), batch.end()), batch.end());

  // plan: misses and their pages; evictions (LRU, not in this batch) until they fit
  const bool shared = c->pool_a == c->pool_b;
  int32_t free_a, free_b;
  lora_pool_num_free(c->pool_a, &free_a);
  lora_pool_num_free(c->pool_b, &free_b);
  std::vector<int32_t> misses;
  int64_t need_a = 0, need_b = 0;
  for (int32_t a : batch) {
    const Entry &e = c->ids[(size_t)a];
    if (e.resident) continue;
    misses.push_back(a);
    const int32_t np = (e.rank + c->page_rows - 1) / c->page_rows;
    need_a += np;
    need_b += np;
  }
  auto fits = [&](int64_t fa, int64_t fb) {
    return shared ? need_a + need_b <= fa : (need_a <= fa && need_b <= fb);
  };
  std::vector<int32_t> victims;
  if (!fits(free_a, free_b)) {
    std::vector<std::pair<uint64_t, int32_t>> lru;
    for (int32_t a = 0; a < c->num_ids; ++a) {
      const Entry &e = c->ids[(size_t)a];
      if (e.resident && !std::binary_search(batch.begin(), batch.end(), a)) lru.push_back({e.stamp, a});
    }
    std::sort(lru.begin(), lru.end());
    // least recently used first, but adapters whose last batch has already
    // completed before those still queued on the compute stream: evicting a
    // queued adapter makes the upload wait for that batch
    auto done = [&](int32_t a) {
      const Entry &e = c->ids[(size_t)a];
      return !e.last_use || hipEventQuery(e.last_use->e) == hipSuccess;
    };
    std::stable_partition(lru.begin(), lru.end(), [&](const std::pair<uint64_t, int32_t> &q) { return done(q.second); });
    int64_t fa = free_a, fb = free_b;
    for (const auto &q : lru) {
      if (fits(fa, fb)) break;
      const Entry &e = c->ids[(size_t)q.second];
      fa += (int64_t)e.pages_a.size() + (shared ? (int64_t)e.pages_b.size() : 0);
      fb += (int64_t)e.pages_b.size();
      victims.push_back(q.second);
    }
    if (!fits(fa, fb))
      return fail(LORA_ENOMEM, "the batch's %zu adapters need more pages than the pools hold",
                  batch.size());
  }

  // the previous batch's adapters: last use completes after everything queued
  // on the compute stream so far
  if (!c->host_only() && !c->last_batch.empty()) {
    std::shared_ptr<Event> ev = std::make_shared<Event>();
    hipError_t e = hipEventCreateWithFlags(&ev->e, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    if ((e = hipEventRecord(ev->e, compute)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    for (int32_t a : c->last_batch) c->ids[(size_t)a].last_use = ev;
  }

  std::vector<TableEntry> pending;
  bool enqueued = false;
  // evictions: wait for their last use, free their pages, clear their table rows
  for (int32_t a : victims) {
    Entry &e = c->ids[(size_t)a];
    if (!c->host_only() && e.last_use) {
      hipError_t he = hipStreamWaitEvent(c->copy, e.last_use->e, 0);
      if (he != hipSuccess) return hip_fail(he, "hipStreamWaitEvent");
    }
    lora_status st = lora_pool_free(c->pool_a, e.pages_a.data(), (int32_t)e.pages_a.size());
    if (st == LORA_OK) st = lora_pool_free(c->pool_b, e.pages_b.data(), (int32_t)e.pages_b.size());
    if (st != LORA_OK) return st;
    table_entries(c, a, 0, {}, {}, true, pending);
    e.pages_a.clear();
    e.pages_b.clear();
    e.resident = false;
    e.last_use.reset();
    ++c->stats.evictions;
    enqueued = true;
  }
  // misses: pages, row uploads, table rows
  std::vector<CopyJob> jobs;
  for (int32_t a : misses) {
    Entry &e = c->ids[(size_t)a];
    const int32_t np = (e.rank + c->page_rows - 1) / c->page_rows;
    e.pages_a.assign((size_t)np, -1);
    e.pages_b.assign((size_t)np, -1);
    lora_status st = lora_pool_alloc(c->pool_a, e.rank, e.pages_a.data());
    if (st == LORA_OK) st = lora_pool_alloc(c->pool_b, e.rank, e.pages_b.data());
    if (st != LORA_OK) return st;  // cannot happen after the plan above
    if (!c->host_only() && e.mapped) {
      // one job per page and pool (rows, then scales)
      for (int32_t i = 0; i < np; ++i) {
        const int32_t r0 = i * c->page_rows, nr = std::min(c->page_rows, e.rank - r0);
        const lora_pool *ps[2] = {c->pool_a, c->pool_b};
        const char *src[2] = {e.dev_a, e.dev_b};
        const char *ssrc[2] = {e.dev_sa, e.dev_sb};
        const int32_t pg[2] = {e.pages_a[(size_t)i], e.pages_b[(size_t)i]};
        for (int s2 = 0; s2 < 2; ++s2) {
          const lora_pool *p = ps[s2];
          const int64_t rb = (int64_t)p->row_bytes;
          jobs.push_back({src[s2] + (int64_t)r0 * rb,
                          p->storage + ((int64_t)pg[s2] * p->page_rows) * rb, (int64_t)nr * rb});
          if (p->scales)
            jobs.push_back({ssrc[s2] + (int64_t)r0 * 4,
                            reinterpret_cast<char *>(p->scales + (int64_t)pg[s2] * p->page_rows),
                            (int64_t)nr * 4});
        }
      }
    } else if (!c->host_only()) {
      st = lora_pool_write_rows(c->pool_a, e.pages_a.data(), e.rank, e.host_a, e.sc_a, c->copy);
      if (st == LORA_OK)
        st = lora_pool_write_rows(c->pool_b, e.pages_b.data(), e.rank, e.host_b, e.sc_b, c->copy);
      if (st != LORA_OK) return st;
    }
    table_entries(c, a, e.rank, e.pages_a, e.pages_b, false, pending);
    e.resident = true;
    ++c->stats.misses;
    c->stats.bytes_uploaded += (int64_t)e.rank * (c->row_bytes_a + c->row_bytes_b) +
                               (e.sc_a ? (int64_t)e.rank * 8 : 0);
    enqueued = true;
  }
  lora_status st = c->host_only() ? LORA_OK : flush_copies(c, jobs);
  if (st != LORA_OK) return st;
  if ((st = flush_updates(c, pending)) != LORA_OK) return st;
  if (enqueued && !c->host_only()) {
    hipEvent_t up;
    hipError_t e = hipEventCreateWithFlags(&up, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(up, c->copy);
    if (e == hipSuccess) e = hipStreamWaitEvent(compute, up, 0);
    if (e == hipSuccess) e = hipEventDestroy(up);
    if (e != hipSuccess) return hip_fail(e, "upload ordering");
  }
  for (int32_t a : batch) c->ids[(size_t)a].stamp = stamp;
  c->stats.hits += (int64_t)(batch.size() - misses.size());
  c->last_batch = batch;
  return ok();
}

extern "C" lora_status lora_cache_get_stats(const lora_cache *c, lora_cache_stats *out) {
  if (!c || !out) return fail(LORA_EINVAL, "null argument");
  lora_cache_stats s = c->stats;
  s.resident = 0;
  s.scattered = 0;
  for (const Entry &e : c->ids) {
    if (!e.resident) continue;
    ++s.resident;
    if (!consecutive(e.pages_a) || !consecutive(e.pages_b)) ++s.scattered;
  }
  lora_pool_num_free(c->pool_a, &s.free_pages_a);
  lora_pool_num_free(c->pool_b, &s.free_pages_b);
  *out = s;
  return ok();
}

extern "C" lora_status lora_cache_pages(const lora_cache *c, int32_t id, int32_t *pages_a,
                                        int32_t *pages_b, int32_t *num_pages) {
  if (!c || !num_pages) return fail(LORA_EINVAL, "null argument");
  if (id < 0 || id >= c->num_ids) return fail(LORA_ERANGE, "adapter id %d outside [0, %d)", id, c->num_ids);
  const Entry &e = c->ids[(size_t)id];
  *num_pages = e.resident ? (int32_t)e.pages_a.size() : 0;
  for (size_t i = 0; e.resident && i < e.pages_a.size(); ++i) {
    if (pages_a) pages_a[i] = e.pages_a[i];
    if (pages_b) pages_b[i] = e.pages_b[i];
  }
  return ok();
}

extern "C" void lora_cache_destroy(lora_cache *c) {
  if (!c) return;
  if (c->copy) {
    (void)hipStreamSynchronize(c->copy);
    (void)hipStreamDestroy(c->copy);
  }
  delete c;
}
