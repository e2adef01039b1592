// Host half of the C ABI: error reporting, the segment build, the one-launch
// work planner and the paged adapter pool's bookkeeping.  Nothing here touches
// the GPU except lora_pool_write_rows (async copies on the caller's stream).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "lora_internal.h"

namespace lora {

static thread_local std::string g_last_error;

lora_status fail(lora_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

lora_status ok() {
  g_last_error.clear();
  return LORA_OK;
}

lora_status hip_fail(hipError_t e, const char *what) {
  return fail(LORA_EHIP, "%s: %s (%s)", what, hipGetErrorString(e), hipGetErrorName(e));
}

}  // namespace lora

using namespace lora;

extern "C" int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

extern "C" const char *lora_last_error(void) { return g_last_error.c_str(); }

extern "C" const char *lora_status_name(lora_status s) {
  switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_EINVAL: return "LORA_EINVAL";
    case LORA_ERANGE: return "LORA_ERANGE";
    case LORA_EUNSUPPORTED: return "LORA_EUNSUPPORTED";
    case LORA_ENOMEM: return "LORA_ENOMEM";
    case LORA_EHIP: return "LORA_EHIP";
    default: return "LORA_UNKNOWN";
  }
}

// --------------------------------------------------------------------------
// Segment build: stable counting sort by adapter id.
extern "C" lora_status lora_segments_build(const int32_t *token_adapter, int32_t num_tokens,
                                           int32_t num_adapters, int32_t *token_perm,
                                           int32_t *seg_starts, int32_t *seg_adapter,
                                           int32_t *num_segments) {
  if (num_tokens < 0 || num_adapters < 0) return fail(LORA_EINVAL, "negative size");
  if (!seg_starts || !num_segments) return fail(LORA_EINVAL, "null seg_starts/num_segments");
  if (num_tokens > 0 && (!token_adapter || !token_perm || !seg_adapter))
    return fail(LORA_EINVAL, "null pointer with num_tokens > 0");
  for (int32_t t = 0; t < num_tokens; ++t) {
    int32_t a = token_adapter[t];
    if (a != LORA_NO_ADAPTER && (a < 0 || a >= num_adapters))
      return fail(LORA_ERANGE, "token %d has adapter id %d outside {-1} U [0, %d)", t, a,
                  num_adapters);
  }
  // count tokens per adapter, then exclusive prefix sum -> first slot per adapter
  std::vector<int32_t> count((size_t)num_adapters + 1, 0);
  for (int32_t t = 0; t < num_tokens; ++t)
    if (token_adapter[t] >= 0) ++count[(size_t)token_adapter[t]];
  std::vector<int32_t> slot((size_t)num_adapters + 1, 0);
  int32_t S = 0, run = 0;
  for (int32_t a = 0; a < num_adapters; ++a) {
    slot[(size_t)a] = run;
    if (count[(size_t)a] > 0) {
      seg_starts[S] = run;
      seg_adapter[S] = a;
      ++S;
    }
    run += count[(size_t)a];
  }
  seg_starts[S] = run;
  // scatter in original order: tokens of one adapter keep their batch order
  for (int32_t t = 0; t < num_tokens; ++t) {
    int32_t a = token_adapter[t];
    if (a >= 0) token_perm[slot[(size_t)a]++] = t;
  }
  *num_segments = S;
  return ok();
}

// --------------------------------------------------------------------------
// Work planner.
namespace {

struct PlanItem {
  lora_item item;
  int64_t weight;  // estimated bytes the item moves, for heaviest-first order
};

// Device order of a plan's items: heaviest first, dealt to the workgroups in
// that order (workgroup k runs item k; consecutive workgroups go to the eight
// XCDs in turn, so every XCD gets an even share of every segment).  Keeping a
// segment's items on one XCD, so that its adapter rows are fetched into one
// L2, was measured slower: the XCD's compute units then all read the same
// rows at once.
std::vector<lora_item> device_order(std::vector<PlanItem> &plan) {
  std::stable_sort(plan.begin(), plan.end(),
                   [](const PlanItem &x, const PlanItem &y) { return x.weight > y.weight; });
  std::vector<lora_item> out;
  out.reserve(plan.size());
  for (const PlanItem &p : plan) out.push_back(p.item);
  return out;
}

}  // namespace

// MFMA expand token tile by output width, measured on MI355X with the
// batches of the benchmark (heterogeneous ranks, prefill, the 70B layer's
// projections): 128-token items ran 4-8 % faster at 8192 columns and 1.5-2 %
// slower (or, at 1024 columns with too few items, much slower) at the other
// widths.  A width takes the choice of the nearest measured one.
struct ExpandTile {
  int32_t cols, tokens;
};
static const ExpandTile kExpandTileByWidth[] = {{1024, 64}, {4096, 64}, {8192, 128}, {14336, 64}, {28672, 64}};
static int32_t expand_tile_by_width(int32_t d_out) {
  const ExpandTile *best = &kExpandTileByWidth[0];
  for (const ExpandTile &e : kExpandTileByWidth)
    if (std::abs((int64_t)d_out - e.cols) < std::abs((int64_t)d_out - best->cols)) best = &e;
  return best->tokens;
}

extern "C" lora_status lora_sgmv_plan(int32_t phase, const int32_t *seg_starts,
                                      const int32_t *seg_adapter, int32_t num_segments,
                                      int32_t num_adapters, const int32_t *host_rank, int32_t dim,
                                      int32_t path_policy, int32_t mfma_min_tokens,
                                      lora_item *items, int32_t capacity, int32_t *num_items) {
  return lora_sgmv_plan_tile(phase, seg_starts, seg_adapter, num_segments, num_adapters, host_rank, dim,
                             path_policy, mfma_min_tokens, 0, items, capacity, num_items);
}

extern "C" lora_status lora_sgmv_plan_tile(int32_t phase, const int32_t *seg_starts,
                                           const int32_t *seg_adapter, int32_t num_segments,
                                           int32_t num_adapters, const int32_t *host_rank, int32_t dim,
                                           int32_t path_policy, int32_t mfma_min_tokens,
                                           int32_t expand_tile_tokens, lora_item *items, int32_t capacity,
                                           int32_t *num_items) {
  if (!num_items) return fail(LORA_EINVAL, "null num_items");
  if (expand_tile_tokens != 0 && expand_tile_tokens != 64 && expand_tile_tokens != LORA_EXPAND_MFMA_TOKENS)
    return fail(LORA_EINVAL, "expand_tile_tokens must be 0, 64 or %d (got %d)", LORA_EXPAND_MFMA_TOKENS,
                expand_tile_tokens);
  if (phase != LORA_PHASE_SHRINK && phase != LORA_PHASE_EXPAND)
    return fail(LORA_EINVAL, "unknown phase %d", phase);
  if (path_policy < LORA_PATH_AUTO || path_policy > LORA_PATH_MFMA)
    return fail(LORA_EINVAL, "unknown path policy %d", path_policy);
  if (num_segments < 0 || capacity < 0 || num_adapters < 0) return fail(LORA_EINVAL, "negative size");
  if (num_segments > 0 && (!seg_starts || !seg_adapter))
    return fail(LORA_EINVAL, "null segment arrays");
  if (phase == LORA_PHASE_EXPAND && (dim <= 0 || dim % 8 != 0))
    return fail(LORA_EUNSUPPORTED, "expand plan needs d_out > 0 and a multiple of 8 (got %d)",
                dim);
  if (phase == LORA_PHASE_SHRINK && (dim < 1 || dim > LORA_MAX_RANK))
    return fail(LORA_EUNSUPPORTED, "shrink plan needs r_max in 1..%d (got %d)", LORA_MAX_RANK, dim);
  if (mfma_min_tokens <= 0) mfma_min_tokens = LORA_DEFAULT_MFMA_MIN_TOKENS;
  if (num_segments > 0 && seg_starts[0] < 0) return fail(LORA_EINVAL, "seg_starts[0] < 0");
  for (int32_t s = 0; s < num_segments; ++s) {
    if (seg_starts[s + 1] <= seg_starts[s])
      return fail(LORA_EINVAL, "seg_starts not strictly increasing at %d", s);
    if (seg_adapter[s] < 0 || seg_adapter[s] >= num_adapters)
      return fail(LORA_ERANGE, "segment %d has adapter %d outside [0, %d)", s, seg_adapter[s],
                  num_adapters);
    if (phase == LORA_PHASE_SHRINK && host_rank) {
      const int32_t r = host_rank[seg_adapter[s]];
      if (r < 1 || r > dim)
        return fail(LORA_ERANGE, "adapter %d has rank %d outside 1..r_max (%d)", seg_adapter[s], r,
                    dim);
    }
  }
  auto is_mfma = [&](int32_t len) {
    return path_policy == LORA_PATH_MFMA || (path_policy == LORA_PATH_AUTO && len >= mfma_min_tokens);
  };
  // Token tile of the expand's MFMA items: the caller's expand_tile_tokens,
  // or (0) LORA_EXPAND_MFMA_TOKENS (two 64-token passes in one workgroup)
  // where the output width's nearest entry of kExpandTileByWidth says so and
  // such items still number at least LORA_EXPAND_LONG_TILE_MIN_ITEMS, else 64.
  int32_t expand_mfma_step = expand_tile_tokens ? expand_tile_tokens : 64;
  if (phase == LORA_PHASE_EXPAND && expand_tile_tokens == 0 &&
      expand_tile_by_width(dim) == LORA_EXPAND_MFMA_TOKENS) {
    const int64_t nblk = (dim + LORA_EXPAND_MFMA_COLS - 1) / LORA_EXPAND_MFMA_COLS;
    int64_t long_items = 0;
    for (int32_t s = 0; s < num_segments; ++s) {
      const int32_t len = seg_starts[s + 1] - seg_starts[s];
      if (is_mfma(len)) long_items += (len + LORA_EXPAND_MFMA_TOKENS - 1) / LORA_EXPAND_MFMA_TOKENS * nblk;
    }
    if (long_items >= LORA_EXPAND_LONG_TILE_MIN_ITEMS) expand_mfma_step = LORA_EXPAND_MFMA_TOKENS;
  }
  std::vector<PlanItem> plan;
  for (int32_t s = 0; s < num_segments; ++s) {
    const int32_t begin = seg_starts[s], len = seg_starts[s + 1] - seg_starts[s];
    const int32_t a = seg_adapter[s];
    const bool mfma = is_mfma(len);
    const int32_t path = mfma ? LORA_PATH_MFMA : LORA_PATH_GATHER;
    if (phase == LORA_PHASE_SHRINK) {
      const int32_t r = host_rank ? host_rank[a] : dim;
      const int32_t step = mfma ? LORA_SHRINK_MFMA_TOKENS : LORA_SHRINK_GATHER_TOKENS;
      const int32_t groups = mfma ? 1 : (r + LORA_SHRINK_GATHER_ROWS - 1) / LORA_SHRINK_GATHER_ROWS;
      for (int32_t m0 = 0; m0 < len; m0 += step) {
        const int32_t cnt = std::min(step, len - m0);
        for (int32_t g = 0; g < groups; ++g) {
          // bytes moved, in units of one d_in row: the item's x rows plus the
          // adapter rows it reads
          const int32_t rows = mfma ? r : std::min(LORA_SHRINK_GATHER_ROWS, r - g * LORA_SHRINK_GATHER_ROWS);
          PlanItem p{{begin + m0, a, cnt | (path << 16), g}, (int64_t)cnt + rows};
          plan.push_back(p);
        }
      }
    } else {
      const int32_t step = mfma ? expand_mfma_step : LORA_EXPAND_GATHER_TOKENS;
      const int32_t cols = mfma ? LORA_EXPAND_MFMA_COLS : LORA_EXPAND_GATHER_COLS;
      const int32_t nblk = (dim + cols - 1) / cols;
      for (int32_t m0 = 0; m0 < len; m0 += step) {
        const int32_t cnt = std::min(step, len - m0);
        for (int32_t b = 0; b < nblk; ++b) {
          const int32_t c = std::min(cols, dim - b * cols);
          // y read and written per token (2 x 2 bytes per column) plus the
          // adapter's B^T rows (16 assumed without host ranks)
          const int32_t r = host_rank ? std::min(std::max(host_rank[a], 1), LORA_MAX_RANK) : 16;
          PlanItem p{{begin + m0, a, cnt | (path << 16), b}, (int64_t)c * (4 * cnt + 2 * r)};
          plan.push_back(p);
        }
      }
    }
  }
  const std::vector<lora_item> order = device_order(plan);
  if (order.size() > (size_t)INT32_MAX) return fail(LORA_ENOMEM, "plan too large");
  *num_items = (int32_t)order.size();
  if (!items) return ok();
  if ((int32_t)order.size() > capacity)
    return fail(LORA_ENOMEM, "plan needs %zu items, capacity %d", order.size(), capacity);
  for (size_t i = 0; i < order.size(); ++i) items[i] = order[i];
  return ok();
}

// Slices of a tiled shrink: k_splits slices of tile_slice_len elements (the
// last one shorter), every one a non-empty multiple of LORA_SHRINK_TILE_K.
static int32_t tile_slice_count(int32_t d_in, int32_t want) {
  const int32_t units = d_in / LORA_SHRINK_TILE_K;
  int32_t s = std::max(1, std::min(want, units));
  while (s > 1 && (int64_t)(s - 1) * lora::tile_slice_len(d_in, s) >= d_in) --s;
  return s;
}

extern "C" lora_status lora_sgmv_plan_tiled(const int32_t *seg_starts, const int32_t *seg_adapter,
                                            int32_t num_segments, int32_t num_adapters,
                                            const int32_t *host_rank, int32_t r_max, int32_t d_in,
                                            int32_t path_policy, int32_t tile_min_tokens,
                                            int32_t max_splits, lora_item *items, int32_t capacity,
                                            int32_t *num_items, int32_t *k_splits) {
  if (!num_items || !k_splits) return fail(LORA_EINVAL, "null num_items or k_splits");
  if (d_in <= 0 || d_in % LORA_SHRINK_TILE_K)
    return fail(LORA_EUNSUPPORTED, "d_in %d is not a positive multiple of %d", d_in, LORA_SHRINK_TILE_K);
  if (r_max > 64) return fail(LORA_EUNSUPPORTED, "tiled shrink needs r_max <= 64 (got %d)", r_max);
  if (max_splits > LORA_MAX_K_SPLITS)
    return fail(LORA_EINVAL, "max_splits %d above %d", max_splits, LORA_MAX_K_SPLITS);
  if (max_splits <= 0) max_splits = LORA_MAX_K_SPLITS;
  if (tile_min_tokens <= 0) tile_min_tokens = LORA_DEFAULT_TILE_MIN_TOKENS;
  // the segment checks are the plain shrink plan's
  int32_t n_plain = 0;
  lora_status st = lora_sgmv_plan(LORA_PHASE_SHRINK, seg_starts, seg_adapter, num_segments, num_adapters,
                                  host_rank, r_max, LORA_PATH_GATHER, 1, nullptr, 0, &n_plain);
  if (st != LORA_OK) return st;
  // AUTO: long segments, and short ones whose gather items would read each x
  // row r / LORA_SHRINK_GATHER_ROWS >= 8 times
  auto tiled = [&](int32_t len, int32_t r) {
    return path_policy == LORA_PATH_MFMA ||
           (path_policy == LORA_PATH_AUTO && (len >= tile_min_tokens || r >= LORA_TILE_MIN_RANK_SHORT));
  };
  // slices: the heaviest tile item (a full token tile and the largest rank)
  // reads about LORA_SHRINK_TILE_ITEM_BYTES of x and A
  int64_t heaviest = 0;
  for (int32_t s = 0; s < num_segments; ++s) {
    const int32_t len = seg_starts[s + 1] - seg_starts[s];
    const int32_t r = host_rank ? host_rank[seg_adapter[s]] : r_max;
    if (!tiled(len, r)) continue;
    heaviest = std::max(heaviest, (int64_t)(std::min(len, LORA_SHRINK_TILE_TOKENS) + r) * d_in * 2);
  }
  const int64_t want = (heaviest + LORA_SHRINK_TILE_ITEM_BYTES - 1) / LORA_SHRINK_TILE_ITEM_BYTES;
  const int32_t splits = tile_slice_count(d_in, (int32_t)std::min<int64_t>(want, max_splits));
  std::vector<PlanItem> plan;
  for (int32_t s = 0; s < num_segments; ++s) {
    const int32_t begin = seg_starts[s], len = seg_starts[s + 1] - seg_starts[s];
    const int32_t a = seg_adapter[s];
    const int32_t r = host_rank ? host_rank[a] : r_max;
    if (tiled(len, r)) {
      for (int32_t m0 = 0; m0 < len; m0 += LORA_SHRINK_TILE_TOKENS) {
        const int32_t cnt = std::min(LORA_SHRINK_TILE_TOKENS, len - m0);
        for (int32_t k = 0; k < splits; ++k)
          plan.push_back({{begin + m0, a, cnt | (LORA_PATH_TILE << 16), k}, (int64_t)cnt + r});
      }
    } else {
      const int32_t groups = (r + LORA_SHRINK_GATHER_ROWS - 1) / LORA_SHRINK_GATHER_ROWS;
      for (int32_t m0 = 0; m0 < len; m0 += LORA_SHRINK_GATHER_TOKENS) {
        const int32_t cnt = std::min(LORA_SHRINK_GATHER_TOKENS, len - m0);
        for (int32_t g = 0; g < groups; ++g) {
          // in units of one slice of a row, as the tile items: a gather item
          // reads its rows over all of d_in
          const int32_t rows = std::min(LORA_SHRINK_GATHER_ROWS, r - g * LORA_SHRINK_GATHER_ROWS);
          plan.push_back({{begin + m0, a, cnt | (LORA_PATH_GATHER << 16), g}, (int64_t)(cnt + rows) * splits});
        }
      }
    }
  }
  const std::vector<lora_item> order = device_order(plan);
  if (order.size() > (size_t)INT32_MAX) return fail(LORA_ENOMEM, "plan too large");
  *num_items = (int32_t)order.size();
  *k_splits = splits;
  if (!items) return ok();
  if ((int32_t)order.size() > capacity)
    return fail(LORA_ENOMEM, "plan needs %zu items, capacity %d", order.size(), capacity);
  for (size_t i = 0; i < order.size(); ++i) items[i] = order[i];
  return ok();
}

extern "C" lora_status lora_sgmv_tiled_pays(const int32_t *seg_starts, const int32_t *seg_adapter,
                                            int32_t num_segments, int32_t num_adapters,
                                            const int32_t *host_rank, int32_t r_max, int32_t d_in,
                                            int32_t dtype, int32_t weight_format, int32_t tile_min_tokens,
                                            int32_t *pays) {
  if (!pays) return fail(LORA_EINVAL, "null pays");
  *pays = 0;
  int32_t n_plain = 0;
  lora_status st = lora_sgmv_plan(LORA_PHASE_SHRINK, seg_starts, seg_adapter, num_segments, num_adapters,
                                  host_rank, r_max, LORA_PATH_GATHER, 1, nullptr, 0, &n_plain);
  if (st != LORA_OK) return st;
  if (dtype != LORA_BF16 || weight_format < LORA_WFMT_PLAIN || weight_format > LORA_WFMT_INT4 || r_max > 64 ||
      d_in <= 0 || d_in % LORA_SHRINK_TILE_K)
    return ok();
  // bytes of one d_in row: x rows are bf16, A rows bf16, FP8 or INT4
  const int64_t x_row = 2 * (int64_t)d_in;
  const int64_t a_row = weight_format == LORA_WFMT_PLAIN ? 2 * (int64_t)d_in
                        : weight_format == LORA_WFMT_FP8_E4M3 ? (int64_t)d_in : (int64_t)d_in / 2;
  if (tile_min_tokens <= 0) tile_min_tokens = LORA_DEFAULT_TILE_MIN_TOKENS;
  // rows each plan's items read through the compute units: the plain plan's
  // MFMA items read A once per LORA_SHRINK_MFMA_TOKENS tokens, its gather
  // items x once per LORA_SHRINK_GATHER_ROWS rows and A once per
  // LORA_SHRINK_GATHER_TOKENS tokens; tile items read x once and A once per
  // LORA_SHRINK_TILE_TOKENS tokens
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  int64_t saved = 0;
  for (int32_t s = 0; s < num_segments; ++s) {
    const int64_t len = seg_starts[s + 1] - seg_starts[s];
    const int64_t r = host_rank ? host_rank[seg_adapter[s]] : r_max;
    if (!(len >= tile_min_tokens || r >= LORA_TILE_MIN_RANK_SHORT)) continue;
    const bool mfma = len >= LORA_DEFAULT_MFMA_MIN_TOKENS;
    const int64_t px = mfma ? len : len * cdiv(r, LORA_SHRINK_GATHER_ROWS);
    const int64_t pa = r * cdiv(len, mfma ? LORA_SHRINK_MFMA_TOKENS : LORA_SHRINK_GATHER_TOKENS);
    saved += (px - len) * x_row + (pa - r * cdiv(len, LORA_SHRINK_TILE_TOKENS)) * a_row;
  }
  *pays = saved >= (int64_t)LORA_TILE_PAYS_BYTES;
  return ok();
}

extern "C" lora_status lora_sgmv_shrink_tiled_workspace(int32_t num_perm, int32_t r_max, int32_t k_splits,
                                                        int64_t *bytes) {
  if (!bytes) return fail(LORA_EINVAL, "null bytes");
  *bytes = 0;
  if (num_perm < 0 || r_max < 1 || r_max > 64 || k_splits < 1 || k_splits > LORA_MAX_K_SPLITS)
    return fail(LORA_EINVAL, "tiled workspace query: num_perm %d, r_max %d, k_splits %d", num_perm, r_max,
                k_splits);
  if (k_splits > 1) *bytes = (int64_t)k_splits * num_perm * r_max * (int64_t)sizeof(float);
  return ok();
}

// --------------------------------------------------------------------------
// Paged pool.

static uint64_t splitmix64(uint64_t &s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

extern "C" lora_status lora_pool_create(int32_t num_pages, int32_t page_rows, int32_t row_width,
                                        int32_t dtype, int32_t weight_format,
                                        void *device_storage, float *device_scales,
                                        uint64_t shuffle_seed, lora_pool **out) {
  if (!out) return fail(LORA_EINVAL, "null out");
  if (num_pages <= 0 || page_rows <= 0 || row_width <= 0)
    return fail(LORA_EINVAL, "pool sizes must be positive");
  if (dtype != LORA_F32 && dtype != LORA_BF16) return fail(LORA_EUNSUPPORTED, "dtype %d", dtype);
  if (weight_format != LORA_WFMT_PLAIN && weight_format != LORA_WFMT_FP8_E4M3 &&
      weight_format != LORA_WFMT_INT4)
    return fail(LORA_EUNSUPPORTED, "weight_format %d", weight_format);
  const bool quant = weight_format != LORA_WFMT_PLAIN;
  if (quant && dtype != LORA_BF16)
    return fail(LORA_EUNSUPPORTED, "quantized adapter rows need bf16 activations");
  if (quant && row_width % 2) return fail(LORA_EINVAL, "INT4 / FP8 rows need an even width");
  if (!device_storage) return fail(LORA_EINVAL, "null storage");
  if (quant != (device_scales != nullptr))
    return fail(LORA_EINVAL, "row scales are required for quantized formats and only for them");
  lora_pool *p = new lora_pool();
  p->num_pages = num_pages;
  p->page_rows = page_rows;
  p->row_width = row_width;
  p->dtype = dtype;
  p->weight_format = weight_format;
  p->row_bytes = weight_format == LORA_WFMT_FP8_E4M3 ? (size_t)row_width
                 : weight_format == LORA_WFMT_INT4   ? (size_t)row_width / 2
                 : (size_t)row_width * (dtype == LORA_BF16 ? 2 : 4);
  p->storage = (char *)device_storage;
  p->scales = device_scales;
  p->free_list.resize((size_t)num_pages);
  for (int32_t i = 0; i < num_pages; ++i) p->free_list[(size_t)i] = i;
  if (shuffle_seed != 0) {  // Fisher-Yates with a splitmix64 stream
    uint64_t s = shuffle_seed;
    for (int32_t i = num_pages - 1; i > 0; --i) {
      int32_t j = (int32_t)(splitmix64(s) % (uint64_t)(i + 1));
      std::swap(p->free_list[(size_t)i], p->free_list[(size_t)j]);
    }
  }
  p->taken.assign((size_t)num_pages, 0);
  *out = p;
  return ok();
}

extern "C" lora_status lora_pool_alloc(lora_pool *p, int32_t rows, int32_t *page_ids) {
  if (!p || !page_ids) return fail(LORA_EINVAL, "null pool or page_ids");
  if (rows <= 0) return fail(LORA_EINVAL, "rows must be positive");
  const int32_t need = (rows + p->page_rows - 1) / p->page_rows;
  if ((int64_t)(p->free_list.size() - p->head) < need)
    return fail(LORA_ENOMEM, "pool has %zu free pages, %d needed", p->free_list.size() - p->head,
                need);
  for (int32_t i = 0; i < need; ++i) {
    int32_t id = p->free_list[p->head++];
    p->taken[(size_t)id] = 1;
    page_ids[i] = id;
  }
  // compact the consumed prefix now and then so the list does not grow forever
  if (p->head > 4096 && p->head * 2 > p->free_list.size()) {
    p->free_list.erase(p->free_list.begin(), p->free_list.begin() + (ptrdiff_t)p->head);
    p->head = 0;
  }
  return ok();
}

extern "C" lora_status lora_pool_free(lora_pool *p, const int32_t *page_ids, int32_t n) {
  if (!p || (n > 0 && !page_ids)) return fail(LORA_EINVAL, "null pool or page_ids");
  if (n < 0) return fail(LORA_EINVAL, "negative count");
  std::vector<uint8_t> seen((size_t)p->num_pages, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = page_ids[i];
    if (id < 0 || id >= p->num_pages || !p->taken[(size_t)id] || seen[(size_t)id])
      return fail(LORA_EINVAL, "page %d is not allocated (or listed twice)", id);
    seen[(size_t)id] = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    p->taken[(size_t)page_ids[i]] = 0;
    p->free_list.push_back(page_ids[i]);
  }
  return ok();
}

extern "C" lora_status lora_pool_num_free(const lora_pool *p, int32_t *num_free) {
  if (!p || !num_free) return fail(LORA_EINVAL, "null argument");
  *num_free = (int32_t)(p->free_list.size() - p->head);
  return ok();
}

extern "C" lora_status lora_pool_write_rows(lora_pool *p, const int32_t *page_ids, int32_t rows,
                                            const void *src, const float *src_scales,
                                            hipStream_t stream) {
  if (!p || !page_ids || !src) return fail(LORA_EINVAL, "null argument");
  if (rows <= 0) return fail(LORA_EINVAL, "rows must be positive");
  if ((p->scales != nullptr) != (src_scales != nullptr))
    return fail(LORA_EINVAL, "row scales are required for quantized pools and only for them");
  const size_t row_bytes = p->row_bytes;
  const int32_t npages = (rows + p->page_rows - 1) / p->page_rows;
  for (int32_t i = 0; i < npages; ++i) {
    int32_t id = page_ids[i];
    if (id < 0 || id >= p->num_pages || !p->taken[(size_t)id])
      return fail(LORA_EINVAL, "page %d is not allocated", id);
  }
  for (int32_t i = 0; i < npages; ++i) {
    const int32_t nr = std::min(p->page_rows, rows - i * p->page_rows);
    char *dst = p->storage + (size_t)page_ids[i] * p->page_rows * row_bytes;
    const char *s = (const char *)src + (size_t)i * p->page_rows * row_bytes;
    hipError_t e = hipMemcpyAsync(dst, s, (size_t)nr * row_bytes, hipMemcpyDefault, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (pool rows)");
    if (p->scales) {
      e = hipMemcpyAsync(p->scales + (size_t)page_ids[i] * p->page_rows,
                         src_scales + (size_t)i * p->page_rows, (size_t)nr * sizeof(float),
                         hipMemcpyDefault, stream);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (pool row scales)");
    }
  }
  return ok();
}

extern "C" void lora_pool_destroy(lora_pool *p) { delete p; }

extern "C" lora_status lora_pool_info(const lora_pool *p, int32_t *num_pages, int32_t *page_rows,
                                      int32_t *row_width, int32_t *dtype, int32_t *weight_format) {
  if (!p) return fail(LORA_EINVAL, "null pool");
  if (num_pages) *num_pages = p->num_pages;
  if (page_rows) *page_rows = p->page_rows;
  if (row_width) *row_width = p->row_width;
  if (dtype) *dtype = p->dtype;
  if (weight_format) *weight_format = p->weight_format;
  return ok();
}
