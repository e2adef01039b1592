// Randomised driver of the library's host half (segment build, planner, page
// pool bookkeeping, error reporting), built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  The three HIP
// runtime calls host.cpp makes are stubbed here with host equivalents: pool
// storage is host memory under the sanitizers, so lora_pool_write_rows copies
// host to host.  Exits non-zero (or the sanitizers abort) on any failure.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "lora_sgmv.h"

extern "C" {
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
const char *hipGetErrorString(hipError_t) { return "stub"; }
const char *hipGetErrorName(hipError_t) { return "stub"; }
}

#define CHECK(c)                                                                  \
  do {                                                                            \
    if (!(c)) {                                                                   \
      std::fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #c); \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

static void segments_and_plans(std::mt19937 &rng) {
  const int n_adapters = 1 + (int)(rng() % 70);
  const int t = (int)(rng() % 700);
  std::vector<int32_t> ids((size_t)t + 1);
  for (int i = 0; i < t; ++i) ids[(size_t)i] = (int32_t)(rng() % (n_adapters + 1)) - 1;
  if (t > 0 && rng() % 10 == 0) ids[rng() % (size_t)t] = n_adapters + (int32_t)(rng() % 3);  // out of range
  std::vector<int32_t> perm((size_t)t + 1), starts((size_t)t + 2), seg((size_t)t + 1);
  int32_t ns = -1;
  const lora_status st = lora_segments_build(ids.data(), t, n_adapters, perm.data(), starts.data(),
                                             seg.data(), &ns);
  if (st != LORA_OK) {
    CHECK(st == LORA_ERANGE);
    CHECK(std::strlen(lora_last_error()) > 0);
    return;
  }
  CHECK(ns >= 0 && ns <= t);
  std::vector<int32_t> ranks((size_t)n_adapters);
  int32_t r_max = 1;
  for (auto &r : ranks) {
    r = 1 + (int32_t)(rng() % 128);
    r_max = std::max(r_max, r);
  }
  for (int phase = 0; phase < 2; ++phase)
    for (int policy = 0; policy < 3; ++policy) {
      const int32_t dim = phase == LORA_PHASE_SHRINK ? r_max : 8 * (1 + (int32_t)(rng() % 2000));
      const int32_t mfma_min = (int32_t)(rng() % 40) - 4;
      int32_t count = -1;
      lora_status s = lora_sgmv_plan(phase, starts.data(), seg.data(), ns, n_adapters, ranks.data(), dim,
                                     policy, mfma_min, nullptr, 0, &count);
      CHECK(s == LORA_OK && count >= 0);
      std::vector<lora_item> items((size_t)count + 1);
      const int32_t cap = count > 0 && rng() % 5 == 0 ? count - 1 : count;  // sometimes too small
      int32_t count2 = -1;
      s = lora_sgmv_plan(phase, starts.data(), seg.data(), ns, n_adapters, ranks.data(), dim, policy,
                         mfma_min, items.data(), cap, &count2);
      CHECK(count2 == count);
      CHECK(cap == count ? s == LORA_OK : s == LORA_ENOMEM);
      if (s == LORA_OK)
        for (int32_t i = 0; i < count; ++i) {
          const int32_t cnt = items[(size_t)i].count_path & 0xffff;
          CHECK(cnt == 0 || (items[(size_t)i].perm_begin + cnt <= starts[(size_t)ns]));
        }
      // the same plan with a given expand tile, and a rejected one
      const int32_t tiles[4] = {0, 64, LORA_EXPAND_MFMA_TOKENS, 96};
      const int32_t tile = tiles[rng() % 4];
      int32_t count3 = -1;
      s = lora_sgmv_plan_tile(phase, starts.data(), seg.data(), ns, n_adapters, ranks.data(), dim, policy,
                              mfma_min, tile, nullptr, 0, &count3);
      CHECK(tile == 96 ? s == LORA_EINVAL : (s == LORA_OK && count3 >= 0));
      if (s == LORA_OK) {
        std::vector<lora_item> it3((size_t)count3 + 1);
        s = lora_sgmv_plan_tile(phase, starts.data(), seg.data(), ns, n_adapters, ranks.data(), dim, policy,
                                mfma_min, tile, it3.data(), count3, &count3);
        CHECK(s == LORA_OK);
      }
    }
  // the tiled planner, its workspace query and the tiled-or-plain choice
  const int32_t d_in = 64 * (int32_t)(rng() % 500) + (rng() % 8 == 0 ? 8 : 0);  // sometimes not a multiple
  for (int policy = 0; policy < 3; ++policy) {
    const int32_t rm = std::min(r_max, (int32_t)(rng() % 2 ? 64 : 128));
    std::vector<int32_t> rk(ranks);
    for (auto &r : rk) r = std::min(r, rm);
    const int32_t tmin = (int32_t)(rng() % 40) - 4, ms = (int32_t)(rng() % 70) - 2;
    int32_t count = -1, ks = -1;
    lora_status s = lora_sgmv_plan_tiled(starts.data(), seg.data(), ns, n_adapters, rk.data(), rm, d_in, policy,
                                         tmin, ms, nullptr, 0, &count, &ks);
    if (d_in <= 0 || d_in % LORA_SHRINK_TILE_K || rm > 64) {
      CHECK(s == LORA_EUNSUPPORTED);
    } else if (ms > LORA_MAX_K_SPLITS) {
      CHECK(s == LORA_EINVAL);
    } else {
      CHECK(s == LORA_OK && count >= 0 && ks >= 1 && ks <= LORA_MAX_K_SPLITS);
      std::vector<lora_item> items((size_t)count + 1);
      int32_t count2 = -1, ks2 = -1;
      s = lora_sgmv_plan_tiled(starts.data(), seg.data(), ns, n_adapters, rk.data(), rm, d_in, policy, tmin, ms,
                               items.data(), count, &count2, &ks2);
      CHECK(s == LORA_OK && count2 == count && ks2 == ks);
      for (int32_t i = 0; i < count; ++i) {
        const int32_t cnt = items[(size_t)i].count_path & 0xffff, path = items[(size_t)i].count_path >> 16;
        CHECK(cnt > 0 && items[(size_t)i].perm_begin + cnt <= starts[(size_t)ns]);
        CHECK(path != LORA_PATH_TILE || (cnt <= LORA_SHRINK_TILE_TOKENS && items[(size_t)i].block < ks));
      }
      int64_t bytes = -1;
      CHECK(lora_sgmv_shrink_tiled_workspace(starts[(size_t)ns], rm, ks, &bytes) == LORA_OK);
      CHECK(ks == 1 ? bytes == 0 : bytes == (int64_t)ks * starts[(size_t)ns] * rm * 4);
    }
    int32_t pays = -1;
    s = lora_sgmv_tiled_pays(starts.data(), seg.data(), ns, n_adapters, rk.data(), rm, d_in, LORA_BF16,
                             LORA_WFMT_PLAIN, tmin, &pays);
    CHECK(s == LORA_OK && (pays == 0 || pays == 1));
  }
}

static void pools(std::mt19937 &rng) {
  const int32_t page_rows = 1 + (int32_t)(rng() % 32), num_pages = 1 + (int32_t)(rng() % 200);
  const int32_t fmt = (int32_t)(rng() % 3);
  const int32_t width = 2 * (1 + (int32_t)(rng() % 64));
  const size_t row_bytes = fmt == LORA_WFMT_FP8_E4M3 ? (size_t)width
                           : fmt == LORA_WFMT_INT4   ? (size_t)width / 2
                                                     : (size_t)width * 2;
  std::vector<char> storage((size_t)num_pages * page_rows * row_bytes);
  std::vector<float> scales((size_t)num_pages * page_rows);
  lora_pool *pool = nullptr;
  lora_status s = lora_pool_create(num_pages, page_rows, width, LORA_BF16, fmt, storage.data(),
                                   fmt == LORA_WFMT_PLAIN ? nullptr : scales.data(), rng(), &pool);
  CHECK(s == LORA_OK && pool);
  std::vector<std::vector<int32_t>> held;
  for (int it = 0; it < 200; ++it) {
    if (held.empty() || rng() % 3) {
      const int32_t rows = 1 + (int32_t)(rng() % (4 * page_rows));
      std::vector<int32_t> ids((size_t)(rows + page_rows - 1) / page_rows);
      s = lora_pool_alloc(pool, rows, ids.data());
      if (s == LORA_ENOMEM) continue;
      CHECK(s == LORA_OK);
      std::vector<char> src((size_t)rows * row_bytes, (char)it);
      std::vector<float> sc((size_t)rows, 1.f);
      s = lora_pool_write_rows(pool, ids.data(), rows, src.data(),
                               fmt == LORA_WFMT_PLAIN ? nullptr : sc.data(), nullptr);
      CHECK(s == LORA_OK);
      held.push_back(ids);
    } else {
      const size_t k = rng() % held.size();
      CHECK(lora_pool_free(pool, held[k].data(), (int32_t)held[k].size()) == LORA_OK);
      CHECK(lora_pool_free(pool, held[k].data(), (int32_t)held[k].size()) == LORA_EINVAL);  // twice
      held.erase(held.begin() + (ptrdiff_t)k);
    }
    int32_t nf = -1;
    CHECK(lora_pool_num_free(pool, &nf) == LORA_OK && nf >= 0 && nf <= num_pages);
  }
  int32_t np = 0, pr = 0;
  CHECK(lora_pool_info(pool, &np, &pr, nullptr, nullptr, nullptr) == LORA_OK);
  CHECK(np == num_pages && pr == page_rows);
  lora_pool_destroy(pool);
}

int main() {
  std::mt19937 rng(12345);
  CHECK(lora_abi_version() == LORA_ABI_VERSION);
  for (int s = -6; s <= 1; ++s) CHECK(lora_status_name(s) != nullptr);
  for (int i = 0; i < 300; ++i) segments_and_plans(rng);
  for (int i = 0; i < 60; ++i) pools(rng);
  std::printf("host driver ok\n");
  return 0;
}
