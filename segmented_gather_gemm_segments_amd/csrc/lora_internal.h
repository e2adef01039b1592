// Declarations shared by the host half (host.cpp) and the kernel half
// (kernels.hip) of the library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "lora_sgmv.h"

// Page pool bookkeeping (host.cpp); the residency cache reads its geometry and
// storage to address pages.
struct lora_pool {
  int32_t num_pages, page_rows, row_width, dtype, weight_format;
  size_t row_bytes;
  char *storage;
  float *scales;                    // [num_pages * page_rows], quantized formats only
  std::vector<int32_t> free_list;   // front = next page handed out
  size_t head = 0;                  // free_list[head..] are free
  std::vector<uint8_t> taken;
};

namespace lora {

// Record an error message for lora_last_error() and return `code`.
lora_status fail(lora_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return LORA_OK.
lora_status ok();
// LORA_EHIP with the HIP error's text.
lora_status hip_fail(hipError_t e, const char *what);

// Length of each of the k_splits slices of d_in in a tiled shrink: the even
// share rounded up to a multiple of LORA_SHRINK_TILE_K (the last slice may be
// shorter; the planner never makes one empty).
inline int32_t tile_slice_len(int32_t d_in, int32_t k_splits) {
  const int32_t even = (d_in + k_splits - 1) / k_splits;
  return (even + LORA_SHRINK_TILE_K - 1) / LORA_SHRINK_TILE_K * LORA_SHRINK_TILE_K;
}

}  // namespace lora
