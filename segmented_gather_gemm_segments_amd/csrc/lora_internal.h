// Declarations shared by the host half (host.cpp) and the kernel half
// (kernels.hip) of the library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include "lora_sgmv.h"

namespace lora {

// Record an error message for lora_last_error() and return `code`.
lora_status fail(lora_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return LORA_OK.
lora_status ok();
// LORA_EHIP with the HIP error's text.
lora_status hip_fail(hipError_t e, const char *what);

}  // namespace lora
