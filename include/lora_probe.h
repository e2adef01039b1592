/* Measurement helpers outside the delta path (the benchmark's floors), beside
 * lora_probe_stream_read in lora_sgmv.h.  Same status codes and conventions
 * as lora_sgmv.h. */
#ifndef LORA_PROBE_H
#define LORA_PROBE_H

#include "lora_sgmv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The price of a device-scope release per workgroup, what a reduction across
 * the workgroups of one launch has to pay: 2 * pairs workgroups each write 64
 * floats to part [2 * pairs * 64]; with fence = 1 each then releases them at
 * device scope and counts itself on counters[pair] [pairs], and the second of
 * each pair acquires and writes the sum of both to out [pairs * 64],
 * resetting its counter to 0 (fence = 0: the writes only).  No workgroup
 * waits for another.  All pointers device memory; counters must hold zeros
 * before the first call, and every call leaves them zero; calls that overlap
 * race on the counters.  Errors: LORA_EINVAL (pairs outside 0..2^20, fence
 * not 0 or 1, a null pointer), LORA_EHIP. */
lora_status lora_probe_release(int32_t pairs, int32_t fence, float *part, uint32_t *counters, float *out,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_PROBE_H */
