// Measurement helper, outside the delta path: a bare streaming read of given
// size and workgroup count.  bench.py times it to show what a kernel that
// moves a given number of bytes with a given number of workgroups cannot beat
// on this device (the launch and memory-latency floor of small launches).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lora_internal.h"
#include "lora_probe.h"

using namespace lora;

namespace {

// Workgroup g reads the 16-byte chunks [g n16, (g + 1) n16) of src, eight
// loads in flight per thread (NT: with the non-temporal hint), and folds them
// into one word that is stored only in the (practically impossible) case that
// it equals a magic value, so the loads stay live while nothing is written.
typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 probe_load(const uint4 *p) {
  if constexpr (NT) {
    const probe_u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const probe_u32x4 *>(p));
    return make_uint4(q.x, q.y, q.z, q.w);
  } else {
    return *p;
  }
}
template <bool NT>
__global__ __launch_bounds__(1024) void stream_read_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                           uint32_t *__restrict__ sink) {
  const uint4 *p = src + (int64_t)blockIdx.x * n16;
  const int nt = blockDim.x;
  uint32_t acc = 0;
  int64_t i = threadIdx.x;
  for (; i + 7 * (int64_t)nt < n16; i += 8 * (int64_t)nt) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = probe_load<NT>(p + i + u * nt);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += nt) {
    const uint4 v = probe_load<NT>(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// The cost of a device-scope release per workgroup (the pattern a reduction
// across workgroups of one launch needs): workgroup b of 2 * pairs writes 64
// values; with FENCE it then releases them at device scope, counts itself on
// its pair's counter, and the pair's second arriver acquires and adds both
// workgroups' values in a fixed order, then puts the counter back to zero so
// that the next launch starts from zero.  Nothing waits on another workgroup.
template <bool FENCE>
__global__ __launch_bounds__(256) void release_pair_kernel(float *__restrict__ part, unsigned *__restrict__ cnt,
                                                           float *__restrict__ out) {
  const int b = blockIdx.x, tid = threadIdx.x, pair = b >> 1;
  float acc = 0.f;
  for (int i = 0; i < 64; ++i) acc = fmaf(acc, 1.0001f, (float)(tid + i));
  if (tid < 64) part[(size_t)b * 64 + tid] = acc;
  if constexpr (FENCE) {
    __shared__ unsigned arrived;
    __threadfence();
    __syncthreads();
    if (tid == 0) arrived = atomicAdd(&cnt[pair], 1u);
    __syncthreads();
    if (arrived == 1u) {
      __threadfence();
      if (tid < 64) out[(size_t)pair * 64 + tid] = part[(size_t)(2 * pair) * 64 + tid] +
                                                    part[(size_t)(2 * pair + 1) * 64 + tid];
      if (tid == 0) atomicExch(&cnt[pair], 0u);
    }
  }
}

}  // namespace

extern "C" lora_status lora_probe_release(int32_t pairs, int32_t fence, float *part, uint32_t *counters,
                                          float *out, hipStream_t stream) {
  if (pairs < 0) return fail(LORA_EINVAL, "negative pairs");
  if (fence != 0 && fence != 1) return fail(LORA_EINVAL, "fence must be 0 or 1");
  if (pairs == 0) return ok();
  if (!part || !counters || !out) return fail(LORA_EINVAL, "null pointer");
  if (pairs > (1 << 20)) return fail(LORA_EINVAL, "more than 2^20 pairs");
  if (fence)
    hipLaunchKernelGGL(release_pair_kernel<true>, dim3(2 * pairs), dim3(256), 0, stream, part, counters, out);
  else
    hipLaunchKernelGGL(release_pair_kernel<false>, dim3(2 * pairs), dim3(256), 0, stream, part, counters, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

extern "C" lora_status lora_probe_stream_read(const void *src, int64_t bytes_per_group, int32_t groups,
                                              int32_t threads, int32_t nontemporal, uint32_t *sink,
                                              hipStream_t stream) {
  if (groups < 0 || bytes_per_group < 0) return fail(LORA_EINVAL, "negative size");
  if (groups == 0 || bytes_per_group == 0) return ok();
  if (!src || !sink) return fail(LORA_EINVAL, "null pointer");
  if (((uintptr_t)src & 15u) || bytes_per_group % 16)
    return fail(LORA_EINVAL, "src and bytes_per_group must be multiples of 16 bytes");
  if (threads < 64 || threads > 1024 || threads % 64)
    return fail(LORA_EINVAL, "threads must be a multiple of 64 in 64..1024");
  if (nontemporal != 0 && nontemporal != 1) return fail(LORA_EINVAL, "nontemporal must be 0 or 1");
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(groups), dim3(threads), 0, stream, (const uint4 *)src,
                       bytes_per_group / 16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(groups), dim3(threads), 0, stream, (const uint4 *)src,
                       bytes_per_group / 16, sink);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}
