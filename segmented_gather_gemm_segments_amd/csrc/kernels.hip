// Kernel half of the library: the shrink and expand kernels for gfx950
// (CDNA4), their launchers, and argument validation.
//
// Operation ("Multi-LoRA serving: the single translator with a thousand
// glossaries", section "SGMV: the kernel that holds it all up"):
//   shrink   v[t][j] = sum_k A_{a(t)}[j][k] x[t][k]               j < r_{a(t)}
//   expand   y[t][i] = round(y[t][i] + sum_j B_{a(t)}[i][j] v[t][j])
// Every adapter of a batch is handled by one launch per phase.  A work item
// names up to 64 tokens of one adapter; its workgroup takes one of two paths:
//   * gather/GEMV (short segments, decode): lanes run along the contiguous
//     dimension of the adapter rows with 16-byte loads; shrink reduces the
//     lane partials with a cross-lane butterfly and a fixed-order sum over the
//     four waves;
//   * MFMA (long segments): the per-adapter product is a dense GEMM and runs on
//     v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (fp32).
//     The bf16 expand feeds the fp32 v to the matrix cores as a pair of bf16
//     values hi + lo (two MFMA K-halves): hi = RNE(v), lo = RNE(v - hi) keep
//     about 16 significant bits of v (relative error at most about 2^-17), far
//     more than one bf16 (8 bits) but fewer than fp32's 24, so the MFMA and
//     gather expands agree to rounding, not bit for bit;
//   * tiled shrink (long segments, bf16 activations): 64-token tiles of x and
//     A streamed into LDS by direct global-to-LDS loads, over slices of d_in
//     whose partial products a second launch adds in slice order.
// The per-token (decode) mode has the same two paths plus a fused kernel that
// runs one token's shrink and expand in one workgroup.
// No floating-point atomics: every output element is produced by one thread
// and summation orders are fixed, so repeated runs are bit-identical.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "lora_internal.h"

using namespace lora;

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kThreads = 256;  // 4 waves of 64

// ----------------------------------------------------------------- weights
// Adapter rows are stored in one of four element types W: bf16 (uint16_t) or
// fp32 (float) like the activations, or -- with bf16 activations only -- OCP
// FP8 E4M3 (Fp8) or two's-complement INT4 (Int4), each row with an fp32 scale.
// A row's value is code * scale ("Multi-LoRA Inference Serving": FP8 adapter
// storage halves the adapter bytes, INT4 adapters are dequantised in the
// layer).  The scales factor out of both phases exactly: the shrink multiplies
// v[j] by A row j's scale after its sum, the expand multiplies v[j] by B^T
// row j's scale before use, and the codes themselves convert exactly to fp32
// (and to bf16).
struct Fp8 {};
struct Int4 {};

template <typename W> struct WT;  // bytes per 8-element chunk; per-row scale?
template <> struct WT<uint16_t> { static constexpr int kChunk = 16; static constexpr bool kScaled = false; };
template <> struct WT<float> { static constexpr int kChunk = 32; static constexpr bool kScaled = false; };
template <> struct WT<Fp8> { static constexpr int kChunk = 8; static constexpr bool kScaled = true; };
template <> struct WT<Int4> { static constexpr int kChunk = 4; static constexpr bool kScaled = true; };

struct DevW {
  const char *a_pages;
  const char *b_pages;
  const int32_t *rank;
  const int32_t *a_pt;
  const int32_t *b_pt;
  const float *a_sc;   // per stored row (page * page_rows + row in page); quantized rows only
  const float *b_sc;
  int64_t a_row_bytes, b_row_bytes;
  int32_t d_in, d_out, num_adapters, r_max, page_rows, max_pages, num_pages_a, num_pages_b;
};

// ----------------------------------------------------------------- debug checks
// With LORA_DEBUG (the debug build of the library) the kernels record the bad
// device-side values they skip -- a page id outside the pool for a row below
// the rank, an adapter id outside {-1} U [0, N), a rank outside 1..r_max, a
// token index outside the batch, a malformed plan item -- as LORA_DEBUG_* bits
// in a device word that lora_debug_flags reads back.  Every kernel still
// skips such values and exits normally; release builds compile the checks
// away.
#ifndef LORA_DEBUG
#define LORA_DEBUG 0
#endif
#if LORA_DEBUG
__device__ uint32_t g_debug_flags;
__device__ __forceinline__ void debug_flag(uint32_t bit) {
  __hip_atomic_fetch_or(&g_debug_flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#define LORA_CHECK(cond, bit) \
  do {                        \
    if (!(cond)) debug_flag(bit); \
  } while (0)
#else
#define LORA_CHECK(cond, bit) \
  do {                        \
  } while (0)
#endif

// Storage index (page * page_rows + row in page) of row j of adapter a through
// the page table, or -1 when the page id is out of range (the row then
// contributes nothing).  The page-id load is unconditional (clamped index) so
// that several rows' lookups can be in flight together.
__device__ __forceinline__ int64_t row_index(const DevW &w, const int32_t *pt, int32_t num_pages,
                                             int a, int j) {
  int page, r_in;
  if (pt) {
    const int pi = j / w.page_rows;
    page = pt[(int64_t)a * w.max_pages + (pi < w.max_pages ? pi : w.max_pages - 1)];
    if (pi >= w.max_pages) page = -1;
    r_in = j - pi * w.page_rows;
  } else {
    page = a;
    r_in = j;
  }
  if ((unsigned)page >= (unsigned)num_pages) return -1;
  return (int64_t)page * w.page_rows + r_in;
}

// Byte address of row j of adapter a's A (or B^T); nullptr when out of range.
// (Called for rows below the adapter's rank only.)
__device__ __forceinline__ const char *a_row(const DevW &w, int a, int j) {
  const int64_t i = row_index(w, w.a_pt, w.num_pages_a, a, j);
  LORA_CHECK(i >= 0, LORA_DEBUG_BAD_PAGE);
  return i < 0 ? nullptr : w.a_pages + i * w.a_row_bytes;
}
__device__ __forceinline__ const char *b_row(const DevW &w, int a, int j) {
  const int64_t i = row_index(w, w.b_pt, w.num_pages_b, a, j);
  LORA_CHECK(i >= 0, LORA_DEBUG_BAD_PAGE);
  return i < 0 ? nullptr : w.b_pages + i * w.b_row_bytes;
}
// Scale of row j (1 for unquantized rows or an out-of-range page).
template <typename W>
__device__ __forceinline__ float a_scale(const DevW &w, int a, int j) {
  if constexpr (!WT<W>::kScaled) return 1.f;
  const int64_t i = row_index(w, w.a_pt, w.num_pages_a, a, j);
  LORA_CHECK(i >= 0, LORA_DEBUG_BAD_PAGE);
  return i < 0 ? 0.f : w.a_sc[i];
}
template <typename W>
__device__ __forceinline__ float b_scale(const DevW &w, int a, int j) {
  if constexpr (!WT<W>::kScaled) return 1.f;
  const int64_t i = row_index(w, w.b_pt, w.num_pages_b, a, j);
  LORA_CHECK(i >= 0, LORA_DEBUG_BAD_PAGE);
  return i < 0 ? 0.f : w.b_sc[i];
}

// One side of the adapter storage: A rows or B^T rows.
struct Side {
  const char *pages;
  const int32_t *pt;
  const float *sc;
  int64_t row_bytes;
  int32_t num_pages;
};
__device__ __forceinline__ Side side_a(const DevW &w) {
  return {w.a_pages, w.a_pt, w.a_sc, w.a_row_bytes, w.num_pages_a};
}
__device__ __forceinline__ Side side_b(const DevW &w) {
  return {w.b_pages, w.b_pt, w.b_sc, w.b_row_bytes, w.num_pages_b};
}

// Branch-free pointer select (a conditional expression on pointers tends to
// become a branch per row).
__device__ __forceinline__ const char *sel_ptr(bool c, const char *p, const char *q) {
  const uintptr_t m = (uintptr_t)0 - (uintptr_t)c;
  return reinterpret_cast<const char *>((reinterpret_cast<uintptr_t>(p) & m) |
                                        (reinterpret_cast<uintptr_t>(q) & ~m));
}

// Addresses of rows j0 .. j0+15 of adapter a on one side, offset to element
// `col` (rows at or past `r`, or on an out-of-range page, get `safe`), and,
// when SC, the lane scale `lsc`: lane l holds the scale of row j0 + (l & 15)
// (0 for rows without one; 1 for unquantized rows), read back per row with
// row_sc -- one vector load for the 16 scales instead of 16 dependent scalar
// loads.  Lanes 0..15 of the wave must all execute this call.  When the 16
// rows lie in one page (the usual case: 16-row pages, j0 a multiple of 16) a
// single page lookup serves them all; a dense stack needs none.  AL: the
// caller guarantees that case (dense rows, or pages of a multiple of 16 rows
// with j0 a multiple of 16), and the per-row fallback is not compiled.  The
// scale load is unconditional (index 0 stands in for rows without one).
template <typename W, bool SC = true, bool AL = false>
__device__ __forceinline__ void rows16(const DevW &w, const Side &sd, int a, int j0, int r, int col,
                                       const char *safe, const char *(&rp)[16], float &lsc) {
  const int pr = w.page_rows;
  const int64_t cofs = (int64_t)(col >> 3) * WT<W>::kChunk;
  const int li = threadIdx.x & 15;
  if (AL || !sd.pt || (pr >= 16 && j0 % pr + 16 <= pr)) {
    int page, r0;
    if (sd.pt) {
      const int pi = j0 / pr;
      page = sd.pt[(int64_t)a * w.max_pages + (pi < w.max_pages ? pi : w.max_pages - 1)];
      page = pi < w.max_pages ? page : -1;
      r0 = j0 - pi * pr;
    } else {
      page = a;
      r0 = j0;
    }
    const bool ok = (unsigned)page < (unsigned)sd.num_pages;
    LORA_CHECK(ok || j0 >= r, LORA_DEBUG_BAD_PAGE);
    const int64_t i0 = (int64_t)(ok ? page : 0) * pr + r0;
    const char *base = sd.pages + i0 * sd.row_bytes + cofs;
#pragma unroll
    for (int i = 0; i < 16; ++i) rp[i] = sel_ptr(ok && j0 + i < r, base + i * sd.row_bytes, safe);
    if constexpr (SC && WT<W>::kScaled) {
      const bool in = ok && j0 + li < r;
      const float s = sd.sc[in ? i0 + li : 0];
      lsc = in ? s : 0.f;
    } else {
      lsc = 1.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t idx = j0 + i < r ? row_index(w, sd.pt, sd.num_pages, a, j0 + i) : -1;
      LORA_CHECK(idx >= 0 || j0 + i >= r, LORA_DEBUG_BAD_PAGE);
      rp[i] = idx >= 0 ? sd.pages + idx * sd.row_bytes + cofs : safe;
    }
    if constexpr (SC && WT<W>::kScaled) {
      const int64_t idx = j0 + li < r ? row_index(w, sd.pt, sd.num_pages, a, j0 + li) : -1;
      const float s = sd.sc[idx >= 0 ? idx : 0];
      lsc = idx >= 0 ? s : 0.f;
    } else {
      lsc = 1.f;
    }
  }
}
// Scale of row j0 + i from a lane scale of rows16 (i uniform, 0..15).
template <typename W>
__device__ __forceinline__ float row_sc(float lsc, int i) {
  if constexpr (!WT<W>::kScaled) return 1.f;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsc), i));
}
template <typename W, bool AL = false>
__device__ __forceinline__ void b_rows16(const DevW &w, int a, int j0, int r, int col, const char *safe,
                                         const char *(&rp)[16], float &lsc) {
  rows16<W, true, AL>(w, side_b(w), a, j0, r, col, safe, rp, lsc);
}

// Byte addresses of N rows j[i] (>= 0) of adapter a on one side, each plus
// `ofs`, or `safe` where !use[i] or the row's page is past the page table or
// out of range; stored[i] gets the row's storage index (page * page_rows + row
// in page), or -1 where `safe` is returned.  All N page-id loads are issued
// (clamped indices, unconditional) before any is used, and the rest is
// selects, not branches: the lookups overlap each other and do not wait for
// loads issued before them.  Storage indices fit int32: to_dev rejects pools
// of more than 2^31 - 1 stored rows.
template <int N>
__device__ __forceinline__ void rows_addr(const DevW &w, const Side &sd, int a, const int (&j)[N],
                                          const bool (&use)[N], int64_t ofs, const char *safe,
                                          const char *(&p)[N], int (&stored)[N]) {
  const int pr = w.page_rows;
  int page[N], r_in[N];
  if (sd.pt) {
    const int32_t *row = sd.pt + (int64_t)a * w.max_pages;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int pi = j[i] / pr;
      page[i] = row[min(pi, w.max_pages - 1)];
      r_in[i] = j[i] - pi * pr;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) page[i] = j[i] / pr < w.max_pages ? page[i] : -1;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      page[i] = a;
      r_in[i] = j[i];
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool ok = use[i] && (unsigned)page[i] < (unsigned)sd.num_pages;
    LORA_CHECK(ok || !use[i], LORA_DEBUG_BAD_PAGE);
    const int idx = (int)((unsigned)page[i] * (unsigned)pr + (unsigned)r_in[i]);
    stored[i] = ok ? idx : -1;
    p[i] = sel_ptr(ok, sd.pages + (int64_t)(ok ? idx : 0) * sd.row_bytes + ofs, safe);
  }
}

__device__ __forceinline__ int adapter_rank(const DevW &w, int a) {
  int r = w.rank[a];
  return r < 0 ? 0 : (r > w.r_max ? w.r_max : r);
}
// The rank of an adapter that a token uses (checked in the debug build).
__device__ __forceinline__ int used_rank(const DevW &w, int a) {
  const int r = w.rank[a];
  LORA_CHECK(r >= 1 && r <= w.r_max, LORA_DEBUG_BAD_RANK);
  return r < 0 ? 0 : (r > w.r_max ? w.r_max : r);
}
// An adapter id read from the device: -1 (no adapter) or in [0, N).
__device__ __forceinline__ void check_id(const DevW &w, int a) {
  LORA_CHECK(a == LORA_NO_ADAPTER || (a >= 0 && a < w.num_adapters), LORA_DEBUG_BAD_ADAPTER);
}

// ----------------------------------------------------------------- elements
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 8 consecutive elements -> fp32 (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void load8(const uint16_t *p, float (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
  o[4] = bf16_lo(u.z); o[5] = bf16_hi(u.z); o[6] = bf16_lo(u.w); o[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void load8(const float *p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t *p, const float (&o)[8]) {
  uint4 u;
  u.x = bf16_rne(o[0]) | (bf16_rne(o[1]) << 16);
  u.y = bf16_rne(o[2]) | (bf16_rne(o[3]) << 16);
  u.z = bf16_rne(o[4]) | (bf16_rne(o[5]) << 16);
  u.w = bf16_rne(o[6]) | (bf16_rne(o[7]) << 16);
  *reinterpret_cast<uint4 *>(p) = u;
}
__device__ __forceinline__ void store8(float *p, const float (&o)[8]) {
  *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<float4 *>(p + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

// MFMA operand fragments: 8 consecutive elements of one row per lane.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> { uint4 u; };
template <> struct Frag<float> { float4 a, b; };

__device__ __forceinline__ void frag_load(Frag<uint16_t> &f, const uint16_t *p) {
  f.u = *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void frag_load(Frag<float> &f, const float *p) {
  f.a = *reinterpret_cast<const float4 *>(p);
  f.b = *reinterpret_cast<const float4 *>(p + 4);
}
__device__ __forceinline__ void frag_zero(Frag<uint16_t> &f) { f.u = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void frag_zero(Frag<float> &f) {
  f.a = make_float4(0, 0, 0, 0);
  f.b = f.a;
}

// D += A·B over the 8 k-elements held per lane.  For both types the k index
// contracted is (lane group, element), identical for A and B, so the product
// is a plain dot product over the 32 k of the step whatever order the unit
// uses internally.
__device__ __forceinline__ f32x4_t frag_mfma(const Frag<uint16_t> &a, const Frag<uint16_t> &b,
                                             f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                 __builtin_bit_cast(bf16x8_t, b.u), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t frag_mfma(const Frag<float> &a, const Frag<float> &b,
                                             f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ----------------------------------------------------------------- reductions
constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Reduce-scatter of NV values (a power of two <= 64) over the 64 lanes of a
// wave: on return lane l holds the wave-wide sum of vals[l >> (6 - log2 NV)].
// Halving butterfly steps with masks 32, 16, ... while values remain, then
// plain butterflies for the rest.  The masks are always applied in the order
// 32 .. 1, so every value is summed over the same lane tree whatever NV is: a
// token's result does not depend on how many values were reduced beside it.
template <int NV>
__device__ __forceinline__ float wave_reduce_scatter(float (&vals)[NV]) {
  static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of two <= 64");
  constexpr int LOG = ilog2(NV);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int step = 0; step < LOG; ++step) {
    const int n = NV >> step;
    const int m = 32 >> step;
    // bitwise select (v_bfi_b32): a value select here would be folded into
    // an address select and push the array out of registers
    const uint32_t up = (lane & m) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const uint32_t lo = __float_as_uint(vals[i]), hi = __float_as_uint(vals[i + n / 2]);
      const float keep = __uint_as_float((up & hi) | (~up & lo));
      const float send = __uint_as_float((up & lo) | (~up & hi));
      vals[i] = keep + __shfl_xor(send, m, 64);
    }
  }
  float s = vals[0];
#pragma unroll
  for (int m = 32 >> LOG; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  return s;
}

// Raw 8-element chunks (16 B of bf16 or 32 B of fp32): loads are issued as a
// batch first and converted afterwards, so a thread keeps many in flight.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> { uint4 u; };
template <> struct Raw8<float> { float4 a, b; };
__device__ __forceinline__ void raw_load(Raw8<uint16_t> &r, const uint16_t *p) {
  r.u = *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void raw_load(Raw8<float> &r, const float *p) {
  r.a = *reinterpret_cast<const float4 *>(p);
  r.b = *reinterpret_cast<const float4 *>(p + 4);
}
__device__ __forceinline__ void raw_cvt(const Raw8<uint16_t> &r, float (&o)[8]) {
  o[0] = bf16_lo(r.u.x); o[1] = bf16_hi(r.u.x); o[2] = bf16_lo(r.u.y); o[3] = bf16_hi(r.u.y);
  o[4] = bf16_lo(r.u.z); o[5] = bf16_hi(r.u.z); o[6] = bf16_lo(r.u.w); o[7] = bf16_hi(r.u.w);
}
__device__ __forceinline__ void raw_cvt(const Raw8<float> &r, float (&o)[8]) {
  o[0] = r.a.x; o[1] = r.a.y; o[2] = r.a.z; o[3] = r.a.w;
  o[4] = r.b.x; o[5] = r.b.y; o[6] = r.b.z; o[7] = r.b.w;
}
__device__ __forceinline__ void raw_zero(Raw8<uint16_t> &r) { r.u = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void raw_zero(Raw8<float> &r) {
  r.a = make_float4(0.f, 0.f, 0.f, 0.f);
  r.b = r.a;
}
// Element e (0..7, a compile-time index after unrolling) of a raw chunk, as stored.
__device__ __forceinline__ uint16_t raw_elem(const Raw8<uint16_t> &r, int e) {
  const uint32_t wd = e < 2 ? r.u.x : e < 4 ? r.u.y : e < 6 ? r.u.z : r.u.w;
  return (uint16_t)(e & 1 ? wd >> 16 : wd & 0xffffu);
}
__device__ __forceinline__ float raw_elem(const Raw8<float> &r, int e) {
  const float4 q = e < 4 ? r.a : r.b;
  const int i = e & 3;
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// Quantized weight chunks: 8 FP8 E4M3 codes (8 bytes) or 8 INT4 codes (4 bytes).
template <> struct Raw8<Fp8> { uint2 u; };
template <> struct Raw8<Int4> { uint32_t u; };

// Loads of one 8-element weight chunk from a byte address.  ST: the load
// carries the non-temporal hint, for rows that no later load of the launch
// reads again (on this device a stream of such loads moves 10-15 % more bytes
// per second than plain loads once it spans ~100 MB or more; where other
// items read the same rows later, the hint costs more than it saves).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool ST = false>
__device__ __forceinline__ void wload(Raw8<uint16_t> &r, const char *p) {
  if constexpr (ST) {
    const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    r.u = make_uint4(q.x, q.y, q.z, q.w);
  } else {
    r.u = *reinterpret_cast<const uint4 *>(p);
  }
}
template <bool ST = false>
__device__ __forceinline__ void wload(Raw8<float> &r, const char *p) {
  raw_load(r, reinterpret_cast<const float *>(p));
}
template <bool ST = false>
__device__ __forceinline__ void wload(Raw8<Fp8> &r, const char *p) {
  if constexpr (ST) {
    const u32x2_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    r.u = make_uint2(q.x, q.y);
  } else {
    r.u = *reinterpret_cast<const uint2 *>(p);
  }
}
template <bool ST = false>
__device__ __forceinline__ void wload(Raw8<Int4> &r, const char *p) {
  if constexpr (ST) r.u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
  else r.u = *reinterpret_cast<const uint32_t *>(p);
}
__device__ __forceinline__ void raw_zero(Raw8<Fp8> &r) { r.u = make_uint2(0, 0); }
__device__ __forceinline__ void raw_zero(Raw8<Int4> &r) { r.u = 0; }

// Codes to fp32, exactly: FP8 E4M3 through the converter (gfx950 decodes the
// OCP encoding), INT4 by sign extension of each nibble (element e in bits
// 4e .. 4e+3).
__device__ __forceinline__ void raw_cvt(const Raw8<Fp8> &r, float (&o)[8]) {
  const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(r.u.x, false);
  const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(r.u.x, true);
  const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8(r.u.y, false);
  const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8(r.u.y, true);
  o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
  o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
}
__device__ __forceinline__ void raw_cvt(const Raw8<Int4> &r, float (&o)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)((int32_t)(r.u << (28 - 4 * e)) >> 28);
}

// The 8 elements as bf16 bit patterns (exact for every weight type used with
// bf16 activations: FP8 E4M3 and INT4 values are bf16 values).
__device__ __forceinline__ uint4 raw_bf16(const Raw8<uint16_t> &r) { return r.u; }
template <typename W>
__device__ __forceinline__ uint4 raw_bf16(const Raw8<W> &r) {
  float f[8];
  raw_cvt(r, f);
  return make_uint4((__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u),
                    (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xffff0000u),
                    (__float_as_uint(f[4]) >> 16) | (__float_as_uint(f[5]) & 0xffff0000u),
                    (__float_as_uint(f[6]) >> 16) | (__float_as_uint(f[7]) & 0xffff0000u));
}

// Element e of a weight chunk in the activation type T's representation (bf16
// bits for T = uint16_t, the value for T = float), for LDS staging.
template <typename T, typename W>
__device__ __forceinline__ T w_as_t(const Raw8<W> &r, int e) {
  if constexpr (sizeof(T) == 4) {
    return raw_elem(r, e);
  } else {
    const uint4 b = raw_bf16(r);
    const uint32_t wd = e < 2 ? b.x : e < 4 ? b.y : e < 6 ? b.z : b.w;
    return (uint16_t)(e & 1 ? wd >> 16 : wd & 0xffffu);
  }
}

// Byte offset of element k (a multiple of 8) within a weight row.
// (k * bytes-per-element with a compile-time factor, so that offsets of
// unrolled steps fold into the load instructions' immediates)
template <typename W>
__device__ __forceinline__ int wofs(int k) {
  if constexpr (WT<W>::kChunk >= 8) return k * (WT<W>::kChunk / 8);
  else return k >> 1;  // INT4: two elements per byte (k is a multiple of 8)
}

// MFMA A-operand fragment (8 consecutive k of one weight row) from a byte
// address: loaded as is for bf16 / fp32 rows, converted exactly to bf16 for
// quantized rows (whose codes are bf16 values; the row scale is applied to the
// MFMA result).
template <typename T, typename W>
__device__ __forceinline__ void wfrag_load(Frag<T> &f, const char *p) {
  if constexpr (sizeof(T) == 4) {
    frag_load(f, reinterpret_cast<const float *>(p));
  } else {
    Raw8<W> r;
    wload(r, p);
    f.u = raw_bf16(r);
  }
}

// ----------------------------------------------------------------- shrink cores
// Token list of the current item in LDS: toks[0..cnt).  Tokens outside
// [0, num_tokens) are skipped.
constexpr int kMaxItemTokens = 256;
constexpr int kRowGroup = LORA_SHRINK_GATHER_ROWS;    // rows of A per segmented gather item
constexpr int kGatherCols = LORA_EXPAND_GATHER_COLS;  // columns of y per segmented gather item
static_assert(kGatherCols == kThreads * 8, "one 8-column chunk per thread");
#ifndef LORA_SGMV_SHRINK_THREADS
#define LORA_SGMV_SHRINK_THREADS 512
#endif
constexpr int kSgmvShrinkThreads = LORA_SGMV_SHRINK_THREADS;  // threads of a segmented shrink workgroup
static_assert(kSgmvShrinkThreads % 64 == 0 && kSgmvShrinkThreads <= 1024, "whole waves, <= 1024");

// Per-token (BGMV) work split: rows of A per shrink workgroup, and threads per
// expand workgroup (8 columns of y per thread).
#ifndef LORA_BGMV_SHRINK_ROWS
#define LORA_BGMV_SHRINK_ROWS 2
#endif
#ifndef LORA_BGMV_EXPAND_THREADS
#define LORA_BGMV_EXPAND_THREADS 128
#endif
constexpr int kBgmvRows = LORA_BGMV_SHRINK_ROWS;
constexpr int kBgmvExpandThreads = LORA_BGMV_EXPAND_THREADS;
static_assert(kBgmvRows == 1 || kBgmvRows == 2 || kBgmvRows == 4, "BGMV shrink rows: 1, 2 or 4");
static_assert(kBgmvExpandThreads % 64 == 0 && kBgmvExpandThreads <= kThreads, "whole waves");

// LDS of a shrink workgroup of NW waves.
template <int NW>
struct alignas(16) ShrinkSmem {
  int toks[kMaxItemTokens];
  union {
    float red_gemv[NW * 64];           // one value per (wave, value index)
    float red_mfma[NW * 4 * 4 * 64];   // [wave][row tile][element][lane]
  };
};

// One gather/GEMV shrink tile: tokens toks[g0 .. g0+ntok) (ntok <= TG) against
// the rows [j0, j0+nr) (nr <= RB) of adapter a.  The 64 NW threads split d_in
// into 8-element chunks (thread tid: k = 8 tid + 512 NW s); each pass issues
// the loads of two such steps (TG x chunks and RB A chunks each) before the
// first FMA, and the x chunks of a token are reused across the rows in
// registers.  Rows and tokens beyond the tile read a safe in-bounds address
// (row 0 of x) and their sums are dropped.  The TG x RB lane partials are
// reduce-scattered over the wave and the NW wave results summed in wave order,
// so a token's result does not depend on TG or on which other tokens share the
// tile (for a given NW).
template <typename T, typename W, int TG, int RB, int NW, bool ST, typename SM>
__device__ __forceinline__ void shrink_rows_tile(const DevW &w, int a, int j0, int nr, const int *toks, int g0,
                                 int ntok, int num_tokens, const T *__restrict__ x,
                                 float *__restrict__ v, SM &sm) {
  constexpr int kStep = NW * 64 * 8;
  constexpr int NV = TG * RB;
  constexpr int SH = 6 - ilog2(NV);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T *safe = x;
  const T *xr[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int tok = t < ntok ? uniform(toks[g0 + t]) : -1;
    xr[t] = (tok >= 0 && tok < num_tokens) ? x + (int64_t)tok * w.d_in : safe;
  }
  const char *ar[RB];
#pragma unroll
  for (int jj = 0; jj < RB; ++jj) {
    const char *p = jj < nr ? a_row(w, a, j0 + jj) : nullptr;
    ar[jj] = p ? p : reinterpret_cast<const char *>(safe);
  }
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  // uniform trip count; every load is issued unconditionally (a step past
  // d_in reads chunk 0 and is not accumulated) so a pass keeps all its loads
  // in flight together
  for (int base = 0; base < w.d_in; base += 2 * kStep) {
    const int k0 = base + tid * 8, k1 = k0 + kStep;
    const bool one = k0 < w.d_in, two = k1 < w.d_in;
    const int c0 = one ? k0 : 0, c1 = two ? k1 : 0;
    Raw8<T> xa[TG], xb[TG];
    Raw8<W> aa[RB], ab[RB];
#pragma unroll
    for (int t = 0; t < TG; ++t) raw_load(xa[t], xr[t] + c0);
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) wload<ST>(aa[jj], ar[jj] + wofs<W>(c0));
#pragma unroll
    for (int t = 0; t < TG; ++t) raw_load(xb[t], xr[t] + c1);
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) wload<ST>(ab[jj], ar[jj] + wofs<W>(c1));
    float xv[TG][8];
    if (one) {
#pragma unroll
      for (int t = 0; t < TG; ++t) raw_cvt(xa[t], xv[t]);
#pragma unroll
      for (int jj = 0; jj < RB; ++jj) {
        float av[8];
        raw_cvt(aa[jj], av);
#pragma unroll
        for (int t = 0; t < TG; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t * RB + jj] = fmaf(av[e], xv[t][e], acc[t * RB + jj]);
      }
    }
    if (two) {
#pragma unroll
      for (int t = 0; t < TG; ++t) raw_cvt(xb[t], xv[t]);
#pragma unroll
      for (int jj = 0; jj < RB; ++jj) {
        float av[8];
        raw_cvt(ab[jj], av);
#pragma unroll
        for (int t = 0; t < TG; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t * RB + jj] = fmaf(av[e], xv[t][e], acc[t * RB + jj]);
      }
    }
  }
  const float part = wave_reduce_scatter<NV>(acc);
  if ((lane & ((1 << SH) - 1)) == 0) sm.red_gemv[wave * 64 + (lane >> SH)] = part;
  __syncthreads();
  if (tid < NV) {
    float s = sm.red_gemv[tid];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) s += sm.red_gemv[wv * 64 + tid];
    const int t = tid / RB, jj = tid % RB;
    if (t < ntok && jj < nr) {
      const int tok = toks[g0 + t];
      if (tok >= 0 && tok < num_tokens)
        v[(int64_t)tok * w.r_max + j0 + jj] = WT<W>::kScaled ? s * a_scale<W>(w, a, j0 + jj) : s;
    }
  }
  __syncthreads();
}

// Gather/GEMV shrink of tokens toks[0..cnt) of adapter a over its row group
// [j0, j0 + nr), nr <= RB: groups of up to 4 tokens, the last of 1 to 4.
// LAST: the last group reads the rows non-temporally (the item is the only
// reader of its row group, and that group its last).
template <typename T, typename W, int RB, int NW, bool LAST, typename SM>
__device__ __forceinline__ void shrink_gemv(const DevW &w, int a, int j0, int nr, const int *toks, int cnt,
                            int num_tokens, const T *__restrict__ x, float *__restrict__ v, SM &sm) {
  int g0 = 0;
  for (; g0 + 4 < cnt; g0 += 4)
    shrink_rows_tile<T, W, 4, RB, NW, false>(w, a, j0, nr, toks, g0, 4, num_tokens, x, v, sm);
  const int rest = cnt - g0;
  if (rest == 1) shrink_rows_tile<T, W, 1, RB, NW, LAST>(w, a, j0, nr, toks, g0, 1, num_tokens, x, v, sm);
  else if (rest == 2) shrink_rows_tile<T, W, 2, RB, NW, LAST>(w, a, j0, nr, toks, g0, 2, num_tokens, x, v, sm);
  else if (rest >= 3) shrink_rows_tile<T, W, 4, RB, NW, LAST>(w, a, j0, nr, toks, g0, rest, num_tokens, x, v, sm);
}

// One MFMA shrink tile: 16 tokens (this lane's token row xp, or a safe row)
// against RT row tiles of 16 starting at j0.  The NW waves take interleaved
// 32-element k-steps; each batch issues the loads of U steps before its
// MFMAs.  Lanes beyond the rank or the tile read safe rows whose outputs are
// dropped; the last, partial k-step zeroes both operands past d_in.  The wave
// results are summed in wave order.
template <typename T, typename W, int RT, int NW>
__device__ __forceinline__ void shrink_mfma_tile(const DevW &w, int a, int r, int j0, const T *xp, int tok,
                                 const T *__restrict__ x, float *__restrict__ v, ShrinkSmem<NW> &sm) {
  constexpr int U = RT == 1 ? 8 : 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const char *safe = reinterpret_cast<const char *>(x);
  const char *ap[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = j0 + rt * 16 + m;
    const char *p = row < r ? a_row(w, a, row) : nullptr;
    ap[rt] = p ? p : safe;
  }
  f32x4_t acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int full = w.d_in >> 5;             // k-steps entirely inside d_in
  const int nsteps = (w.d_in + 31) >> 5;
  int s = wave;
  for (; s + NW * (U - 1) < full; s += NW * U) {
    Frag<T> xf[U], af[U][RT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + NW * u) * 32 + g * 8;
      frag_load(xf[u], xp + k);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) wfrag_load<T, W>(af[u][rt], ap[rt] + wofs<W>(k));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = frag_mfma(af[u][rt], xf[u], acc[rt]);
  }
  for (; s < nsteps; s += NW) {
    const int k = s * 32 + g * 8;
    const bool kin = k < w.d_in;
    const int kc = kin ? k : 0;       // loads stay unconditional; past d_in they are zeroed
    Frag<T> xf, af[RT];
    frag_load(xf, xp + kc);
    if (!kin) frag_zero(xf);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      wfrag_load<T, W>(af[rt], ap[rt] + wofs<W>(kc));
      if (!kin) frag_zero(af[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = frag_mfma(af[rt], xf, acc[rt]);
  }
  // lane (g, m) of row tile rt holds D[4g + e][m] = v[tok(m)][j0 + 16 rt + 4g + e]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.red_mfma[((wave * 4 + rt) * 4 + e) * 64 + lane] = acc[rt][e];
  __syncthreads();
  if (wave < RT) {
    const int rt = wave;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s4 = sm.red_mfma[(rt * 4 + e) * 64 + lane];
#pragma unroll
      for (int wv = 1; wv < NW; ++wv) s4 += sm.red_mfma[((wv * 4 + rt) * 4 + e) * 64 + lane];
      const int j = j0 + rt * 16 + 4 * g + e;
      if (tok >= 0 && j < r)
        v[(int64_t)tok * w.r_max + j] = WT<W>::kScaled ? s4 * a_scale<W>(w, a, j) : s4;
    }
  }
  __syncthreads();
}

// MFMA shrink for tokens toks[0..cnt) of adapter a: 16-token tiles, passes of
// up to 64 rows.
template <typename T, typename W, int NW>
__device__ __forceinline__ void shrink_mfma(const DevW &w, int a, int r, const int *toks, int cnt, int num_tokens,
                            const T *__restrict__ x, float *__restrict__ v, ShrinkSmem<NW> &sm) {
  const int m = threadIdx.x & 15;
  for (int m0 = 0; m0 < cnt; m0 += 16) {
    int tok = m0 + m < cnt ? toks[m0 + m] : -1;
    if (tok >= num_tokens) tok = -1;
    const T *xp = tok >= 0 ? x + (int64_t)tok * w.d_in : x;
    for (int j0 = 0; j0 < r; j0 += 64) {
      const int nrt = min(4, (r - j0 + 15) >> 4);
      switch (nrt) {
        case 1: shrink_mfma_tile<T, W, 1, NW>(w, a, r, j0, xp, tok, x, v, sm); break;
        case 2: shrink_mfma_tile<T, W, 2, NW>(w, a, r, j0, xp, tok, x, v, sm); break;
        case 3: shrink_mfma_tile<T, W, 3, NW>(w, a, r, j0, xp, tok, x, v, sm); break;
        default: shrink_mfma_tile<T, W, 4, NW>(w, a, r, j0, xp, tok, x, v, sm); break;
      }
    }
  }
}

// ----------------------------------------------------------------- expand cores
// The MFMA expand stages the rank dimension kExpandK indices at a time, so the
// LDS of a workgroup (about 31 KiB) lets several workgroups share a CU.
#ifndef LORA_EXPAND_K
#define LORA_EXPAND_K 32
#endif
constexpr int kExpandK = LORA_EXPAND_K;
static_assert(kExpandK % 16 == 0 && kExpandK <= 64, "rank chunk: 16, 32, 48 or 64");
template <typename T> struct ExpandCfg;
template <> struct ExpandCfg<uint16_t> { static constexpr int kRowStride = kExpandK + 8; };  // j + pad
template <> struct ExpandCfg<float> { static constexpr int kRowStride = kExpandK + 4; };

constexpr int kVStride = kExpandK + 4;  // LDS row stride (floats) of the staged v rows: j + pad
// bf16 activations: each staged v row holds the chunk's bf16 hi parts, then
// its bf16 lo parts (v = hi + lo to about 16 significant bits), then a pad; the
// split is done once per staged chunk instead of in every wave's MFMA loop.
constexpr int kVhlStride = 2 * kExpandK + 8;  // bf16 elements

template <typename T>
struct alignas(16) ExpandSmem {
  int toks[kMaxItemTokens];
  T bt[4 * 64 * ExpandCfg<T>::kRowStride];  // MFMA path, per wave: [64 cols][j]
  union {
    float vs[64 * kVStride];       // MFMA path, fp32: [token][j] of the 64 tokens
    uint16_t vhl[64 * kVhlStride];  // MFMA path, bf16: [token][hi j | lo j | pad]
  };
};

// One gather/GEMV expand tile: tokens toks[g0 .. g0+ntok) (ntok <= TG) over
// the 8 NT columns of block cb (NT = threads of the workgroup).  Thread tid
// owns the 8 consecutive columns 8 (NT cb + tid) and runs the whole rank sum
// for them itself -- no cross-lane or cross-wave reduction, no barrier.  B^T rows are loaded 16 at a time
// (16-byte loads, all issued before the first FMA); the y chunks of the tile's
// tokens are fetched at the start; v is read as uniform values.  Every output
// is y + sum_j v_j b_j summed in ascending j, independent of TG.
template <typename T, typename W, int TG, int NT, bool ST = false>
__device__ __forceinline__ void expand_cols_tile(const DevW &w, int a, int r, int cb, const int *toks, int g0,
                                 int ntok, int num_tokens, const float *__restrict__ v,
                                 T *__restrict__ y) {
  // columns past d_out compute on column 0 and store nothing (the whole wave
  // stays active: rows16's lane scales need lanes 0..15)
  const int col_t = (cb * NT + (int)threadIdx.x) * 8;
  const bool cin = col_t < w.d_out;
  const int col = cin ? col_t : 0;
  int tk[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int tok = t < ntok ? uniform(toks[g0 + t]) : -1;
    tk[t] = (tok >= 0 && tok < num_tokens) ? tok : -1;
  }
  // every load is issued unconditionally (token row 0 stands in for an absent
  // token; its values are not used) so the tile's loads are in flight together
  Raw8<T> yraw[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) raw_load(yraw[t], y + (int64_t)(tk[t] >= 0 ? tk[t] : 0) * w.d_out + col);
  const char *safe = w.b_pages;
  const bool vec_v = (w.r_max & 3) == 0;
  float acc[TG][8];
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
  for (int j0 = 0; j0 < r; j0 += 16) {
    // all 16 row addresses first (their page lookups in flight together), then
    // all 16 row loads
    const char *rp[16];
    float lsc;
    b_rows16<W>(w, a, j0, r, col, safe, rp, lsc);
    Raw8<W> braw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wload<ST>(braw[i], rp[i]);
    // v[tok][j0 .. j0+16): the same address in every lane, read with 16-byte
    // vector loads (one request per wave) where r_max keeps them aligned
    float vj[TG][16];
    if (vec_v && j0 + 16 <= w.r_max) {
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const float *vr = v + (int64_t)(tk[t] >= 0 ? tk[t] : 0) * w.r_max + j0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *reinterpret_cast<const float4 *>(vr + 4 * q);
          vj[t][4 * q] = f.x; vj[t][4 * q + 1] = f.y; vj[t][4 * q + 2] = f.z; vj[t][4 * q + 3] = f.w;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const float *vr = v + (int64_t)(tk[t] >= 0 ? tk[t] : 0) * w.r_max;
#pragma unroll
        for (int i = 0; i < 16; ++i) vj[t][i] = vr[min(j0 + i, w.r_max - 1)];
      }
    }
    // B^T row scales fold into v (quantized rows; 1 otherwise)
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        vj[t][i] = (tk[t] >= 0 && j0 + i < r) ? (WT<W>::kScaled ? vj[t][i] * row_sc<W>(lsc, i) : vj[t][i]) : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (j0 + i < r) {
        float bv[8];
        raw_cvt(braw[i], bv);
#pragma unroll
        for (int t = 0; t < TG; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(vj[t][i], bv[e], acc[t][e]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (cin && tk[t] >= 0) {
      float yv[8];
      raw_cvt(yraw[t], yv);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] += acc[t][e];
      store8(y + (int64_t)tk[t] * w.d_out + col, yv);
    }
  }
}

// Gather expand of tokens toks[0..cnt) over column block cb: groups of up to
// 4 tokens, the last of 1 to 4.  LAST: a one-token item reads its B block
// non-temporally (a one-token segment, or the last item of a segment in the
// heaviest-first plan order: no later item reads that block; the hint on the
// last items of longer segments measured no gain).
template <typename T, typename W, int NT, bool LAST = false>
__device__ __forceinline__ void expand_gemv(const DevW &w, int a, int r, int cb, const int *toks, int cnt,
                            int num_tokens, const float *__restrict__ v, T *__restrict__ y) {
  int g0 = 0;
  for (; g0 + 4 <= cnt; g0 += 4) expand_cols_tile<T, W, 4, NT>(w, a, r, cb, toks, g0, 4, num_tokens, v, y);
  const int rest = cnt - g0;
  if (rest == 1) expand_cols_tile<T, W, 1, NT, LAST>(w, a, r, cb, toks, g0, 1, num_tokens, v, y);
  else if (rest == 2) expand_cols_tile<T, W, 2, NT>(w, a, r, cb, toks, g0, 2, num_tokens, v, y);
  else if (rest == 3) expand_cols_tile<T, W, 4, NT>(w, a, r, cb, toks, g0, 3, num_tokens, v, y);
}

// Column of the wave's 64-column slab that MFMA row `rho` of sub-tile `t`
// stands for.  Chosen so that after the MFMA, lane (g, m) holds 8 consecutive
// columns 32q + 8g .. +7 of token m in sub-tiles 2q and 2q+1: one 16-byte y
// access per lane instead of four 4-byte ones.
__device__ __forceinline__ int slab_col(int t, int rho) {
  return 32 * (t >> 1) + 8 * (rho >> 2) + 4 * (t & 1) + (rho & 3);
}

// v[tok][jb .. jb+7] as 8 floats (zero past nj or for no token).
__device__ __forceinline__ void load_v8(const float *vr, int jb, int nj, bool vec, float (&o)[8]) {
  if (vr && vec && jb + 8 <= nj) {
    const float4 p = *reinterpret_cast<const float4 *>(vr + jb);
    const float4 q = *reinterpret_cast<const float4 *>(vr + jb + 4);
    o[0] = p.x; o[1] = p.y; o[2] = p.z; o[3] = p.w; o[4] = q.x; o[5] = q.y; o[6] = q.z; o[7] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (vr && jb + e < nj) ? vr[jb + e] : 0.f;
  }
}

// Stages rows jc .. jc + 8 NR of this wave's 64-column B^T slab into LDS,
// transposed ([column][j]); lane l takes the row pairs 2p, 2p + 1 with
// p = (l >> 3) + 8 i, columns 8 (l & 7) .. +7, and writes each column's two
// rank indices as one 4-byte (bf16) or 8-byte (fp32) LDS word.  Rows past nj
// (the rank) and columns past d_out are zero.  The row addresses come from
// one batch of page lookups and the NR loads are issued unconditionally (safe
// address, zero-selected) before the first store.  slab_issue issues the
// loads, slab_store writes them, so other loads can be issued in between.
template <typename T, typename W, int NR>
__device__ __forceinline__ void slab_issue(const DevW &w, int a, int jc, int nj, int c0, int lane,
                                           Raw8<W> (&braw)[NR], int (&stored)[NR]) {
  static_assert(NR % 2 == 0, "row pairs");
  const int cc = (lane & 7) * 8;
  int jrow[NR];
  bool use[NR];
  const char *rp[NR];
#pragma unroll
  for (int it = 0; it < NR; ++it) {
    const int jr = 2 * ((lane >> 3) + 8 * (it >> 1)) + (it & 1);
    jrow[it] = jc + jr;
    use[it] = jr < nj && c0 + cc < w.d_out;
  }
  rows_addr<NR>(w, side_b(w), a, jrow, use, wofs<W>(c0 + cc), w.b_pages, rp, stored);
#pragma unroll
  for (int it = 0; it < NR; ++it) wload(braw[it], rp[it]);
}

template <typename T, typename W, int NR>
__device__ __forceinline__ void slab_store(const Raw8<W> (&braw)[NR], const int (&stored)[NR], T *bt,
                                           int lane) {
  constexpr int RS = ExpandCfg<T>::kRowStride;
  static_assert(RS % 2 == 0, "pair words stay aligned");
  const int cc = (lane & 7) * 8;
#pragma unroll
  for (int ip = 0; ip < NR / 2; ++ip) {
    const int jr = 2 * ((lane >> 3) + 8 * ip);
    Raw8<W> b0 = braw[2 * ip], b1 = braw[2 * ip + 1];
    if (stored[2 * ip] < 0) raw_zero(b0);
    if (stored[2 * ip + 1] < 0) raw_zero(b1);
    if constexpr (sizeof(T) == 2) {
      // bf16 bits of the two rows; column e's pair is (row 2p: element e, row
      // 2p + 1: element e) = the low or high halves of word e / 2 of each
      const uint4 u0 = raw_bf16(b0), u1 = raw_bf16(b1);
      const uint32_t w0[4] = {u0.x, u0.y, u0.z, u0.w}, w1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pair = (e & 1) ? __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], 0x07060302u)
                                      : __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], 0x05040100u);
        *reinterpret_cast<uint32_t *>(bt + (cc + e) * RS + jr) = pair;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<float2 *>(bt + (cc + e) * RS + jr) =
            make_float2(w_as_t<T, W>(b0, e), w_as_t<T, W>(b1, e));
    }
  }
}

template <typename T, typename W, int NR>
__device__ __forceinline__ void stage_slab(const DevW &w, int a, int jc, int nj, int c0, T *bt, int lane) {
  Raw8<W> braw[NR];
  int stored[NR];
  slab_issue<T, W, NR>(w, a, jc, nj, c0, lane, braw, stored);
  slab_store<T, W, NR>(braw, stored, bt, lane);
}

// Line-complete y access of a wave's 64-column slab (bf16): for token tile tt
// (16 tokens) and half h, lane l covers token 16 tt + 8 h + (l >> 3) of the
// pass and columns c0 + 8 (l & 7) .. +7, so eight lanes share each 128-byte
// line and a wave instruction touches eight whole lines.  (The MFMA layout,
// lane (g, m) = token m, 64 bytes of each of 16 rows per instruction, reads
// and writes half lines and runs at a fraction of the bandwidth.)  The MFMA
// results reach this layout through the wave's own LDS slab region.
// Token of lane l in half h of token tile tt of the pass at m0 (-1 if none).
__device__ __forceinline__ int yline_token(const int *toks, int m0, int cnt, int num_tokens, int tt, int h) {
  const int i = m0 + tt * 16 + 8 * h + ((threadIdx.x & 63) >> 3);
  const int t = i < cnt ? toks[i] : -1;
  return (t >= 0 && t < num_tokens) ? t : -1;
}
__device__ __forceinline__ void yline_load(const uint16_t *y, int d_out, int c0, const int *toks, int m0,
                                           int cnt, int num_tokens, Raw8<uint16_t> (&yraw)[4][2]) {
  const int col = c0 + 8 * (threadIdx.x & 7);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = yline_token(toks, m0, cnt, num_tokens, tt, h);
      raw_load(yraw[tt][h], y + (int64_t)(t >= 0 ? t : 0) * d_out + (col < d_out ? col : 0));
    }
}
// y += the MFMA results of token tile tt (acc[t]: lane (g, m) holds columns
// 32q + 8g .. +7 of token m in sub-tiles 2q, 2q + 1), one rounding, stored
// line-complete.  tr: the wave's LDS region (16 x 68 floats), free for the
// wave's own use (no other wave reads it).
__device__ __forceinline__ void yline_update(float *tr, const f32x4_t (&acc)[4], const Raw8<uint16_t> (&yraw)[2],
                                             const int *toks, int m0, int cnt, int num_tokens, int tt,
                                             uint16_t *y, int d_out, int c0) {
  constexpr int kTs = 68;  // row stride (floats): conflict-free writes and reads
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    *reinterpret_cast<f32x4_t *>(&tr[m * kTs + 32 * q + 8 * g]) = acc[2 * q];
    *reinterpret_cast<f32x4_t *>(&tr[m * kTs + 32 * q + 8 * g + 4]) = acc[2 * q + 1];
  }
  __builtin_amdgcn_wave_barrier();
  const int cl = 8 * (lane & 7), col = c0 + cl;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float *src = &tr[(8 * h + (lane >> 3)) * kTs + cl];
    const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(src);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(src + 4);
    const int t = yline_token(toks, m0, cnt, num_tokens, tt, h);
    if (t >= 0 && col < d_out) {
      float yv[8];
      raw_cvt(yraw[h], yv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        yv[e] += lo[e];
        yv[4 + e] += hi[e];
      }
      store8(y + (int64_t)t * d_out + col, yv);
    }
  }
  __builtin_amdgcn_wave_barrier();  // the next tile's writes come after these reads
}
static_assert(16 * 68 * sizeof(float) <= 64 * ExpandCfg<uint16_t>::kRowStride * sizeof(uint16_t),
              "a wave's slab region holds one token tile of fp32 results");

// MFMA expand for tokens toks[0..cnt) of adapter a over the 256 columns of
// block `blk` (wave w: 64 columns), 64 tokens (four 16-token tiles) at a time.
// D[col][token] = B^T-slab^T · v^T.  The y chunks of the 64 tokens are fetched
// first; then, in one round trip, each wave loads its B^T slab (64 columns x
// up to 64 rank indices, stored transposed in LDS) and the workgroup loads the
// 64 tokens' v rows (stored in LDS); after one barrier the slab fragments of a
// 16-index K block are read once and used by all four token tiles.  bf16: v is
// split into hi + lo bf16 (about 16 significant bits of v) so each K=32 MFMA
// covers 16 rank indices;
// fp32: 16x16x4 steps.
template <typename T, typename W>
__device__ __forceinline__ void expand_mfma(const DevW &w, int a, int r, int blk, const int *toks, int cnt,
                            int num_tokens, const float *__restrict__ v, T *__restrict__ y,
                            ExpandSmem<T> &sm) {
  constexpr int RS = ExpandCfg<T>::kRowStride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int c0 = blk * LORA_EXPAND_MFMA_COLS + wave * 64;
  const bool vec_v = (w.r_max & 3) == 0;
  T *bt = sm.bt + wave * 64 * RS;
  for (int m0 = 0; m0 < cnt; m0 += 64) {
    const int ntt = min(4, (cnt - m0 + 15) >> 4);
    int tok[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int i = m0 + tt * 16 + m;
      const int t = (tt < ntt && i < cnt) ? toks[i] : -1;
      tok[tt] = (t >= 0 && t < num_tokens) ? t : -1;
    }
    // prefetch y, issued unconditionally (row 0 / column 0 stand in where
    // there is no token or column; those values are never stored): bf16 in
    // the line-complete layout, fp32 in the MFMA layout (lane (g, m) of tile
    // tt touches columns c0 + 32q + 8g .. +7)
    Raw8<T> yraw[4][2];
    if constexpr (sizeof(T) == 2) {
      yline_load(y, w.d_out, c0, toks, m0, cnt, num_tokens, yraw);
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int col = c0 + 32 * q + 8 * g;
          const int64_t row = tok[tt] >= 0 ? tok[tt] : 0;
          raw_load(yraw[tt][q], y + row * w.d_out + (col < w.d_out ? col : 0));
        }
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[tt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int jc = 0; jc < r; jc += kExpandK) {
      const int nj = min(kExpandK, r - jc);
      const int nj16 = (nj + 15) & ~15;
      const int nq = nj16 >> 2;  // float4 groups per staged v row
      __syncthreads();  // previous users of the slab and of the v rows are done
      // v rows of the 64 tokens (issued first), then this wave's B^T rows
      // jc .. jc+nj16; all loads unconditional (safe addresses, zero-selected),
      // so they are in flight together before the first LDS store
      constexpr int kVIt = 64 * (kExpandK / 4) / kThreads;  // float4 groups per thread
      float4 vq[kVIt];
#pragma unroll
      for (int it = 0; it < kVIt; ++it) {
        const int idx = tid + kThreads * it;     // (token, float4 group) pairs
        const int ti = idx / nq, q = idx - ti * nq;
        const int i = m0 + ti;
        const int t = (ti < 64 && i < cnt) ? toks[i] : -1;
        const bool ok = t >= 0 && t < num_tokens;
        const int j = jc + 4 * q;
        const float *vr = v + (int64_t)(ok ? t : 0) * w.r_max;
        if (vec_v && j + 4 <= w.r_max) {
          vq[it] = *reinterpret_cast<const float4 *>(vr + j);
        } else {
          vq[it].x = vr[min(j, w.r_max - 1)];
          vq[it].y = vr[min(j + 1, w.r_max - 1)];
          vq[it].z = vr[min(j + 2, w.r_max - 1)];
          vq[it].w = vr[min(j + 3, w.r_max - 1)];
        }
        vq[it].x = ok && j < r ? vq[it].x : 0.f;
        vq[it].y = ok && j + 1 < r ? vq[it].y : 0.f;
        vq[it].z = ok && j + 2 < r ? vq[it].z : 0.f;
        vq[it].w = ok && j + 3 < r ? vq[it].w : 0.f;
        if constexpr (WT<W>::kScaled) {  // B^T row scales fold into v
          // the four rows' page lookups in one batch, the scale loads unconditional
          int jrow[4], stored[4];
          bool use[4];
          const char *unused[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            jrow[e] = min(j + e, r - 1);
            use[e] = j + e < r;
          }
          rows_addr<4>(w, side_b(w), a, jrow, use, 0, w.b_pages, unused, stored);
          float sc[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sl = w.b_sc[stored[e] >= 0 ? stored[e] : 0];
            sc[e] = stored[e] >= 0 ? sl : 0.f;
          }
          vq[it].x *= sc[0];
          vq[it].y *= sc[1];
          vq[it].z *= sc[2];
          vq[it].w *= sc[3];
        }
      }
      switch (nj16 >> 3) {
        case 2: stage_slab<T, W, 2>(w, a, jc, nj, c0, bt, lane); break;
        case 4: stage_slab<T, W, 4>(w, a, jc, nj, c0, bt, lane); break;
        case 6: if constexpr (kExpandK >= 48) stage_slab<T, W, 6>(w, a, jc, nj, c0, bt, lane); break;
        default: if constexpr (kExpandK >= 64) stage_slab<T, W, 8>(w, a, jc, nj, c0, bt, lane); break;
      }
#pragma unroll
      for (int it = 0; it < kVIt; ++it) {
        const int idx = tid + kThreads * it;
        const int ti = idx / nq, q = idx - ti * nq;
        if (ti < 64) {
          if constexpr (sizeof(T) == 2) {
            // v = hi + lo, each a bf16: hi = RNE(v), lo = RNE(v - hi)
            const float f[4] = {vq[it].x, vq[it].y, vq[it].z, vq[it].w};
            uint32_t hb[4], lb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hb[e] = bf16_rne(f[e]);
              lb[e] = bf16_rne(f[e] - __uint_as_float(hb[e] << 16));
            }
            uint16_t *row = &sm.vhl[ti * kVhlStride + 4 * q];
            *reinterpret_cast<uint2 *>(row) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            *reinterpret_cast<uint2 *>(row + kExpandK) =
                make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
          } else {
            *reinterpret_cast<float4 *>(&sm.vs[ti * kVStride + 4 * q]) = vq[it];
          }
        }
      }
      __syncthreads();
      for (int kb = 0; kb * 16 < nj; ++kb) {
        if constexpr (sizeof(T) == 2) {
          // A operand (B^T slab, transposed): sub-tile t, row rho = m -> column slab_col(t, m),
          // rank indices kb*16 + (g&1)*8 .. +7 for both the hi (g < 2) and lo (g >= 2) halves
          const int jb = kb * 16 + (g & 1) * 8;
          bf16x8_t aop[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            aop[t] = __builtin_bit_cast(bf16x8_t,
                                        *reinterpret_cast<const uint4 *>(bt + slab_col(t, m) * RS + jb));
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (tt < ntt) {
              // lanes g < 2 take the hi parts, g >= 2 the lo parts of v[tok][jb .. jb+7]
              const bf16x8_t bop = *reinterpret_cast<const bf16x8_t *>(
                  &sm.vhl[(tt * 16 + m) * kVhlStride + (g >> 1) * kExpandK + jb]);
#pragma unroll
              for (int t = 0; t < 4; ++t)
                acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[t], bop, acc[tt][t], 0, 0, 0);
            }
          }
        } else {
          // four K=4 steps: lane group g takes rank index kb*16 + 4q + g
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = kb * 16 + 4 * q + g;
            float aop[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) aop[t] = bt[slab_col(t, m) * RS + j];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              if (tt < ntt) {
                const float bop = sm.vs[(tt * 16 + m) * kVStride + j];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[t], bop, acc[tt][t], 0, 0, 0);
              }
            }
          }
        }
      }
    }
    // y update
    if constexpr (sizeof(T) == 2) {
      float *tr = reinterpret_cast<float *>(bt);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        if (tt < ntt) yline_update(tr, acc[tt], yraw[tt], toks, m0, cnt, num_tokens, tt, y, w.d_out, c0);
    } else {
      // lane (g, m) holds columns c0 + 32q + 8g .. +7 of token tok[tt]
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int col = c0 + 32 * q + 8 * g;
          if (tt < ntt && tok[tt] >= 0 && col < w.d_out) {
            float yv[8];
            raw_cvt(yraw[tt][q], yv);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              yv[e] += acc[tt][2 * q][e];
              yv[4 + e] += acc[tt][2 * q + 1][e];
            }
            store8(y + (int64_t)tok[tt] * w.d_out + col, yv);
          }
        }
      }
    }
  }
}

// MFMA expand for ranks up to 8 NR (one staged chunk, NR = 2 or 4): the same
// arithmetic as expand_mfma, with the order of the loads changed.  The chunk's v and B^T
// loads are issued before the tokens' y chunks, so that waiting for the
// chunk (loads complete in issue order) does not wait for y: the LDS staging,
// the barrier and the MFMAs overlap y's flight.  Straight-line within a pass
// of 64 tokens, so no loop-carried state makes the compiler wait for y early.
template <typename T, typename W, int NR>
__device__ __forceinline__ void expand_mfma_one(const DevW &w, int a, int r, int blk, const int *toks,
                                                int cnt, int num_tokens, const float *__restrict__ v,
                                                T *__restrict__ y, ExpandSmem<T> &sm) {
  constexpr int RS = ExpandCfg<T>::kRowStride;
  constexpr int KQ = 2 * NR;                 // float4 groups of v per token (8 NR indices)
  constexpr int VIT = 64 * KQ / kThreads;    // float4 groups per thread
  static_assert(VIT * kThreads == 64 * KQ && 8 * NR <= kExpandK, "whole groups; fits the slab");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int c0 = blk * LORA_EXPAND_MFMA_COLS + wave * 64;
  const bool vec_v = (w.r_max & 3) == 0;
  T *bt = sm.bt + wave * 64 * RS;
  for (int m0 = 0; m0 < cnt; m0 += 64) {
    const int ntt = min(4, (cnt - m0 + 15) >> 4);
    // ---- this thread's v groups: (token ti of the pass, indices 4q .. 4q+3)
    float4 vq[VIT];
    float sc[VIT][4];
    bool okv[VIT];
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + kThreads * it;
      const int ti = idx / KQ, q = idx % KQ, j = 4 * q;
      const int iv = m0 + ti;
      const int tl = toks[min(iv, cnt - 1)];
      const int tv = iv < cnt ? tl : -1;
      okv[it] = tv >= 0 && tv < num_tokens;
      const float *vr = v + (int64_t)(okv[it] ? tv : 0) * w.r_max;
      if (vec_v) {  // uniform; indices past r_max are zeroed below
        vq[it] = *reinterpret_cast<const float4 *>(vr + min(j, w.r_max - 4));
      } else {
        vq[it].x = vr[min(j, w.r_max - 1)];
        vq[it].y = vr[min(j + 1, w.r_max - 1)];
        vq[it].z = vr[min(j + 2, w.r_max - 1)];
        vq[it].w = vr[min(j + 3, w.r_max - 1)];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[it][e] = 1.f;
      if constexpr (WT<W>::kScaled) {  // B^T row scales, folded into v
        int jrow[4], stored[4];
        bool use[4];
        const char *unused[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          jrow[e] = min(j + e, r - 1);
          use[e] = j + e < r;
        }
        rows_addr<4>(w, side_b(w), a, jrow, use, 0, w.b_pages, unused, stored);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sl = w.b_sc[stored[e] >= 0 ? stored[e] : 0];
          sc[it][e] = stored[e] >= 0 ? sl : 0.f;
        }
      }
    }
    // ---- this wave's B^T slab rows 0 .. 8 NR - 1
    Raw8<W> braw[NR];
    int bstored[NR];
    slab_issue<T, W, NR>(w, a, 0, r, c0, lane, braw, bstored);
    // ---- then the y chunks (row 0 / column 0 stand in where there is no
    // token or column; those values are never stored): bf16 in the
    // line-complete layout, fp32 in the MFMA layout (lane (g, m) of tile tt
    // touches columns c0 + 32q + 8g .. +7)
    int tok[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int i = m0 + tt * 16 + m;
      const int t = (tt < ntt && i < cnt) ? toks[i] : -1;
      tok[tt] = (t >= 0 && t < num_tokens) ? t : -1;
    }
    Raw8<T> yraw[4][2];
    if constexpr (sizeof(T) == 2) {
      yline_load(y, w.d_out, c0, toks, m0, cnt, num_tokens, yraw);
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int col = c0 + 32 * qq + 8 * g;
          const int64_t row = tok[tt] >= 0 ? tok[tt] : 0;
          raw_load(yraw[tt][qq], y + row * w.d_out + (col < w.d_out ? col : 0));
        }
    }
    // ---- stage the chunk
    if (m0 > 0) __syncthreads();  // the previous pass's readers of the slab and v rows are done
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + kThreads * it;
      const int ti = idx / KQ, q = idx % KQ, j = 4 * q;
      const float f[4] = {vq[it].x, vq[it].y, vq[it].z, vq[it].w};
      float fv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) fv[e] = okv[it] && j + e < r ? f[e] * sc[it][e] : 0.f;
      if constexpr (sizeof(T) == 2) {
        // v = hi + lo, each a bf16: hi = RNE(v), lo = RNE(v - hi)
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hb[e] = bf16_rne(fv[e]);
          lb[e] = bf16_rne(fv[e] - __uint_as_float(hb[e] << 16));
        }
        uint16_t *row = &sm.vhl[ti * kVhlStride + 4 * q];
        *reinterpret_cast<uint2 *>(row) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2 *>(row + kExpandK) =
            make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
      } else {
        *reinterpret_cast<float4 *>(&sm.vs[ti * kVStride + 4 * q]) =
            make_float4(fv[0], fv[1], fv[2], fv[3]);
      }
    }
    slab_store<T, W, NR>(braw, bstored, bt, lane);
    __syncthreads();
    f32x4_t acc[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[tt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb * 16 < r; ++kb) {
      if constexpr (sizeof(T) == 2) {
        // A operand (B^T slab, transposed): sub-tile t, row rho = m -> column
        // slab_col(t, m), rank indices kb*16 + (g&1)*8 .. +7 for the hi
        // (g < 2) and lo (g >= 2) halves; B operand: v's hi or lo parts
        const int jb = kb * 16 + (g & 1) * 8;
        bf16x8_t aop[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          aop[t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(bt + slab_col(t, m) * RS + jb));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (tt < ntt) {
            const bf16x8_t bop = *reinterpret_cast<const bf16x8_t *>(
                &sm.vhl[(tt * 16 + m) * kVhlStride + (g >> 1) * kExpandK + jb]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[t], bop, acc[tt][t], 0, 0, 0);
          }
        }
      } else {
        // four K=4 steps: lane group g takes rank index kb*16 + 4q + g
#pragma unroll
        for (int qk = 0; qk < 4; ++qk) {
          const int jj = kb * 16 + 4 * qk + g;
          float aop[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) aop[t] = bt[slab_col(t, m) * RS + jj];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (tt < ntt) {
              const float bop = sm.vs[(tt * 16 + m) * kVStride + jj];
#pragma unroll
              for (int t = 0; t < 4; ++t)
                acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[t], bop, acc[tt][t], 0, 0, 0);
            }
          }
        }
      }
    }
    // ---- y update
    if constexpr (sizeof(T) == 2) {
      float *tr = reinterpret_cast<float *>(bt);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        if (tt < ntt) yline_update(tr, acc[tt], yraw[tt], toks, m0, cnt, num_tokens, tt, y, w.d_out, c0);
    } else {
      // lane (g, m) holds columns c0 + 32q + 8g .. +7 of token tok[tt]
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int col = c0 + 32 * qq + 8 * g;
          if (tt < ntt && tok[tt] >= 0 && col < w.d_out) {
            float yv[8];
            raw_cvt(yraw[tt][qq], yv);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              yv[e] += acc[tt][2 * qq][e];
              yv[4 + e] += acc[tt][2 * qq + 1][e];
            }
            store8(y + (int64_t)tok[tt] * w.d_out + col, yv);
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------- kernels
__device__ __forceinline__ bool decode_item(const lora_item &it, const DevW &w, int num_perm,
                                            int &pb, int &a, int &cnt, int &path, int &blk) {
  pb = it.perm_begin;
  a = it.adapter;
  cnt = it.count_path & 0xffff;
  path = it.count_path >> 16;
  blk = it.block;
  if (a < 0 || a >= w.num_adapters || pb < 0 || cnt <= 0 || cnt > kMaxItemTokens ||
      pb + cnt > num_perm || blk < 0) {
    LORA_CHECK(false, LORA_DEBUG_BAD_ITEM);
    return false;
  }
  return true;
}

template <typename T, typename W, int NT>
__global__ __launch_bounds__(NT) void sgmv_shrink_kernel(DevW w, const int32_t *__restrict__ perm,
                                                         int32_t num_perm,
                                                         const lora_item *__restrict__ items,
                                                         int32_t num_tokens,
                                                         const T *__restrict__ x,
                                                         float *__restrict__ v) {
  constexpr int NW = NT / 64;
  __shared__ ShrinkSmem<NW> sm;
  const lora_item it = items[blockIdx.x];
  int pb, a, cnt, path, blk;
  if (!decode_item(it, w, num_perm, pb, a, cnt, path, blk)) return;
  const int r = used_rank(w, a);
  if (path != LORA_PATH_MFMA && blk >= (r + kRowGroup - 1) / kRowGroup) return;
  const int j0 = path == LORA_PATH_MFMA ? 0 : blk * kRowGroup;
  for (int i = threadIdx.x; i < cnt; i += NT) {
    sm.toks[i] = perm[pb + i];
    LORA_CHECK((unsigned)sm.toks[i] < (unsigned)num_tokens, LORA_DEBUG_BAD_TOKEN);
  }
  __syncthreads();
  if (path == LORA_PATH_MFMA)
    shrink_mfma<T, W, NW>(w, a, r, sm.toks, cnt, num_tokens, x, v, sm);
  else
    shrink_gemv<T, W, kRowGroup, NW, true>(w, a, j0, min(kRowGroup, r - j0), sm.toks, cnt, num_tokens, x, v, sm);
}

// ----------------------------------------------------------------- tiled shrink
// Segmented shrink for bf16 activations (bf16, FP8 or INT4 rows) in 64-token
// tiles: an item is up to 64 tokens of one segment and one slice [kb, ke) of
// d_in.  Its four waves own one 16-token tile each; the tokens' x rows and the
// adapter's A rows (up to MAXR) stream through LDS in stages of 64 elements
// (an x row's stage is 128 bytes, one cache line; an A row's 128, 64 or 32
// bytes), loaded by global_load_lds_dwordx4 (lane l of a wave's load lands at
// the load's LDS base + 16 l: eight lanes per x row, each wave load covers
// eight whole lines), so no registers stage them.  Stages
// rotate through kTileStages buffers with up to kTileStages - 1 of them in
// flight; each wave waits only for its own loads of the stage it is about to
// use, then one barrier makes every wave's share visible.  A rows are read
// from HBM once per item and shared by the four waves; x rows once.  The
// chunks of a row are permuted by an XOR of the row index (LDS slot
// c ^ (row & 7)), so that the eight lanes of an LDS read phase hit eight bank
// groups (A rows of FP8 or INT4 codes: c ^ (row & 3) or c ^ (row & 1) over
// their four or two chunks).  Rows past the rank and tokens past the item
// load a row that is loaded anyway (the last valid one); their products are
// never stored.
constexpr int kTileTokens = LORA_SHRINK_TILE_TOKENS;
constexpr int kTileK = LORA_SHRINK_TILE_K;
#ifndef LORA_TILE_STAGES
#define LORA_TILE_STAGES 4
#endif
constexpr int kTileStages = LORA_TILE_STAGES;
static_assert(kTileTokens == 64 && kTileK == 64, "four 16-token tiles; eight 16-byte chunks per row");
static_assert(kTileStages >= 2 && kTileStages <= 4, "two to four stage buffers");

__device__ __forceinline__ int tile_slot(int row, int c) { return c ^ (row & 7); }

// s_waitcnt: at most N vector-memory operations of this wave outstanding,
// the other counters not waited for (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vm_n(int n) {  // n wave-uniform, 0..8
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    default: wait_vm<8>(); break;
  }
}

// Workgroup barrier without a global-memory fence: __syncthreads() would first
// wait for every outstanding global load (the later stages too).  Each wave
// has already waited for its own loads of the stage the barrier publishes
// (their LDS writes are complete when the wave's vmcnt drops); the barrier
// waits for the wave's own LDS reads (lgkmcnt), so no wave can start loading
// into a buffer another wave is still reading, and the "memory" clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct alignas(16) TileSmem {
  int toks[kTileTokens];
  float red_gemv[4 * 64];  // gather items of the same launch
};

typedef __attribute__((address_space(3))) void lds_void;
// Cache-policy operand of the tile loads (2 = non-temporal): the x rows of a
// tile item are read by that item alone; the A rows are read again by the
// segment's other token tiles.
constexpr int kTileAPolicy = 0;
constexpr int kTileXPolicy = 2;

// v rows of the tokens toks[0..cnt) (token_perm entries) of a chunk = the sum of their k_splits
// partials part[slice][pb + i][j], added in slice order.  A thread takes four
// consecutive outputs of one token (a 16-byte load per slice when r_max and r
// are multiples of 4) and issues the loads of eight slices before adding them.
__device__ __forceinline__ void tile_sum_slices(const DevW &w, int r, int cnt, int pb, int k_splits, int num_perm,
                                                int num_tokens, const int *toks, const float *__restrict__ part,
                                                float *__restrict__ v) {
  const int q4 = (r + 3) >> 2;
  const int64_t stride = (int64_t)num_perm * w.r_max;
  const bool vec = (w.r_max & 3) == 0 && (r & 3) == 0;
  for (int e = (int)threadIdx.x; e < cnt * q4; e += kThreads) {
    const int i = e / q4, j = (e - i * q4) * 4;
    const int t = toks[i];
    const float *pp = part + (int64_t)(pb + i) * w.r_max + j;
    auto load4 = [&](int s) {
      const float *q = pp + s * stride;
      if (vec) return *reinterpret_cast<const f32x4_t *>(q);
      f32x4_t o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = j + c < r ? q[c] : 0.f;
      return o;
    };
    f32x4_t sum = load4(0);
    int s = 1;
    for (; s + 8 <= k_splits; s += 8) {
      f32x4_t q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = load4(s + u);
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += q[u];
    }
    for (; s < k_splits; ++s) sum += load4(s);
    if (t >= 0 && t < num_tokens) {
      float *dst = v + (int64_t)t * w.r_max + j;
      if (vec) {
        *reinterpret_cast<f32x4_t *>(dst) = sum;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (j + c < r) dst[c] = sum[c];
      }
    }
  }
}

// One tile item with RT row tiles (r <= 16 RT <= MAXR).  Buffers: x0..x3
// (64 x 64 bf16 each) and a0..a3 (MAXR x 64), separate LDS variables so the
// compiler tells them apart.
// Stage geometry of the A rows for row type W: a stage row is kTileK
// elements, kArb bytes (128 for bf16, 64 for FP8, 32 for INT4); a wave load
// covers kArpi rows of kAlpr 16-byte chunks each.
template <typename W>
struct TileA {
  static constexpr int kArb = kTileK * WT<W>::kChunk / 8;
  static constexpr int kAlpr = kArb / 16;
  static constexpr int kArpi = 64 / kAlpr;
  // LDS slot of chunk c of row `row` (an involution, as tile_slot)
  __device__ static __forceinline__ int slot(int row, int c) { return c ^ (row & (kAlpr - 1)); }
  // the MFMA A fragment of k-step ks for lane group g: 8 elements as bf16
  __device__ static __forceinline__ bf16x8_t frag(const uint16_t *ba, int row, int ks, int g) {
    const char *rb = reinterpret_cast<const char *>(ba) + row * kArb;
    if constexpr (WT<W>::kChunk == 16) {
      return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(rb + slot(row, 4 * ks + g) * 16));
    } else if constexpr (WT<W>::kChunk == 8) {
      Raw8<W> q;
      q.u = *reinterpret_cast<const uint2 *>(rb + slot(row, 2 * ks + (g >> 1)) * 16 + (g & 1) * 8);
      return __builtin_bit_cast(bf16x8_t, raw_bf16(q));
    } else {
      Raw8<W> q;
      q.u = *reinterpret_cast<const uint32_t *>(rb + slot(row, ks) * 16 + g * 4);
      return __builtin_bit_cast(bf16x8_t, raw_bf16(q));
    }
  }
};

template <typename W, int RT, int MAXR>
__device__ __forceinline__ void tile_item(const DevW &w, int a, int r, int cnt, int kb, int ke, int pb,
                                          int slice, int k_splits, int num_perm, int num_tokens,
                                          const int *toks, const uint16_t *__restrict__ x,
                                          float *__restrict__ v, float *__restrict__ part, uint16_t *x0,
                                          uint16_t *x1, uint16_t *x2, uint16_t *x3, uint16_t *a0, uint16_t *a1,
                                          uint16_t *a2, uint16_t *a3) {
  static_assert(RT >= 1 && 16 * RT <= MAXR, "row tiles");
  using TA = TileA<W>;
  constexpr int NS = kTileStages;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane >> 3, lc = lane & 7;  // x: row of a wave load, LDS slot
  const bool xact = 16 * wave < cnt;        // this wave's token tile has tokens
  // x rows of this wave's two loads per stage: token rows 16 wave + 8 i + lr
  const char *xp[2];
  int xrow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * wave + 8 * i + lr;
    const int t = toks[row < cnt ? row : cnt - 1];
    const bool ok = t >= 0 && t < num_tokens;
    xrow[i] = row;
    xp[i] = reinterpret_cast<const char *>(x + (ok ? (int64_t)t * w.d_in : 0));
  }
  // A loads: NA per stage (kArpi rows each); wave takes loads wave, wave + 4
  constexpr int NA = (16 * RT + TA::kArpi - 1) / TA::kArpi;
  const int na = (NA > wave ? 1 : 0) + (NA > wave + 4 ? 1 : 0);
  const int alr = lane / TA::kAlpr, alc = lane % TA::kAlpr;
  const char *ap[2];
  int arow[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = TA::kArpi * (wave + 4 * u) + alr;
    const int rr = row < r ? row : r - 1;
    const char *p = (wave + 4 * u < NA) ? a_row(w, a, rr) : nullptr;
    arow[u] = row;
    ap[u] = p ? p : reinterpret_cast<const char *>(x);
  }
  const int nw = (xact ? 2 : 0) + na;  // this wave's loads per stage
  const int nst = (ke - kb) / kTileK;

  auto issue = [&](auto bc, int s) {
    constexpr int B = decltype(bc)::value;
    uint16_t *bx = B == 0 ? x0 : B == 1 ? x1 : B == 2 ? x2 : x3;
    uint16_t *ba = B == 0 ? a0 : B == 1 ? a1 : B == 2 ? a2 : a3;
    const int k = kb + s * kTileK;
    if (xact) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(xp[i] + (int64_t)(k + tile_slot(xrow[i], lc) * 8) * 2,
                                         (lds_void *)(bx + (16 * wave + 8 * i) * kTileK), 16, 0,
                                         kTileXPolicy);
    }
    const int64_t kbytes = (int64_t)k * WT<W>::kChunk / 8;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (u < na)
        __builtin_amdgcn_global_load_lds(ap[u] + kbytes + TA::slot(arow[u], alc) * 16,
                                         (lds_void *)(reinterpret_cast<char *>(ba) +
                                                      TA::kArpi * (wave + 4 * u) * TA::kArb),
                                         16, 0, kTileAPolicy);
  };

  f32x4_t acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int m = lane & 15, g = lane >> 4;

  auto step = [&](auto bc, int t) {
    constexpr int B = decltype(bc)::value;
    const uint16_t *bx = B == 0 ? x0 : B == 1 ? x1 : B == 2 ? x2 : x3;
    const uint16_t *ba = B == 0 ? a0 : B == 1 ? a1 : B == 2 ? a2 : a3;
    // this wave's loads of stage t have landed once no more than those of the
    // later issued stages are outstanding
    const int later = min(NS - 2, nst - 1 - t);
    wait_vm_n(later * nw);
    lds_barrier();  // every wave's share of stage t; buffer (t - 1) % NS free
    if (t + NS - 1 < nst) issue(std::integral_constant<int, (B + NS - 1) % NS>{}, t + NS - 1);
    if (xact) {
#pragma unroll
      for (int ks = 0; ks < kTileK / 32; ++ks) {
        const int ch = 4 * ks + g;
        const int xr = 16 * wave + m;
        const bf16x8_t xf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4 *>(bx + xr * kTileK + tile_slot(xr, ch) * 8));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8_t af = TA::frag(ba, 16 * rt + m, ks, g);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xf, acc[rt], 0, 0, 0);
        }
      }
    }
  };

  issue(std::integral_constant<int, 0>{}, 0);
  if (NS > 2 && 1 < nst) issue(std::integral_constant<int, 1 % NS>{}, 1);
  if (NS > 3 && 2 < nst) issue(std::integral_constant<int, 2 % NS>{}, 2);
  for (int t0 = 0; t0 < nst; t0 += NS) {
    step(std::integral_constant<int, 0>{}, t0);
    if (t0 + 1 < nst) step(std::integral_constant<int, 1 % NS>{}, t0 + 1);
    if (NS > 2 && t0 + 2 < nst) step(std::integral_constant<int, 2 % NS>{}, t0 + 2);
    if (NS > 3 && t0 + 3 < nst) step(std::integral_constant<int, 3 % NS>{}, t0 + 3);
  }
  __syncthreads();  // the next item of this workgroup (none) or the exit: no buffer reuse after this
  // lane (g, m) of row tile rt holds D[4g + e][m]: row 16 rt + 4g + e of token 16 wave + m;
  // quantized rows: each slice's partial times the row's scale (the scale
  // factors out of the row sum)
  const int i = 16 * wave + m;
  if (xact && i < cnt) {
    const int t = toks[i];
    if (t >= 0 && t < num_tokens) {
      float *dst = k_splits == 1 ? v + (int64_t)t * w.r_max
                                 : part + ((int64_t)slice * num_perm + pb + i) * w.r_max;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * rt + 4 * g + e;
          if (j < r) dst[j] = WT<W>::kScaled ? acc[rt][e] * a_scale<W>(w, a, j) : acc[rt][e];
        }
    }
  }
}

// Launch 1 of the tiled shrink: tile items (block = slice) and the gather
// items of the short segments (block = row group).  W: the row type (bf16,
// FP8 E4M3 or INT4; activations bf16).
template <typename W, int MAXR>
__global__ __launch_bounds__(kThreads) void sgmv_shrink_tiled_kernel(
    DevW w, const int32_t *__restrict__ perm, int32_t num_perm, const lora_item *__restrict__ items,
    int32_t num_tokens, int32_t k_splits, int32_t k_slice, const uint16_t *__restrict__ x,
    float *__restrict__ v, float *__restrict__ part) {
  // uint16_t elements of an A stage buffer: whole wave loads of kArpi rows
  // (one INT4 load covers 32 rows, more than MAXR = 16)
  constexpr int kArows = (MAXR + TileA<W>::kArpi - 1) / TileA<W>::kArpi * TileA<W>::kArpi;
  constexpr int kAe = kArows * TileA<W>::kArb / 2;
  __shared__ __attribute__((aligned(16))) uint16_t x0[kTileTokens * kTileK], x1[kTileTokens * kTileK];
  __shared__ __attribute__((aligned(16))) uint16_t x2[kTileStages > 2 ? kTileTokens * kTileK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t x3[kTileStages > 3 ? kTileTokens * kTileK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t a0[kAe], a1[kAe];
  __shared__ __attribute__((aligned(16))) uint16_t a2[kTileStages > 2 ? kAe : 8];
  __shared__ __attribute__((aligned(16))) uint16_t a3[kTileStages > 3 ? kAe : 8];
  __shared__ TileSmem sm;
  const lora_item it = items[blockIdx.x];
  int pb, a, cnt, path, blk;
  if (!decode_item(it, w, num_perm, pb, a, cnt, path, blk)) return;
  if (cnt > kTileTokens) {
    LORA_CHECK(false, LORA_DEBUG_BAD_ITEM);
    return;
  }
  const int r = used_rank(w, a);
  if (r == 0) return;
  if (path == LORA_PATH_TILE) {
    if (blk >= k_splits || r > MAXR) {
      LORA_CHECK(false, LORA_DEBUG_BAD_ITEM);
      return;
    }
  } else if (blk >= (r + kRowGroup - 1) / kRowGroup) {
    return;
  }
  for (int i = threadIdx.x; i < cnt; i += kThreads) {
    sm.toks[i] = perm[pb + i];
    LORA_CHECK((unsigned)sm.toks[i] < (unsigned)num_tokens, LORA_DEBUG_BAD_TOKEN);
  }
  __syncthreads();
  if (path == LORA_PATH_TILE) {
    const int kb = blk * k_slice, ke = min(w.d_in, kb + k_slice);
    if (kb >= ke) return;
    const int nrt = (r + 15) >> 4;
#define LORA_TILE_CASE(RT)                                                                                \
  tile_item<W, RT, MAXR>(w, a, r, cnt, kb, ke, pb, blk, k_splits, num_perm, num_tokens, sm.toks, x, v, part, \
                         x0, x1, x2, x3, a0, a1, a2, a3)
    if (nrt == 1) LORA_TILE_CASE(1);
    else if constexpr (MAXR >= 32) {
      if (nrt == 2) LORA_TILE_CASE(2);
      else if constexpr (MAXR >= 64) {
        if (nrt == 3) LORA_TILE_CASE(3);
        else LORA_TILE_CASE(4);
      }
    }
#undef LORA_TILE_CASE
  } else {
    const int j0 = blk * kRowGroup;
    shrink_gemv<uint16_t, W, kRowGroup, kThreads / 64, true>(w, a, j0, min(kRowGroup, r - j0), sm.toks, cnt,
                                                        num_tokens, x, v, sm);
  }
}

// Launch 2 of the tiled shrink (k_splits > 1): v = the sum of each token's
// k_splits partials, added in slice order.  The workgroup of slice s of a
// tile item takes the s-th of k_splits even shares of the item's tokens' rows
// (so every workgroup of the launch has work).  (Adding the slices in the
// last tile item of a chunk to finish, counted with an atomic, was measured
// 3-6x slower: each arrival needs a device-scope release, which writes back
// the L2.)
__global__ __launch_bounds__(kThreads) void sgmv_shrink_tiled_reduce_kernel(
    DevW w, const int32_t *__restrict__ perm, int32_t num_perm, const lora_item *__restrict__ items,
    int32_t num_tokens, int32_t k_splits, const float *__restrict__ part, float *__restrict__ v) {
  const lora_item it = items[blockIdx.x];
  int pb, a, cnt, path, blk;
  if (!decode_item(it, w, num_perm, pb, a, cnt, path, blk)) return;
  if (path != LORA_PATH_TILE || blk >= k_splits || cnt > kTileTokens) return;
  const int r = adapter_rank(w, a);
  const int i0 = (int)((int64_t)cnt * blk / k_splits), i1 = (int)((int64_t)cnt * (blk + 1) / k_splits);
  if (i0 >= i1 || r == 0) return;
  // token ids straight from token_perm: their loads go out with the partials'
  tile_sum_slices(w, r, i1 - i0, pb + i0, k_splits, num_perm, num_tokens, perm + pb + i0, part, v);
}

template <typename T, typename W>
// bf16 activations: registers bounded so that three waves share a SIMD (three
// workgroups per CU; the staged rank chunk keeps LDS within that too).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1)))
void sgmv_expand_kernel(DevW w, const int32_t *__restrict__ perm,
                                                               int32_t num_perm,
                                                               const lora_item *__restrict__ items,
                                                               int32_t num_tokens,
                                                               const float *__restrict__ v,
                                                               T *__restrict__ y) {
  __shared__ ExpandSmem<T> sm;
  const lora_item it = items[blockIdx.x];
  int pb, a, cnt, path, blk;
  if (!decode_item(it, w, num_perm, pb, a, cnt, path, blk)) return;
  const int cols = path == LORA_PATH_MFMA ? LORA_EXPAND_MFMA_COLS : kGatherCols;
  if ((int64_t)blk * cols >= w.d_out) return;
  for (int i = threadIdx.x; i < cnt; i += kThreads) {
    sm.toks[i] = perm[pb + i];
    LORA_CHECK((unsigned)sm.toks[i] < (unsigned)num_tokens, LORA_DEBUG_BAD_TOKEN);
  }
  __syncthreads();
  const int r = used_rank(w, a);
  if (path == LORA_PATH_MFMA) {
    // one-chunk ranks take the early-load path (up to 32 for unscaled rows;
    // quantized rows' scale registers would spill there past 16)
    constexpr int kOne = WT<W>::kScaled ? 16 : kExpandK;
    if (r <= 16) expand_mfma_one<T, W, 2>(w, a, r, blk, sm.toks, cnt, num_tokens, v, y, sm);
    else if (r <= kOne) expand_mfma_one<T, W, kOne / 8>(w, a, r, blk, sm.toks, cnt, num_tokens, v, y, sm);
    else expand_mfma<T, W>(w, a, r, blk, sm.toks, cnt, num_tokens, v, y, sm);
  }
  else
    expand_gemv<T, W, kThreads, true>(w, a, r, blk, sm.toks, cnt, num_tokens, v, y);
}

// Workgroup b of a launch runs on XCD b % 8 (the dispatcher deals workgroups to
// the eight XCDs in turn).  With the grid padded to a multiple of 8, logical
// index (b % 8) * (grid / 8) + b / 8 hands each XCD a contiguous run of logical
// indices, so neighbouring work units -- the row groups of one adapter, which
// read the same x rows -- share that XCD's L2.
__device__ __forceinline__ int xcd_logical(int b, int grid) { return (b & 7) * (grid >> 3) + (b >> 3); }

inline int pad8(int n) { return (n + 7) & ~7; }

// Collects, in token order, the tokens of ids[c0 .. c0+CH) whose adapter is
// `a` into toks[] (room for CH entries); returns their count.  All NT threads
// must call it; threads CH.. take no token.
template <int NT, int CH = NT>
__device__ __forceinline__ int gather_adapter_tokens(const int32_t *__restrict__ ids, int num_tokens, int c0, int a,
                                     int *toks, int *wave_cnt, int num_adapters) {
  static_assert(CH <= NT, "one token per thread");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = c0 + tid;
  const int id = ids[t < num_tokens ? t : num_tokens - 1];  // unconditional load
  LORA_CHECK(a != 0 || t >= num_tokens || id == LORA_NO_ADAPTER || (id >= 0 && id < num_adapters),
             LORA_DEBUG_BAD_ADAPTER);
  const bool hit = tid < CH && t < num_tokens && id == a;
  const unsigned long long mask = __ballot(hit);
  if (lane == 0) wave_cnt[wave] = __popcll(mask);
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    base += i < wave ? wave_cnt[i] : 0;
    total += wave_cnt[i];
  }
  if (hit) toks[base + __popcll(mask & ((1ull << lane) - 1ull))] = t;
  __syncthreads();
  return total;
}

// Per-token (BGMV) shrink.  Work unit u is a token (token-major) or an adapter
// (adapter-major); each unit is split into groups of RB rows, one per workgroup
// of kThreads threads.  (The segmented shrink runs wider workgroups; a token's
// v then agrees between the two paths to rounding, not bit for bit, since the
// k split and the wave reduction depend on the number of waves.)
template <typename T, typename W, int RB>
__global__ __launch_bounds__(kThreads) void bgmv_shrink_kernel(DevW w, const int32_t *__restrict__ ids,
                                                               int32_t num_tokens, int32_t adapter_major,
                                                               int32_t units, int32_t groups,
                                                               const T *__restrict__ x,
                                                               float *__restrict__ v) {
  constexpr int NW = kThreads / 64;
  __shared__ ShrinkSmem<NW> sm;
  __shared__ int wave_cnt[NW];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  if (L >= units * groups) return;
  const int u = L / groups, j0 = (L - u * groups) * RB;
  if (!adapter_major) {
    const int t = u;
    const int a = ids[t];
    check_id(w, a);
    if (a < 0 || a >= w.num_adapters) return;
    const int r = used_rank(w, a);
    if (j0 >= r) return;
    if (threadIdx.x == 0) sm.toks[0] = t;
    __syncthreads();
    shrink_gemv<T, W, RB, NW, false>(w, a, j0, min(RB, r - j0), sm.toks, 1, num_tokens, x, v, sm);
  } else {
    const int a = u;
    const int r = adapter_rank(w, a);
    if (j0 >= r) return;
    constexpr int CH = kThreads < kMaxItemTokens ? kThreads : kMaxItemTokens;
    for (int c0 = 0; c0 < num_tokens; c0 += CH) {
      const int n = gather_adapter_tokens<kThreads, CH>(ids, num_tokens, c0, a, sm.toks, wave_cnt,
                                                          w.num_adapters);
      if (n > 0) used_rank(w, a);
      if (n > 0) shrink_gemv<T, W, RB, NW, false>(w, a, j0, min(RB, r - j0), sm.toks, n, num_tokens, x, v, sm);
      __syncthreads();
    }
  }
}

// Per-token (BGMV) expand.  Work unit u as above, split into column blocks of
// 8 NT columns, one per workgroup of NT threads.
template <typename T, typename W, int NT>
__global__ __launch_bounds__(NT) void bgmv_expand_kernel(DevW w, const int32_t *__restrict__ ids,
                                                         int32_t num_tokens, int32_t adapter_major,
                                                         int32_t units, int32_t groups,
                                                         const float *__restrict__ v,
                                                         T *__restrict__ y) {
  __shared__ int toks[NT];
  __shared__ int wave_cnt[NT / 64];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  if (L >= units * groups) return;
  const int u = L / groups, cb = L - u * groups;
  if (!adapter_major) {
    const int t = u;
    const int a = ids[t];
    check_id(w, a);
    if (a < 0 || a >= w.num_adapters) return;
    const int tok1[1] = {t};
    expand_cols_tile<T, W, 1, NT>(w, a, used_rank(w, a), cb, tok1, 0, 1, num_tokens, v, y);
  } else {
    const int a = u;
    const int r = adapter_rank(w, a);
    for (int c0 = 0; c0 < num_tokens; c0 += NT) {
      const int n = gather_adapter_tokens<NT>(ids, num_tokens, c0, a, toks, wave_cnt, w.num_adapters);
      if (n > 0) used_rank(w, a);
      if (n > 0) expand_gemv<T, W, NT>(w, a, r, cb, toks, n, num_tokens, v, y);
      __syncthreads();
    }
  }
}

// Fused per-token (BGMV) delta: shrink and expand of one token in one
// workgroup of NT = 512 threads, for decode batches where both phases are
// small and each separate launch would pay its own start-up and round trips.
// Work unit (token t, column block cb).  The loads of the first shrink pass
// (x chunk, 16 A rows) and of the first expand pass (y chunk, 16 B^T rows) are
// all issued before any arithmetic, so the common case (r <= 16, d_in and the
// column block <= 4096) costs one round trip after the adapter id: v[t] is
// reduced over the workgroup into LDS, then each thread owns 8 columns and
// runs the whole rank sum for them.  Every thread's k chunks and the wave and
// workgroup reduction orders are fixed, so results are run-to-run identical.
constexpr int kFusedThreads = 512;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedPass = kFusedThreads * 8;  // d elements per pass of the workgroup
constexpr int kFusedMinGroups = 256;             // workgroups a launch aims for (one per CU)

struct alignas(16) FusedSmem {
  float red[kFusedWaves * 16];
  float vs[LORA_MAX_RANK];
};

// Addresses of rows j0 .. j0+15 of adapter a's A (offset k), `safe` past `r`
// or on an out-of-range page.
template <typename W, bool AL = false>
__device__ __forceinline__ void a_rows16(const DevW &w, int a, int j0, int r, int k, const char *safe,
                                         const char *(&rp)[16]) {
  float unused;
  rows16<W, false, AL>(w, side_a(w), a, j0, r, k, safe, rp, unused);
}
// As a_rows16, with the lane scale of the 16 A rows (see rows16).
template <typename W, bool AL = false>
__device__ __forceinline__ void a_rows16_sc(const DevW &w, int a, int j0, int r, int k, const char *safe,
                                            const char *(&rp)[16], float &lsc) {
  rows16<W, true, AL>(w, side_a(w), a, j0, r, k, safe, rp, lsc);
}

// Scale of row j of adapter a's A, loaded unconditionally (index 0 stands in
// when `use` is false or the page is out of range; the result is then 0).
template <typename W>
__device__ __forceinline__ float a_scale_any(const DevW &w, int a, int j, bool use) {
  const int64_t i = row_index(w, w.a_pt, w.num_pages_a, a, j);
  LORA_CHECK(!use || i >= 0, LORA_DEBUG_BAD_PAGE);
  const bool in = use && i >= 0;
  const float s = w.a_sc[in ? i : 0];
  return in ? s : 0.f;
}

// Work unit u = (entry u / nblk of the token order, column block u % nblk):
// one token's shrink and expand over columns [c_begin, c_end).  Units are
// placed XCD-aware (consecutive units on one XCD), so when the token order
// groups the tokens of an adapter (the segment order of the batch) those
// tokens run on one XCD and read the adapter's rows through its L2 once.  The prologue is arranged so that
// the whole first pass costs as few dependent round trips as possible: the x
// and y chunks need only the token and are requested before its adapter id
// arrives; the first 16 A and B^T rows need only the adapter id and are
// requested before its rank arrives (rows below min(16, r_max) exist in
// storage, in a dense stack and, through the page table, in a pool; rows at or
// past the rank are fetched but never used).  Nothing branches on the adapter
// id or the rank before these loads are consumed -- a token without a valid
// adapter takes rank 0 and safe addresses, and its first pass runs on them
// with every store suppressed -- so the compiler cannot sink the loads past
// the id or rank wait.  The A and B^T rows are read with the non-temporal
// hint: the tokens that share an adapter run together on one XCD, so their
// reads meet in its L2 while the lines are still there (12.6 -> 11.9 us on a
// 256-token decode batch).
template <typename T, typename W, bool AL>
__device__ __forceinline__ void fused_unit(const DevW &w, const int32_t *__restrict__ ids, int t, int cb,
                                           int block_cols, const T *__restrict__ x,
                                           float *__restrict__ v, T *__restrict__ y, FusedSmem &sm) {
  const int c_begin = cb * block_cols, c_end = min(w.d_out, c_begin + block_cols);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T *xr = x + (int64_t)t * w.d_in;
  T *yr = y + (int64_t)t * w.d_out;

  // ---- token-only loads: first x chunk and first y chunk
  const int kc0 = tid * 8 < w.d_in ? tid * 8 : 0;
  const int col0 = c_begin + tid * 8;
  const int colc0 = col0 < c_end ? col0 : c_begin;
  Raw8<T> x0, y0;
  raw_load(x0, xr + kc0);
  raw_load(y0, yr + colc0);

  const int a_id = ids[t];
  const bool valid = a_id >= 0 && a_id < w.num_adapters;
  check_id(w, a_id);
  const int a = valid ? a_id : 0;

  // ---- adapter-only loads: A and B^T rows 0 .. rs-1 (and their scales);
  // not for fp32 rows, whose 32 chunks would not fit in registers
  constexpr bool PF = WT<W>::kChunk <= 16;
  const int rs = valid ? min(16, w.r_max) : 0;
  const char *safe_a = reinterpret_cast<const char *>(x), *safe_b = w.b_pages;
  Raw8<W> a0[16], b0[16];
  float lsc_b0 = 1.f;
  float asc = 1.f;  // scale of A row jc + tid (threads 0..15: lane == tid)
  if constexpr (PF) {
    const char *ap0[16], *bp0[16];
    a_rows16_sc<W, AL>(w, a, 0, rs, kc0, safe_a, ap0, asc);
    b_rows16<W, AL>(w, a, 0, rs, colc0, safe_b, bp0, lsc_b0);
#pragma unroll
    for (int i = 0; i < 16; ++i) wload<true>(a0[i], ap0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) wload<true>(b0[i], bp0[i]);
  } else if constexpr (WT<W>::kScaled) {
    asc = a_scale_any<W>(w, a, tid, tid < rs);
  }

  const int r = valid ? used_rank(w, a) : 0;

  // ---- shrink: v[j] = sum_k A[j][k] x[k], 16 rows at a time (the first
  // 16 always, see above)
  // the FMAs of one k pass: acc[i] += A[i][k..k+7] . x[k..k+7]
  auto fma_pass = [&](float (&acc)[16], const Raw8<T> &xraw, const Raw8<W> (&araw)[16], bool kin) {
    if (kin) {
      float xv[8];
      raw_cvt(xraw, xv);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float av[8];
        raw_cvt(araw[i], av);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i] = fmaf(av[e], xv[e], acc[i]);
      }
    }
  };
  // one k pass of rows jc .. jc+15 from memory
  auto load_pass = [&](float (&acc)[16], int jc, int k0) {
    const int k = k0 + tid * 8;
    const bool kin = k < w.d_in;
    const int kc = kin ? k : 0;
    Raw8<T> xraw;
    Raw8<W> araw[16];
    raw_load(xraw, xr + kc);
    const char *ap[16];
    a_rows16<W, AL>(w, a, jc, r, kc, safe_a, ap);
#pragma unroll
    for (int i = 0; i < 16; ++i) wload<true>(araw[i], ap[i]);
    fma_pass(acc, xraw, araw, kin);
  };
  // reduce the 16 row sums over the workgroup: reduce-scatter in each wave,
  // then the waves in order (rows at or past the rank are never used)
  auto reduce_rows = [&](float (&acc)[16], int jc) {
    const float part = wave_reduce_scatter<16>(acc);
    if ((lane & 3) == 0) sm.red[wave * 16 + (lane >> 2)] = part;
    __syncthreads();
    if (tid < 16) {
      float sum = sm.red[tid];
#pragma unroll
      for (int wv = 1; wv < kFusedWaves; ++wv) sum += sm.red[wv * 16 + tid];
      if constexpr (WT<W>::kScaled) sum *= asc;
      sm.vs[jc + tid] = sum;
      if (v && cb == 0 && jc + tid < r) v[(int64_t)t * w.r_max + jc + tid] = sum;
    }
    __syncthreads();
  };
  {
    // rows 0..15 over the first k pass from the prologue's chunks, in
    // straight-line code: a loop here would merge the prologue's pending
    // loads with the loop's own at its header, and the compiler would then
    // wait for all of them (the B^T rows too) before the first FMA
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    Raw8<W> araw[16];
    if constexpr (PF) {
#pragma unroll
      for (int i = 0; i < 16; ++i) araw[i] = a0[i];
    } else {
      const char *ap[16];
      a_rows16<W, AL>(w, a, 0, r, kc0, safe_a, ap);
#pragma unroll
      for (int i = 0; i < 16; ++i) wload<true>(araw[i], ap[i]);
    }
    fma_pass(acc, x0, araw, tid * 8 < w.d_in);
    for (int k0 = kFusedPass; k0 < w.d_in; k0 += kFusedPass) load_pass(acc, 0, k0);
    reduce_rows(acc, 0);
  }
  for (int jc = 16; jc < r; jc += 16) {
    if constexpr (WT<W>::kScaled) asc = a_scale_any<W>(w, a, jc + tid, tid < 16 && jc + tid < r);
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < w.d_in; k0 += kFusedPass) load_pass(acc, jc, k0);
    reduce_rows(acc, jc);
  }

  // ---- expand: y[col] += sum_j B^T[j][col] v[j], 8 columns per thread
  for (int c0 = c_begin; c0 < c_end; c0 += kFusedPass) {
    const int col = c0 + tid * 8;
    const bool cin = col < c_end;
    const int colc = cin ? col : c_begin;
    Raw8<T> yraw;
    if (c0 == c_begin) yraw = y0;
    else raw_load(yraw, yr + colc);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 == 0 || j0 < r; j0 += 16) {
      Raw8<W> braw[16];
      float lsc;
      if (PF && c0 == c_begin && j0 == 0) {
        lsc = lsc_b0;
#pragma unroll
        for (int i = 0; i < 16; ++i) braw[i] = b0[i];
      } else {
        const char *bp[16];
        b_rows16<W, AL>(w, a, j0, r, colc, safe_b, bp, lsc);
#pragma unroll
        for (int i = 0; i < 16; ++i) wload<true>(braw[i], bp[i]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (j0 + i < r) {
          const float vj = WT<W>::kScaled ? sm.vs[j0 + i] * row_sc<W>(lsc, i) : sm.vs[j0 + i];
          float bv[8];
          raw_cvt(braw[i], bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(vj, bv[e], acc[e]);
        }
      }
    }
    if (cin && r > 0) {
      float yv[8];
      raw_cvt(yraw, yv);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] += acc[e];
      store8(yr + col, yv);
    }
  }
}

template <typename T, typename W, bool AL>
__global__ __launch_bounds__(kFusedThreads) void bgmv_fused_kernel(DevW w, const int32_t *__restrict__ ids,
                                                                   int32_t num_tokens,
                                                                   const int32_t *__restrict__ torder,
                                                                   int32_t units, int32_t nblk,
                                                                   int32_t block_cols,
                                                                   const T *__restrict__ x,
                                                                   float *__restrict__ v,
                                                                   T *__restrict__ y) {
  __shared__ FusedSmem sm;
  const int u = xcd_logical(blockIdx.x, gridDim.x);
  const int slot = u / nblk, cb = u - slot * nblk;
  if (slot >= units) return;
  const int t = torder ? torder[slot] : slot;
  if ((unsigned)t >= (unsigned)num_tokens) return;
  fused_unit<T, W, AL>(w, ids, t, cb, block_cols, x, v, y, sm);
}

// Several projections of the same input in one launch (the q, k and v of an
// attention layer: each with its own adapter matrices and output, all reading
// the token's x).  Work unit = (entry of the token order, projection p, column
// block of p); the units of one token are consecutive and placed on one XCD,
// so x is fetched once for all its projections.  Each unit's arithmetic is the
// single-projection kernel's, so results are bit-identical to separate
// launches.
constexpr int kMaxProj = 4;
template <typename T>
struct MultiArgs {
  DevW w[kMaxProj];
  T *y[kMaxProj];
  float *v[kMaxProj];
  int32_t block_cols[kMaxProj];
  int32_t first[kMaxProj + 1];  // units of projections 0 .. p-1 within a token
};

template <typename T, typename W, bool AL>
__global__ __launch_bounds__(kFusedThreads) void bgmv_fused_multi_kernel(MultiArgs<T> m, int32_t np,
                                                                         const int32_t *__restrict__ ids,
                                                                         int32_t num_tokens,
                                                                         const int32_t *__restrict__ torder,
                                                                         int32_t units,
                                                                         const T *__restrict__ x) {
  __shared__ FusedSmem sm;
  const int per = m.first[np];
  const int u = xcd_logical(blockIdx.x, gridDim.x);
  const int slot = u / per, k = u - slot * per;
  if (slot >= units) return;
  const int t = torder ? torder[slot] : slot;
  if ((unsigned)t >= (unsigned)num_tokens) return;
  // the unit's projection, and its arguments chosen by uniform selects with
  // constant indices (a computed index into the argument block would copy it
  // to scratch; a call per projection would inline the body four times)
  const int p = (np > 1 && k >= m.first[1]) + (np > 2 && k >= m.first[2]) + (np > 3 && k >= m.first[3]);
  DevW w;
#define LORA_SEL(f) w.f = p == 0 ? m.w[0].f : p == 1 ? m.w[1].f : p == 2 ? m.w[2].f : m.w[3].f
  LORA_SEL(a_pages); LORA_SEL(b_pages); LORA_SEL(rank); LORA_SEL(a_pt); LORA_SEL(b_pt);
  LORA_SEL(a_sc); LORA_SEL(b_sc); LORA_SEL(a_row_bytes); LORA_SEL(b_row_bytes);
  LORA_SEL(d_in); LORA_SEL(d_out); LORA_SEL(num_adapters); LORA_SEL(r_max); LORA_SEL(page_rows);
  LORA_SEL(max_pages); LORA_SEL(num_pages_a); LORA_SEL(num_pages_b);
#undef LORA_SEL
  const int first = p == 0 ? m.first[0] : p == 1 ? m.first[1] : p == 2 ? m.first[2] : m.first[3];
  const int bc = p == 0 ? m.block_cols[0] : p == 1 ? m.block_cols[1] : p == 2 ? m.block_cols[2] : m.block_cols[3];
  float *vp = p == 0 ? m.v[0] : p == 1 ? m.v[1] : p == 2 ? m.v[2] : m.v[3];
  T *yp = p == 0 ? m.y[0] : p == 1 ? m.y[1] : p == 2 ? m.y[2] : m.y[3];
  fused_unit<T, W, AL>(w, ids, t, k - first, bc, x, vp, yp, sm);
}

// Fused per-token delta, adapter-major: work unit (adapter a, column block
// cb); the workgroup finds a's tokens by scanning the device ids, computes
// their v (up to 4 tokens at a time) with the adapter's A rows held in
// registers across the tokens, reduces v into LDS, and expands its columns
// with the B^T rows likewise shared by the tokens.  Units of one adapter share
// an XCD (and so its L2), so each adapter's rows cross the fabric once however
// many tokens use them.  Each token's arithmetic (per-thread k chunks, wave
// and workgroup reduction orders, per-column rank sums) is the same as in the
// token-major fused kernel, so the two orders give identical results.
struct alignas(16) FusedAmSmem {
  int toks[kFusedThreads];
  int wave_cnt[kFusedWaves];
  float red[kFusedWaves * 64];
  float vs[4][LORA_MAX_RANK];
};

template <typename T, typename W, int TG>
__device__ __forceinline__ void fused_am_group(const DevW &w, int a, int r, int c_begin, int c_end,
                                               const int *toks, int g0, int ntok,
                                               const T *__restrict__ x, float *__restrict__ v,
                                               T *__restrict__ y, bool write_v, FusedAmSmem &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tk[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) tk[t] = t < ntok ? uniform(toks[g0 + t]) : toks[g0];
  const char *safe_a = reinterpret_cast<const char *>(x), *safe_b = w.b_pages;
  // shrink: acc[t][i] = sum over this thread's k chunks of A[jc+i][k] x_t[k]
  for (int jc = 0; jc < r; jc += 16) {
    float acc[TG * 16];
#pragma unroll
    for (int i = 0; i < TG * 16; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < w.d_in; k0 += kFusedPass) {
      const int k = k0 + tid * 8;
      const bool kin = k < w.d_in;
      const int kc = kin ? k : 0;
      const char *ap[16];
      a_rows16<W>(w, a, jc, r, kc, safe_a, ap);
      Raw8<T> xraw[TG];
      Raw8<W> araw[16];
#pragma unroll
      for (int t = 0; t < TG; ++t) raw_load(xraw[t], x + (int64_t)tk[t] * w.d_in + kc);
#pragma unroll
      for (int i = 0; i < 16; ++i) wload(araw[i], ap[i]);
      if (kin) {
        float xv[TG][8];
#pragma unroll
        for (int t = 0; t < TG; ++t) raw_cvt(xraw[t], xv[t]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float av[8];
          raw_cvt(araw[i], av);
#pragma unroll
          for (int t = 0; t < TG; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[t * 16 + i] = fmaf(av[e], xv[t][e], acc[t * 16 + i]);
        }
      }
    }
    constexpr int NV = TG * 16, SH = 6 - ilog2(NV);
    const float part = wave_reduce_scatter<NV>(acc);
    if ((lane & ((1 << SH) - 1)) == 0) sm.red[wave * 64 + (lane >> SH)] = part;
    __syncthreads();
    if (tid < NV) {
      float sum = sm.red[tid];
#pragma unroll
      for (int wv = 1; wv < kFusedWaves; ++wv) sum += sm.red[wv * 64 + tid];
      const int t = tid >> 4, i = tid & 15;
      if constexpr (WT<W>::kScaled) sum *= jc + i < r ? a_scale<W>(w, a, jc + i) : 0.f;
      sm.vs[t][jc + i] = sum;
      if (write_v && t < ntok && jc + i < r) v[(int64_t)tk[t] * w.r_max + jc + i] = sum;
    }
    __syncthreads();
  }
  // expand: thread owns 8 columns per pass; the B^T rows are loaded once per
  // pass and shared by the group's tokens
  for (int c0 = c_begin; c0 < c_end; c0 += kFusedPass) {
    const int col = c0 + tid * 8;
    const bool cin = col < c_end;
    const int colc = cin ? col : c_begin;
    Raw8<T> yraw[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) raw_load(yraw[t], y + (int64_t)tk[t] * w.d_out + colc);
    float acc[TG][8];
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
    for (int j0 = 0; j0 < r; j0 += 16) {
      const char *bp[16];
      float lsc;
      b_rows16<W>(w, a, j0, r, colc, safe_b, bp, lsc);
      Raw8<W> braw[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) wload(braw[i], bp[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (j0 + i < r) {
          float bv[8];
          raw_cvt(braw[i], bv);
#pragma unroll
          for (int t = 0; t < TG; ++t) {
            const float vj = WT<W>::kScaled ? sm.vs[t][j0 + i] * row_sc<W>(lsc, i) : sm.vs[t][j0 + i];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(vj, bv[e], acc[t][e]);
          }
        }
      }
    }
    if (cin) {
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        if (t < ntok) {
          float yv[8];
          raw_cvt(yraw[t], yv);
#pragma unroll
          for (int e = 0; e < 8; ++e) yv[e] += acc[t][e];
          store8(y + (int64_t)tk[t] * w.d_out + col, yv);
        }
      }
    }
  }
  __syncthreads();  // vs is rewritten by the next group
}

template <typename T, typename W>
__global__ __launch_bounds__(kFusedThreads) void bgmv_fused_am_kernel(DevW w, const int32_t *__restrict__ ids,
                                                                      int32_t num_tokens, int32_t nblk,
                                                                      int32_t block_cols,
                                                                      const T *__restrict__ x,
                                                                      float *__restrict__ v,
                                                                      T *__restrict__ y) {
  __shared__ FusedAmSmem sm;
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  if (L >= w.num_adapters * nblk) return;
  const int a = L / nblk, cb = L - a * nblk;
  const int r = adapter_rank(w, a);
  const int c_begin = cb * block_cols, c_end = min(w.d_out, c_begin + block_cols);
  for (int c0 = 0; c0 < num_tokens; c0 += kFusedThreads) {
    const int n = gather_adapter_tokens<kFusedThreads>(ids, num_tokens, c0, a, sm.toks, sm.wave_cnt,
                                                         w.num_adapters);
    if (n > 0) used_rank(w, a);
    int g0 = 0;
    for (; g0 + 4 <= n; g0 += 4)
      fused_am_group<T, W, 4>(w, a, r, c_begin, c_end, sm.toks, g0, 4, x, v, y, v && cb == 0, sm);
    const int rest = n - g0;
    if (rest == 1)
      fused_am_group<T, W, 1>(w, a, r, c_begin, c_end, sm.toks, g0, 1, x, v, y, v && cb == 0, sm);
    else if (rest == 2)
      fused_am_group<T, W, 2>(w, a, r, c_begin, c_end, sm.toks, g0, 2, x, v, y, v && cb == 0, sm);
    else if (rest == 3)
      fused_am_group<T, W, 4>(w, a, r, c_begin, c_end, sm.toks, g0, 3, x, v, y, v && cb == 0, sm);
    __syncthreads();
  }
}

// ----------------------------------------------------------------- validation
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Bytes of one stored adapter row of d elements.
int64_t row_bytes(int32_t dtype, int32_t wf, int32_t d) {
  if (wf == LORA_WFMT_FP8_E4M3) return d;
  if (wf == LORA_WFMT_INT4) return d / 2;
  return (int64_t)d * (dtype == LORA_BF16 ? 2 : 4);
}

// Calls f(T{}, W{}) with the activation type T and the adapter-row type W of w
// (validated by to_dev): (bf16, bf16), (fp32, fp32), (bf16, FP8 E4M3) or
// (bf16, INT4).
template <typename F>
void with_types(const lora_weights *w, F &&f) {
  if (w->dtype == LORA_F32) f(float{}, float{});
  else if (w->weight_format == LORA_WFMT_FP8_E4M3) f(uint16_t{}, Fp8{});
  else if (w->weight_format == LORA_WFMT_INT4) f(uint16_t{}, Int4{});
  else f(uint16_t{}, uint16_t{});
}

lora_status to_dev(const lora_weights *w, DevW *d) {
  if (!w) return fail(LORA_EINVAL, "null weights");
  if (w->dtype != LORA_F32 && w->dtype != LORA_BF16)
    return fail(LORA_EUNSUPPORTED, "unknown dtype %d", w->dtype);
  if (w->d_in <= 0 || w->d_out <= 0 || w->d_in % 8 || w->d_out % 8)
    return fail(LORA_EUNSUPPORTED, "d_in (%d) and d_out (%d) must be positive multiples of 8",
                w->d_in, w->d_out);
  if (w->r_max < 1 || w->r_max > LORA_MAX_RANK)
    return fail(LORA_EUNSUPPORTED, "r_max %d outside 1..%d", w->r_max, LORA_MAX_RANK);
  if (w->num_adapters < 0) return fail(LORA_EINVAL, "negative num_adapters");
  if (w->page_rows <= 0) return fail(LORA_EINVAL, "page_rows must be positive");
  if (w->num_pages_a <= 0 || w->num_pages_b <= 0) return fail(LORA_EINVAL, "empty page pool");
  // the kernels form stored-row numbers (page * page_rows + row) in 32 bits
  if ((int64_t)w->num_pages_a * w->page_rows > INT32_MAX ||
      (int64_t)w->num_pages_b * w->page_rows > INT32_MAX)
    return fail(LORA_EINVAL, "page pool of more than 2^31 - 1 stored rows (%d or %d pages of %d rows)",
                w->num_pages_a, w->num_pages_b, w->page_rows);
  const int32_t wf = w->weight_format;
  if (wf != LORA_WFMT_PLAIN && wf != LORA_WFMT_FP8_E4M3 && wf != LORA_WFMT_INT4)
    return fail(LORA_EUNSUPPORTED, "unknown weight_format %d", wf);
  if (wf != LORA_WFMT_PLAIN) {
    if (w->dtype != LORA_BF16)
      return fail(LORA_EUNSUPPORTED, "quantized adapter rows need bf16 activations");
    if (!w->a_scales || !w->b_scales) return fail(LORA_EINVAL, "quantized rows need row scales");
    if (((uintptr_t)w->a_scales & 3u) || ((uintptr_t)w->b_scales & 3u))
      return fail(LORA_EINVAL, "row scales must be 4-byte aligned");
  }
  if (!w->a_pages || !w->b_pages || !w->rank) return fail(LORA_EINVAL, "null weight pointer");
  if (!aligned16(w->a_pages) || !aligned16(w->b_pages))
    return fail(LORA_EINVAL, "page storage must be 16-byte aligned");
  if ((w->a_page_table == nullptr) != (w->b_page_table == nullptr))
    return fail(LORA_EINVAL, "give both page tables or neither");
  if (w->a_page_table) {
    if (w->max_pages < (w->r_max + w->page_rows - 1) / w->page_rows)
      return fail(LORA_EINVAL, "max_pages %d too small for r_max %d with %d-row pages",
                  w->max_pages, w->r_max, w->page_rows);
  } else {
    if (w->page_rows < w->r_max)
      return fail(LORA_EINVAL, "dense stacks need page_rows (%d) >= r_max (%d)", w->page_rows,
                  w->r_max);
    if (w->num_pages_a < w->num_adapters || w->num_pages_b < w->num_adapters)
      return fail(LORA_EINVAL, "dense stacks need one page per adapter");
  }
  if (w->host_rank)
    for (int32_t a = 0; a < w->num_adapters; ++a)
      if (w->host_rank[a] < 1 || w->host_rank[a] > w->r_max)
        return fail(LORA_ERANGE, "adapter %d has rank %d outside 1..r_max (%d)", a,
                    w->host_rank[a], w->r_max);
  d->a_pages = (const char *)w->a_pages;
  d->b_pages = (const char *)w->b_pages;
  d->a_sc = wf == LORA_WFMT_PLAIN ? nullptr : w->a_scales;
  d->b_sc = wf == LORA_WFMT_PLAIN ? nullptr : w->b_scales;
  d->a_row_bytes = row_bytes(w->dtype, wf, w->d_in);
  d->b_row_bytes = row_bytes(w->dtype, wf, w->d_out);
  d->rank = w->rank;
  d->a_pt = w->a_page_table;
  d->b_pt = w->b_page_table;
  d->d_in = w->d_in;
  d->d_out = w->d_out;
  d->num_adapters = w->num_adapters;
  d->r_max = w->r_max;
  d->page_rows = w->page_rows;
  d->max_pages = w->a_page_table ? w->max_pages : 1;
  d->num_pages_a = w->num_pages_a;
  d->num_pages_b = w->num_pages_b;
  return LORA_OK;
}

lora_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}

lora_status check_sgmv_args(const int32_t *perm, int32_t num_perm, const lora_item *items,
                            int32_t num_items, int32_t num_tokens, const void *in, const void *out) {
  if (num_perm < 0 || num_items < 0 || num_tokens < 0) return fail(LORA_EINVAL, "negative size");
  if (num_items > 0 && num_tokens > 0) {
    if (!perm || !items || !in || !out) return fail(LORA_EINVAL, "null pointer");
    if (!aligned16(in) || !aligned16(out) || !aligned16(items))
      return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  }
  return LORA_OK;
}

// Automatic order.  Shrink: adapter-major when adapters carry one to four
// tokens on average (each adapter's A rows are then read by one group of
// workgroups instead of once per token, and no workgroup serialises many
// tokens).  Expand: token-major (no scan of the ids; an adapter's B^T rows,
// shared by its tokens, come from cache).
int bgmv_order(int phase, int order, int num_tokens, int num_adapters) {
  if (order == LORA_BGMV_TOKEN_MAJOR || order == LORA_BGMV_ADAPTER_MAJOR) return order;
  if (phase == LORA_PHASE_SHRINK)
    return (num_adapters <= num_tokens && num_tokens <= 4 * num_adapters) ? LORA_BGMV_ADAPTER_MAJOR
                                                                          : LORA_BGMV_TOKEN_MAJOR;
  return LORA_BGMV_TOKEN_MAJOR;
}

}  // namespace

// ----------------------------------------------------------------- debug word
extern "C" lora_status lora_debug_flags(uint32_t *flags, int32_t clear) {
  if (!flags) return fail(LORA_EINVAL, "null flags");
  *flags = 0;
#if LORA_DEBUG
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_debug_flags), sizeof(uint32_t), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the debug word");
  if (clear) {
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "clearing the debug word");
  }
  return ok();
#else
  (void)clear;
  return fail(LORA_EUNSUPPORTED, "library built without LORA_DEBUG (load liblora_sgmv_debug.so)");
#endif
}

// ----------------------------------------------------------------- C ABI
extern "C" lora_status lora_sgmv_shrink(const lora_weights *w, const int32_t *token_perm,
                                        int32_t num_perm, const lora_item *items,
                                        int32_t num_items, int32_t num_tokens, const void *x,
                                        float *v, hipStream_t stream) {
  DevW d;
  lora_status st = to_dev(w, &d);
  if (st != LORA_OK) return st;
  if ((st = check_sgmv_args(token_perm, num_perm, items, num_items, num_tokens, x, v)) != LORA_OK)
    return st;
  if (num_items == 0 || num_tokens == 0) return ok();
  with_types(w, [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    // bf16 rows with ranks above 32: an MFMA item reads up to four 16-row
    // tiles of A per k-step against one of x, and twice the waves per item
    // keep twice the k-steps in flight (the other element types would spill
    // registers at 1024 threads)
    constexpr bool kWide = sizeof(T) == 2 && !WT<W>::kScaled;
    if (kWide && w->r_max > 32)
      hipLaunchKernelGGL((sgmv_shrink_kernel<T, W, kWide ? 2 * kSgmvShrinkThreads : kSgmvShrinkThreads>),
                         dim3(num_items), dim3(kWide ? 2 * kSgmvShrinkThreads : kSgmvShrinkThreads), 0,
                         stream, d, token_perm, num_perm, items, num_tokens, (const T *)x, v);
    else
      hipLaunchKernelGGL((sgmv_shrink_kernel<T, W, kSgmvShrinkThreads>), dim3(num_items),
                         dim3(kSgmvShrinkThreads), 0, stream, d, token_perm, num_perm, items,
                         num_tokens, (const T *)x, v);
  });
  return check_launch("sgmv shrink launch");
}

extern "C" lora_status lora_sgmv_shrink_tiled(const lora_weights *w, const int32_t *token_perm,
                                              int32_t num_perm, const lora_item *items,
                                              int32_t num_items, int32_t num_tokens, int32_t k_splits,
                                              const void *x, float *v, void *workspace,
                                              int64_t workspace_bytes, hipStream_t stream) {
  DevW d;
  lora_status st = to_dev(w, &d);
  if (st != LORA_OK) return st;
  if ((st = check_sgmv_args(token_perm, num_perm, items, num_items, num_tokens, x, v)) != LORA_OK)
    return st;
  if (w->dtype != LORA_BF16) return fail(LORA_EUNSUPPORTED, "the tiled shrink needs bf16 activations");
  if (w->r_max > 64) return fail(LORA_EUNSUPPORTED, "the tiled shrink needs r_max <= 64 (got %d)", w->r_max);
  if (w->d_in % LORA_SHRINK_TILE_K)
    return fail(LORA_EUNSUPPORTED, "the tiled shrink needs d_in a multiple of %d (got %d)", LORA_SHRINK_TILE_K,
                w->d_in);
  if (k_splits < 1 || k_splits > LORA_MAX_K_SPLITS)
    return fail(LORA_EINVAL, "k_splits %d outside 1..%d", k_splits, LORA_MAX_K_SPLITS);
  const int32_t slice = tile_slice_len(w->d_in, k_splits);
  if ((int64_t)(k_splits - 1) * slice >= w->d_in)
    return fail(LORA_EINVAL, "k_splits %d leaves an empty slice of d_in %d (a plan built for another d_in)",
                k_splits, w->d_in);
  if (workspace_bytes < 0) return fail(LORA_EINVAL, "negative workspace size");
  const int64_t need = k_splits > 1 ? (int64_t)k_splits * num_perm * w->r_max * (int64_t)sizeof(float) : 0;
  if (need > 0 && (!workspace || !aligned16(workspace)))
    return fail(LORA_EINVAL, "the tiled shrink with k_splits > 1 needs a 16-byte aligned workspace");
  if (workspace_bytes < need)
    return fail(LORA_EINVAL, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)need);
  if (num_items == 0 || num_tokens == 0) return ok();
  float *part = static_cast<float *>(workspace);
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  with_types(w, [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    if constexpr (sizeof(T) == 2) {
      if (w->r_max <= 16)
        hipLaunchKernelGGL((sgmv_shrink_tiled_kernel<W, 16>), dim3(num_items), dim3(kThreads), 0, stream, d,
                           token_perm, num_perm, items, num_tokens, k_splits, slice, xb, v, part);
      else if (w->r_max <= 32)
        hipLaunchKernelGGL((sgmv_shrink_tiled_kernel<W, 32>), dim3(num_items), dim3(kThreads), 0, stream, d,
                           token_perm, num_perm, items, num_tokens, k_splits, slice, xb, v, part);
      else
        hipLaunchKernelGGL((sgmv_shrink_tiled_kernel<W, 64>), dim3(num_items), dim3(kThreads), 0, stream, d,
                           token_perm, num_perm, items, num_tokens, k_splits, slice, xb, v, part);
    }
  });
  if (k_splits > 1)
    hipLaunchKernelGGL(sgmv_shrink_tiled_reduce_kernel, dim3(num_items), dim3(kThreads), 0, stream, d,
                       token_perm, num_perm, items, num_tokens, k_splits, (const float *)part, v);
  return check_launch("sgmv tiled shrink launch");
}

extern "C" lora_status lora_sgmv_expand(const lora_weights *w, const int32_t *token_perm,
                                        int32_t num_perm, const lora_item *items,
                                        int32_t num_items, int32_t num_tokens, const float *v,
                                        void *y, hipStream_t stream) {
  DevW d;
  lora_status st = to_dev(w, &d);
  if (st != LORA_OK) return st;
  if ((st = check_sgmv_args(token_perm, num_perm, items, num_items, num_tokens, v, y)) != LORA_OK)
    return st;
  if (num_items == 0 || num_tokens == 0) return ok();
  with_types(w, [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    hipLaunchKernelGGL((sgmv_expand_kernel<T, W>), dim3(num_items), dim3(kThreads), 0, stream, d,
                       token_perm, num_perm, items, num_tokens, v, (T *)y);
  });
  return check_launch("sgmv expand launch");
}

extern "C" lora_status lora_bgmv_shrink(const lora_weights *w, const int32_t *token_adapter,
                                        int32_t num_tokens, int32_t order, const void *x, float *v,
                                        hipStream_t stream) {
  DevW d;
  lora_status st = to_dev(w, &d);
  if (st != LORA_OK) return st;
  if (num_tokens < 0) return fail(LORA_EINVAL, "negative num_tokens");
  if (order < LORA_BGMV_AUTO || order > LORA_BGMV_ADAPTER_MAJOR)
    return fail(LORA_EINVAL, "unknown order %d", order);
  if (num_tokens == 0 || w->num_adapters == 0) return ok();
  if (!token_adapter || !x || !v) return fail(LORA_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(v)) return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  const int am = bgmv_order(LORA_PHASE_SHRINK, order, num_tokens, w->num_adapters) ==
                 LORA_BGMV_ADAPTER_MAJOR;
  const int units = am ? w->num_adapters : num_tokens;
  const int groups = (w->r_max + kBgmvRows - 1) / kBgmvRows;
  if ((int64_t)units * groups > INT32_MAX - 8) return fail(LORA_EINVAL, "batch too large");
  const dim3 grid(pad8(units * groups));
  with_types(w, [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    hipLaunchKernelGGL((bgmv_shrink_kernel<T, W, kBgmvRows>), grid, dim3(kThreads), 0, stream, d,
                       token_adapter, num_tokens, am, units, groups, (const T *)x, v);
  });
  return check_launch("bgmv shrink launch");
}

extern "C" lora_status lora_bgmv_expand(const lora_weights *w, const int32_t *token_adapter,
                                        int32_t num_tokens, int32_t order, const float *v, void *y,
                                        hipStream_t stream) {
  DevW d;
  lora_status st = to_dev(w, &d);
  if (st != LORA_OK) return st;
  if (num_tokens < 0) return fail(LORA_EINVAL, "negative num_tokens");
  if (order < LORA_BGMV_AUTO || order > LORA_BGMV_ADAPTER_MAJOR)
    return fail(LORA_EINVAL, "unknown order %d", order);
  if (num_tokens == 0 || w->num_adapters == 0) return ok();
  if (!token_adapter || !v || !y) return fail(LORA_EINVAL, "null pointer");
  if (!aligned16(v) || !aligned16(y)) return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  const int am = bgmv_order(LORA_PHASE_EXPAND, order, num_tokens, w->num_adapters) ==
                 LORA_BGMV_ADAPTER_MAJOR;
  const int units = am ? w->num_adapters : num_tokens;
  constexpr int cols = kBgmvExpandThreads * 8;
  const int groups = (w->d_out + cols - 1) / cols;
  if ((int64_t)units * groups > INT32_MAX - 8) return fail(LORA_EINVAL, "batch too large");
  const dim3 grid(pad8(units * groups));
  with_types(w, [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    hipLaunchKernelGGL((bgmv_expand_kernel<T, W, kBgmvExpandThreads>), grid,
                       dim3(kBgmvExpandThreads), 0, stream, d, token_adapter, num_tokens, am, units,
                       groups, v, (T *)y);
  });
  return check_launch("bgmv expand launch");
}

extern "C" lora_status lora_bgmv_fused(const lora_weights *w, const int32_t *token_adapter,
                                       int32_t num_tokens, const int32_t *token_order,
                                       int32_t num_ordered, int32_t order, const void *x, float *v,
                                       void *y, hipStream_t stream) {
  DevW d;
  lora_status st = to_dev(w, &d);
  if (st != LORA_OK) return st;
  if (num_tokens < 0) return fail(LORA_EINVAL, "negative num_tokens");
  if (num_tokens == 0 || w->num_adapters == 0) return ok();
  if (!token_adapter || !x || !y) return fail(LORA_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(y) || (v && !aligned16(v)))
    return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  if (order < LORA_BGMV_AUTO || order > LORA_BGMV_ADAPTER_MAJOR)
    return fail(LORA_EINVAL, "unknown order %d", order);
  if (token_order && (num_ordered < 0 || num_ordered > num_tokens))
    return fail(LORA_EINVAL, "num_ordered %d outside 0..num_tokens", num_ordered);
  // automatic order: token-major
  const bool am = order == LORA_BGMV_ADAPTER_MAJOR;
  const int units = am ? w->num_adapters : (token_order ? num_ordered : num_tokens);
  if (units == 0) return ok();
  // enough column blocks that the launch has at least ~256 workgroups, one
  // per compute unit: token-major blocks are whole 4096-column passes of the
  // 512 threads; adapter-major blocks are 2048 columns (an adapter-major unit
  // already repeats its shrink per block, so finer blocks add parallelism)
  const int pass = am ? kFusedPass / 2 : kFusedPass;
  const int passes = (w->d_out + pass - 1) / pass;
  int nblk = (kFusedMinGroups + units - 1) / units;
  nblk = nblk < 1 ? 1 : (nblk > passes ? passes : nblk);
  const int block_cols = ((passes + nblk - 1) / nblk) * pass;
  nblk = (w->d_out + block_cols - 1) / block_cols;
  if ((int64_t)units * nblk > INT32_MAX - 8) return fail(LORA_EINVAL, "batch too large");
  if (am) {
    const dim3 grid(pad8(units * nblk));
    with_types(w, [&](auto t, auto wt) {
      using T = decltype(t);
      using W = decltype(wt);
      hipLaunchKernelGGL((bgmv_fused_am_kernel<T, W>), grid, dim3(kFusedThreads), 0, stream, d,
                         token_adapter, num_tokens, nblk, block_cols, (const T *)x, v, (T *)y);
    });
    return check_launch("bgmv fused launch");
  }
  const dim3 grid(pad8(units * nblk));
  // 16-row groups never straddle a page: dense rows, or whole multiples of 16
  const bool aligned = !w->a_page_table || w->page_rows % 16 == 0;
  with_types(w, [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    if (aligned)
      hipLaunchKernelGGL((bgmv_fused_kernel<T, W, true>), grid, dim3(kFusedThreads), 0, stream, d,
                         token_adapter, num_tokens, token_order, units, nblk, block_cols,
                         (const T *)x, v, (T *)y);
    else
      hipLaunchKernelGGL((bgmv_fused_kernel<T, W, false>), grid, dim3(kFusedThreads), 0, stream, d,
                         token_adapter, num_tokens, token_order, units, nblk, block_cols,
                         (const T *)x, v, (T *)y);
  });
  return check_launch("bgmv fused launch");
}

extern "C" lora_status lora_bgmv_fused_multi(const lora_weights *const *w, int32_t num_proj,
                                             const int32_t *token_adapter, int32_t num_tokens,
                                             const int32_t *token_order, int32_t num_ordered,
                                             const void *x, float *const *v, void *const *y,
                                             hipStream_t stream) {
  if (!w || !y) return fail(LORA_EINVAL, "null pointer");
  if (num_proj < 1 || num_proj > kMaxProj)
    return fail(LORA_EINVAL, "num_proj %d outside 1..%d", num_proj, kMaxProj);
  if (num_tokens < 0) return fail(LORA_EINVAL, "negative num_tokens");
  if (token_order && (num_ordered < 0 || num_ordered > num_tokens))
    return fail(LORA_EINVAL, "num_ordered %d outside 0..num_tokens", num_ordered);
  MultiArgs<uint16_t> mb{};  // pointers are retyped per element type below
  bool aligned = true;
  for (int p = 0; p < num_proj; ++p) {
    lora_status st = to_dev(w[p], &mb.w[p]);
    if (st != LORA_OK) return st;
    if (w[p]->dtype != w[0]->dtype || w[p]->weight_format != w[0]->weight_format ||
        w[p]->d_in != w[0]->d_in || w[p]->num_adapters != w[0]->num_adapters)
      return fail(LORA_EINVAL, "projection %d differs from projection 0 in dtype, format, d_in "
                  "or adapter count", p);
    if (!y[p] || !aligned16(y[p]) || (v && v[p] && !aligned16(v[p])))
      return fail(LORA_EINVAL, "projection %d: null or misaligned output", p);
    aligned = aligned && (!w[p]->a_page_table || w[p]->page_rows % 16 == 0);
  }
  if (num_tokens == 0 || w[0]->num_adapters == 0) return ok();
  if (!token_adapter || !x) return fail(LORA_EINVAL, "null pointer");
  if (!aligned16(x)) return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  const int units = token_order ? num_ordered : num_tokens;
  if (units == 0) return ok();
  // column blocks: whole 4096-column passes, enough units in all for ~256
  // workgroups
  mb.first[0] = 0;
  for (int p = 0; p < num_proj; ++p) {
    const int passes = (w[p]->d_out + kFusedPass - 1) / kFusedPass;
    int nblk = (kFusedMinGroups + units * num_proj - 1) / (units * num_proj);
    nblk = nblk < 1 ? 1 : (nblk > passes ? passes : nblk);
    mb.block_cols[p] = ((passes + nblk - 1) / nblk) * kFusedPass;
    nblk = (w[p]->d_out + mb.block_cols[p] - 1) / mb.block_cols[p];
    mb.first[p + 1] = mb.first[p] + nblk;
  }
  for (int p = num_proj + 1; p <= kMaxProj; ++p) mb.first[p] = mb.first[num_proj];
  if ((int64_t)units * mb.first[num_proj] > INT32_MAX - 8) return fail(LORA_EINVAL, "batch too large");
  const dim3 grid(pad8(units * mb.first[num_proj]));
  with_types(w[0], [&](auto t, auto wt) {
    using T = decltype(t);
    using W = decltype(wt);
    MultiArgs<T> m{};
    for (int p = 0; p < kMaxProj; ++p) {
      m.w[p] = mb.w[p];
      m.y[p] = p < num_proj ? (T *)y[p] : nullptr;
      m.v[p] = (p < num_proj && v) ? v[p] : nullptr;
      m.block_cols[p] = mb.block_cols[p];
    }
    for (int p = 0; p <= kMaxProj; ++p) m.first[p] = mb.first[p];
    if (aligned)
      hipLaunchKernelGGL((bgmv_fused_multi_kernel<T, W, true>), grid, dim3(kFusedThreads), 0, stream,
                         m, num_proj, token_adapter, num_tokens, token_order, units, (const T *)x);
    else
      hipLaunchKernelGGL((bgmv_fused_multi_kernel<T, W, false>), grid, dim3(kFusedThreads), 0, stream,
                         m, num_proj, token_adapter, num_tokens, token_order, units, (const T *)x);
  });
  return check_launch("bgmv fused multi launch");
}
