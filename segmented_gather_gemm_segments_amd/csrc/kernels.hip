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
//     Expand keeps v exact by splitting it into a bf16 pair hi + lo (two MFMA
//     K-halves), so v never loses precision to bf16.
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
struct DevW {
  const char *a_pages;
  const char *b_pages;
  const int32_t *rank;
  const int32_t *a_pt;
  const int32_t *b_pt;
  int32_t d_in, d_out, num_adapters, r_max, page_rows, max_pages, num_pages_a, num_pages_b;
};

// Row j of adapter a through the page table; nullptr when the page id is out
// of range (the row then contributes nothing).
template <typename T>
__device__ __forceinline__ const T *page_row(const char *base, const int32_t *pt, int32_t num_pages,
                                             const DevW &w, int a, int j, int width) {
  int page, r_in;
  if (pt) {
    const int pi = j / w.page_rows;
    if (pi >= w.max_pages) return nullptr;
    page = pt[(int64_t)a * w.max_pages + pi];
    r_in = j - pi * w.page_rows;
  } else {
    page = a;
    r_in = j;
  }
  if ((unsigned)page >= (unsigned)num_pages) return nullptr;
  return reinterpret_cast<const T *>(base) + ((int64_t)page * w.page_rows + r_in) * width;
}

template <typename T>
__device__ __forceinline__ const T *a_row(const DevW &w, int a, int j) {
  return page_row<T>(w.a_pages, w.a_pt, w.num_pages_a, w, a, j, w.d_in);
}
template <typename T>
__device__ __forceinline__ const T *b_row(const DevW &w, int a, int j) {
  return page_row<T>(w.b_pages, w.b_pt, w.num_pages_b, w, a, j, w.d_out);
}

__device__ __forceinline__ int adapter_rank(const DevW &w, int a) {
  int r = w.rank[a];
  return r < 0 ? 0 : (r > w.r_max ? w.r_max : r);
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

// ----------------------------------------------------------------- shrink cores
// Token list of the current item in LDS: toks[0..cnt).  Tokens outside
// [0, num_tokens) are skipped.
constexpr int kMaxItemTokens = 256;
constexpr int kRowGroup = LORA_SHRINK_GATHER_ROWS;    // rows of A per segmented gather item
constexpr int kGatherCols = LORA_EXPAND_GATHER_COLS;  // columns of y per segmented gather item
constexpr int kStep = kThreads * 8;                   // d elements covered by one pass of 256 threads
static_assert(kGatherCols == kThreads * 8, "one 8-column chunk per thread");

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

struct ShrinkSmem {
  int toks[kMaxItemTokens];
  union {
    float red_gemv[4 * 64];           // one value per (wave, value index)
    float red_mfma[4 * 4 * 4 * 64];   // [wave][row tile][element][lane]
  };
};

// One gather/GEMV shrink tile: tokens toks[g0 .. g0+ntok) (ntok <= TG) against
// the rows [j0, j0+nr) (nr <= 4) of adapter a.  The 256 threads split d_in into
// 8-element chunks (thread tid: k = 8 tid + 2048 s); each pass issues the loads
// of two such steps (TG x chunks and 4 A chunks each) before the first FMA, and
// the x chunks of a token are reused across the 4 rows in registers.  Rows and
// tokens beyond the tile read a safe in-bounds address (row 0 of x) and their
// sums are dropped.  The TG x 4 lane partials are reduce-scattered over the
// wave and the four wave results summed in wave order, so a token's result
// does not depend on TG or on which other tokens share the tile.
template <typename T, int TG, int RB>
__device__ __forceinline__ void shrink_rows_tile(const DevW &w, int a, int j0, int nr, const int *toks, int g0,
                                 int ntok, int num_tokens, const T *__restrict__ x,
                                 float *__restrict__ v, ShrinkSmem &sm) {
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
  const T *ar[RB];
#pragma unroll
  for (int jj = 0; jj < RB; ++jj) {
    const T *p = jj < nr ? a_row<T>(w, a, j0 + jj) : nullptr;
    ar[jj] = p ? p : safe;
  }
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  for (int k = tid * 8; k < w.d_in; k += 2 * kStep) {
    const bool two = k + kStep < w.d_in;
    Raw8<T> xa[TG], aa[RB], xb[TG], ab[RB];
#pragma unroll
    for (int t = 0; t < TG; ++t) raw_load(xa[t], xr[t] + k);
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) raw_load(aa[jj], ar[jj] + k);
    if (two) {
#pragma unroll
      for (int t = 0; t < TG; ++t) raw_load(xb[t], xr[t] + k + kStep);
#pragma unroll
      for (int jj = 0; jj < RB; ++jj) raw_load(ab[jj], ar[jj] + k + kStep);
    }
    float xv[TG][8];
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
    const float s = ((sm.red_gemv[tid] + sm.red_gemv[64 + tid]) + sm.red_gemv[128 + tid]) +
                    sm.red_gemv[192 + tid];
    const int t = tid / RB, jj = tid % RB;
    if (t < ntok && jj < nr) {
      const int tok = toks[g0 + t];
      if (tok >= 0 && tok < num_tokens) v[(int64_t)tok * w.r_max + j0 + jj] = s;
    }
  }
  __syncthreads();
}

// Gather/GEMV shrink of tokens toks[0..cnt) of adapter a over its row group
// [j0, j0 + nr), nr <= RB: groups of up to 4 tokens, one group of 1 to 3 at the end.
template <typename T, int RB>
__device__ __forceinline__ void shrink_gemv(const DevW &w, int a, int j0, int nr, const int *toks, int cnt,
                            int num_tokens, const T *__restrict__ x, float *__restrict__ v,
                            ShrinkSmem &sm) {
  int g0 = 0;
  for (; g0 + 4 <= cnt; g0 += 4)
    shrink_rows_tile<T, 4, RB>(w, a, j0, nr, toks, g0, 4, num_tokens, x, v, sm);
  const int rest = cnt - g0;
  if (rest == 1) shrink_rows_tile<T, 1, RB>(w, a, j0, nr, toks, g0, 1, num_tokens, x, v, sm);
  else if (rest == 2) shrink_rows_tile<T, 2, RB>(w, a, j0, nr, toks, g0, 2, num_tokens, x, v, sm);
  else if (rest == 3) shrink_rows_tile<T, 4, RB>(w, a, j0, nr, toks, g0, 3, num_tokens, x, v, sm);
}

// One MFMA shrink tile: 16 tokens (this lane's token row xp, or a safe row)
// against RT row tiles of 16 starting at j0.  The four waves take interleaved
// 32-element k-steps; each batch issues the loads of U steps before its
// MFMAs.  Lanes beyond the rank or the tile read safe rows whose outputs are
// dropped; the last, partial k-step zeroes both operands past d_in.
template <typename T, int RT>
__device__ __forceinline__ void shrink_mfma_tile(const DevW &w, int a, int r, int j0, const T *xp, int tok,
                                 const T *__restrict__ x, float *__restrict__ v, ShrinkSmem &sm) {
  constexpr int U = RT == 1 ? 8 : 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const T *safe = x;
  const T *ap[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = j0 + rt * 16 + m;
    const T *p = row < r ? a_row<T>(w, a, row) : nullptr;
    ap[rt] = p ? p : safe;
  }
  f32x4_t acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int full = w.d_in >> 5;             // k-steps entirely inside d_in
  const int nsteps = (w.d_in + 31) >> 5;
  int s = wave;
  for (; s + 4 * (U - 1) < full; s += 4 * U) {
    Frag<T> xf[U], af[U][RT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + 4 * u) * 32 + g * 8;
      frag_load(xf[u], xp + k);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) frag_load(af[u][rt], ap[rt] + k);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = frag_mfma(af[u][rt], xf[u], acc[rt]);
  }
  for (; s < nsteps; s += 4) {
    const int k = s * 32 + g * 8;
    const bool kin = k < w.d_in;
    Frag<T> xf, af[RT];
    if (kin) frag_load(xf, xp + k); else frag_zero(xf);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (kin) frag_load(af[rt], ap[rt] + k); else frag_zero(af[rt]);
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
      const float s4 = ((sm.red_mfma[((0 * 4 + rt) * 4 + e) * 64 + lane] +
                         sm.red_mfma[((1 * 4 + rt) * 4 + e) * 64 + lane]) +
                        sm.red_mfma[((2 * 4 + rt) * 4 + e) * 64 + lane]) +
                       sm.red_mfma[((3 * 4 + rt) * 4 + e) * 64 + lane];
      const int j = j0 + rt * 16 + 4 * g + e;
      if (tok >= 0 && j < r) v[(int64_t)tok * w.r_max + j] = s4;
    }
  }
  __syncthreads();
}

// MFMA shrink for tokens toks[0..cnt) of adapter a: 16-token tiles, passes of
// up to 64 rows.
template <typename T>
__device__ __forceinline__ void shrink_mfma(const DevW &w, int a, int r, const int *toks, int cnt, int num_tokens,
                            const T *__restrict__ x, float *__restrict__ v, ShrinkSmem &sm) {
  const int m = threadIdx.x & 15;
  for (int m0 = 0; m0 < cnt; m0 += 16) {
    int tok = m0 + m < cnt ? toks[m0 + m] : -1;
    if (tok >= num_tokens) tok = -1;
    const T *xp = tok >= 0 ? x + (int64_t)tok * w.d_in : x;
    for (int j0 = 0; j0 < r; j0 += 64) {
      const int nrt = min(4, (r - j0 + 15) >> 4);
      switch (nrt) {
        case 1: shrink_mfma_tile<T, 1>(w, a, r, j0, xp, tok, x, v, sm); break;
        case 2: shrink_mfma_tile<T, 2>(w, a, r, j0, xp, tok, x, v, sm); break;
        case 3: shrink_mfma_tile<T, 3>(w, a, r, j0, xp, tok, x, v, sm); break;
        default: shrink_mfma_tile<T, 4>(w, a, r, j0, xp, tok, x, v, sm); break;
      }
    }
  }
}

// ----------------------------------------------------------------- expand cores
template <typename T> struct ExpandCfg;
template <> struct ExpandCfg<uint16_t> { static constexpr int kRowStride = 72; };  // 64 j + pad
template <> struct ExpandCfg<float> { static constexpr int kRowStride = 68; };

template <typename T>
struct ExpandSmem {
  int toks[kMaxItemTokens];
  T bt[4 * 64 * ExpandCfg<T>::kRowStride];  // MFMA path, per wave: [64 cols][j]
};

// One gather/GEMV expand tile: tokens toks[g0 .. g0+ntok) (ntok <= TG) over
// the 8 NT columns of block cb (NT = threads of the workgroup).  Thread tid
// owns the 8 consecutive columns 8 (NT cb + tid) and runs the whole rank sum
// for them itself -- no cross-lane or cross-wave reduction, no barrier.  B^T rows are loaded 16 at a time
// (16-byte loads, all issued before the first FMA); the y chunks of the tile's
// tokens are fetched at the start; v is read as uniform values.  Every output
// is y + sum_j v_j b_j summed in ascending j, independent of TG.
template <typename T, int TG, int NT>
__device__ __forceinline__ void expand_cols_tile(const DevW &w, int a, int r, int cb, const int *toks, int g0,
                                 int ntok, int num_tokens, const float *__restrict__ v,
                                 T *__restrict__ y) {
  const int col = (cb * NT + (int)threadIdx.x) * 8;
  if (col >= w.d_out) return;
  int tk[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int tok = t < ntok ? uniform(toks[g0 + t]) : -1;
    tk[t] = (tok >= 0 && tok < num_tokens) ? tok : -1;
  }
  Raw8<T> yraw[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t)
    if (tk[t] >= 0) raw_load(yraw[t], y + (int64_t)tk[t] * w.d_out + col);
  const T *safe = reinterpret_cast<const T *>(w.b_pages);
  const bool vec_v = (w.r_max & 3) == 0;
  float acc[TG][8];
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
  for (int j0 = 0; j0 < r; j0 += 16) {
    Raw8<T> braw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const T *p = j0 + i < r ? b_row<T>(w, a, j0 + i) : nullptr;
      raw_load(braw[i], p ? p + col : safe);
    }
    // v[tok][j0 .. j0+16): the same address in every lane, read with 16-byte
    // vector loads (one request per wave) where r_max keeps them aligned
    float vj[TG][16];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float *vr = v + (int64_t)(tk[t] >= 0 ? tk[t] : 0) * w.r_max + j0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jq = j0 + 4 * q;
        if (tk[t] >= 0 && vec_v && jq + 4 <= r) {
          const float4 f = *reinterpret_cast<const float4 *>(vr + 4 * q);
          vj[t][4 * q] = f.x; vj[t][4 * q + 1] = f.y; vj[t][4 * q + 2] = f.z; vj[t][4 * q + 3] = f.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vj[t][4 * q + e] = (tk[t] >= 0 && jq + e < r) ? vr[4 * q + e] : 0.f;
        }
      }
    }
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
    if (tk[t] >= 0) {
      float yv[8];
      raw_cvt(yraw[t], yv);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] += acc[t][e];
      store8(y + (int64_t)tk[t] * w.d_out + col, yv);
    }
  }
}

template <typename T, int NT>
__device__ __forceinline__ void expand_gemv(const DevW &w, int a, int r, int cb, const int *toks, int cnt,
                            int num_tokens, const float *__restrict__ v, T *__restrict__ y) {
  int g0 = 0;
  for (; g0 + 4 <= cnt; g0 += 4) expand_cols_tile<T, 4, NT>(w, a, r, cb, toks, g0, 4, num_tokens, v, y);
  const int rest = cnt - g0;
  if (rest == 1) expand_cols_tile<T, 1, NT>(w, a, r, cb, toks, g0, 1, num_tokens, v, y);
  else if (rest == 2) expand_cols_tile<T, 2, NT>(w, a, r, cb, toks, g0, 2, num_tokens, v, y);
  else if (rest == 3) expand_cols_tile<T, 4, NT>(w, a, r, cb, toks, g0, 3, num_tokens, v, y);
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

// MFMA expand for tokens toks[0..cnt) of adapter a over the 256 columns of
// block `blk` (wave w: 64 columns), 64 tokens (four 16-token tiles) at a time.
// D[col][token] = B^T-slab^T · v^T with the B^T slab staged transposed in LDS;
// the slab fragments of a 16-index K block are read once and used by all four
// token tiles.  bf16: v is split into hi + lo bf16 so each K=32 MFMA covers 16
// rank indices exactly; fp32: 16x16x4 steps.  The y chunks of the 64 tokens
// are prefetched before the slab is staged.
template <typename T>
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
    // prefetch y: lane (g, m) of tile tt touches columns c0 + 32q + 8g .. +7
    Raw8<T> yraw[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = c0 + 32 * q + 8 * g;
        if (tt < ntt && tok[tt] >= 0 && col < w.d_out)
          raw_load(yraw[tt][q], y + (int64_t)tok[tt] * w.d_out + col);
      }
    f32x4_t acc[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[tt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int jc = 0; jc < r; jc += 64) {
      const int nj = min(64, r - jc);
      const int nj16 = (nj + 15) & ~15;
      __syncthreads();  // previous users of the slab are done
      // stage B^T rows jc .. jc+nj16 of this wave's 64 columns, transposed
      for (int jr = lane >> 3; jr < nj16; jr += 8) {
        const int cc = (lane & 7) * 8;
        float bv[8];
        const T *br = (jr < nj && c0 + cc < w.d_out) ? b_row<T>(w, a, jc + jr) : nullptr;
        if (br) {
          load8(br + c0 + cc, bv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (sizeof(T) == 2)
            bt[(cc + e) * RS + jr] = (T)(__float_as_uint(bv[e]) >> 16);  // exact: bv is bf16
          else
            bt[(cc + e) * RS + jr] = bv[e];
        }
      }
      __syncthreads();
      const float *vr[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) vr[tt] = tok[tt] >= 0 ? v + (int64_t)tok[tt] * w.r_max + jc : nullptr;
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
              float f[8];
              load_v8(vr[tt], jb, nj, vec_v, f);
              uint32_t h[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                uint32_t hb = bf16_rne(f[e]);
                if (g >= 2) hb = bf16_rne(f[e] - __uint_as_float(hb << 16));
                h[e] = hb;
              }
              const bf16x8_t bop = __builtin_bit_cast(
                  bf16x8_t, make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                       h[4] | (h[5] << 16), h[6] | (h[7] << 16)));
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
                const float bop = (vr[tt] && j < nj) ? vr[tt][j] : 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[t], bop, acc[tt][t], 0, 0, 0);
              }
            }
          }
        }
      }
    }
    // y update: lane (g, m) holds columns c0 + 32q + 8g .. +7 of token tok[tt]
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

// ----------------------------------------------------------------- kernels
__device__ __forceinline__ bool decode_item(const lora_item &it, const DevW &w, int num_perm,
                                            int &pb, int &a, int &cnt, int &path, int &blk) {
  pb = it.perm_begin;
  a = it.adapter;
  cnt = it.count_path & 0xffff;
  path = it.count_path >> 16;
  blk = it.block;
  if (a < 0 || a >= w.num_adapters || pb < 0 || cnt <= 0 || cnt > kMaxItemTokens ||
      pb + cnt > num_perm || blk < 0)
    return false;
  return true;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sgmv_shrink_kernel(DevW w, const int32_t *__restrict__ perm,
                                                               int32_t num_perm,
                                                               const lora_item *__restrict__ items,
                                                               int32_t num_tokens,
                                                               const T *__restrict__ x,
                                                               float *__restrict__ v) {
  __shared__ ShrinkSmem sm;
  const lora_item it = items[blockIdx.x];
  int pb, a, cnt, path, blk;
  if (!decode_item(it, w, num_perm, pb, a, cnt, path, blk)) return;
  const int r = adapter_rank(w, a);
  if (path != LORA_PATH_MFMA && blk >= (r + kRowGroup - 1) / kRowGroup) return;
  const int j0 = path == LORA_PATH_MFMA ? 0 : blk * kRowGroup;
  for (int i = threadIdx.x; i < cnt; i += kThreads) sm.toks[i] = perm[pb + i];
  __syncthreads();
  if (path == LORA_PATH_MFMA)
    shrink_mfma<T>(w, a, r, sm.toks, cnt, num_tokens, x, v, sm);
  else
    shrink_gemv<T, kRowGroup>(w, a, j0, min(kRowGroup, r - j0), sm.toks, cnt, num_tokens, x, v, sm);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sgmv_expand_kernel(DevW w, const int32_t *__restrict__ perm,
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
  for (int i = threadIdx.x; i < cnt; i += kThreads) sm.toks[i] = perm[pb + i];
  __syncthreads();
  const int r = adapter_rank(w, a);
  if (path == LORA_PATH_MFMA)
    expand_mfma<T>(w, a, r, blk, sm.toks, cnt, num_tokens, v, y, sm);
  else
    expand_gemv<T, kThreads>(w, a, r, blk, sm.toks, cnt, num_tokens, v, y);
}

// Workgroup b of a launch runs on XCD b % 8 (the dispatcher deals workgroups to
// the eight XCDs in turn).  With the grid padded to a multiple of 8, logical
// index (b % 8) * (grid / 8) + b / 8 hands each XCD a contiguous run of logical
// indices, so neighbouring work units -- the row groups of one adapter, which
// read the same x rows -- share that XCD's L2.
__device__ __forceinline__ int xcd_logical(int b, int grid) { return (b & 7) * (grid >> 3) + (b >> 3); }

inline int pad8(int n) { return (n + 7) & ~7; }

// Collects, in token order, the tokens of ids[c0 .. c0+NT) whose adapter is
// `a` into toks[]; returns their count.  All NT threads must call it.
template <int NT>
__device__ __forceinline__ int gather_adapter_tokens(const int32_t *__restrict__ ids, int num_tokens, int c0, int a,
                                     int *toks, int *wave_cnt) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = c0 + tid;
  const bool hit = t < num_tokens && ids[t] == a;
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
// (adapter-major); each unit is split into groups of RB rows, one per workgroup.
template <typename T, int RB>
__global__ __launch_bounds__(kThreads) void bgmv_shrink_kernel(DevW w, const int32_t *__restrict__ ids,
                                                               int32_t num_tokens, int32_t adapter_major,
                                                               int32_t units, int32_t groups,
                                                               const T *__restrict__ x,
                                                               float *__restrict__ v) {
  __shared__ ShrinkSmem sm;
  __shared__ int wave_cnt[4];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  if (L >= units * groups) return;
  const int u = L / groups, j0 = (L - u * groups) * RB;
  if (!adapter_major) {
    const int t = u;
    const int a = ids[t];
    if (a < 0 || a >= w.num_adapters) return;
    const int r = adapter_rank(w, a);
    if (j0 >= r) return;
    if (threadIdx.x == 0) sm.toks[0] = t;
    __syncthreads();
    shrink_gemv<T, RB>(w, a, j0, min(RB, r - j0), sm.toks, 1, num_tokens, x, v, sm);
  } else {
    const int a = u;
    const int r = adapter_rank(w, a);
    if (j0 >= r) return;
    for (int c0 = 0; c0 < num_tokens; c0 += kThreads) {
      const int n = gather_adapter_tokens<kThreads>(ids, num_tokens, c0, a, sm.toks, wave_cnt);
      if (n > 0) shrink_gemv<T, RB>(w, a, j0, min(RB, r - j0), sm.toks, n, num_tokens, x, v, sm);
      __syncthreads();
    }
  }
}

// Per-token (BGMV) expand.  Work unit u as above, split into column blocks of
// 8 NT columns, one per workgroup of NT threads.
template <typename T, int NT>
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
    if (a < 0 || a >= w.num_adapters) return;
    const int tok1[1] = {t};
    expand_cols_tile<T, 1, NT>(w, a, adapter_rank(w, a), cb, tok1, 0, 1, num_tokens, v, y);
  } else {
    const int a = u;
    const int r = adapter_rank(w, a);
    for (int c0 = 0; c0 < num_tokens; c0 += NT) {
      const int n = gather_adapter_tokens<NT>(ids, num_tokens, c0, a, toks, wave_cnt);
      if (n > 0) expand_gemv<T, NT>(w, a, r, cb, toks, n, num_tokens, v, y);
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------- validation
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

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
  if (w->reserved != 0) return fail(LORA_EINVAL, "reserved field must be 0");
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

// Automatic order.  Shrink: adapter-major once adapters are no more numerous
// than tokens (each adapter's A rows are then read by one group of workgroups
// instead of once per token).  Expand: token-major unless an adapter carries
// many tokens on average -- a token-major workgroup needs no scan of the ids
// and its B^T rows, shared with the adapter's other tokens, come from cache.
int bgmv_order(int phase, int order, int num_tokens, int num_adapters) {
  if (order == LORA_BGMV_TOKEN_MAJOR || order == LORA_BGMV_ADAPTER_MAJOR) return order;
  if (phase == LORA_PHASE_SHRINK)
    return num_adapters <= num_tokens ? LORA_BGMV_ADAPTER_MAJOR : LORA_BGMV_TOKEN_MAJOR;
  return num_tokens >= 16 * num_adapters ? LORA_BGMV_ADAPTER_MAJOR : LORA_BGMV_TOKEN_MAJOR;
}

}  // namespace

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
  if (w->dtype == LORA_BF16)
    hipLaunchKernelGGL(sgmv_shrink_kernel<uint16_t>, dim3(num_items), dim3(kThreads), 0, stream, d,
                       token_perm, num_perm, items, num_tokens, (const uint16_t *)x, v);
  else
    hipLaunchKernelGGL(sgmv_shrink_kernel<float>, dim3(num_items), dim3(kThreads), 0, stream, d,
                       token_perm, num_perm, items, num_tokens, (const float *)x, v);
  return check_launch("sgmv shrink launch");
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
  if (w->dtype == LORA_BF16)
    hipLaunchKernelGGL(sgmv_expand_kernel<uint16_t>, dim3(num_items), dim3(kThreads), 0, stream, d,
                       token_perm, num_perm, items, num_tokens, v, (uint16_t *)y);
  else
    hipLaunchKernelGGL(sgmv_expand_kernel<float>, dim3(num_items), dim3(kThreads), 0, stream, d,
                       token_perm, num_perm, items, num_tokens, v, (float *)y);
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
  if (w->dtype == LORA_BF16)
    hipLaunchKernelGGL((bgmv_shrink_kernel<uint16_t, kBgmvRows>), grid, dim3(kThreads), 0, stream, d,
                       token_adapter, num_tokens, am, units, groups, (const uint16_t *)x, v);
  else
    hipLaunchKernelGGL((bgmv_shrink_kernel<float, kBgmvRows>), grid, dim3(kThreads), 0, stream, d,
                       token_adapter, num_tokens, am, units, groups, (const float *)x, v);
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
  if (w->dtype == LORA_BF16)
    hipLaunchKernelGGL((bgmv_expand_kernel<uint16_t, kBgmvExpandThreads>), grid,
                       dim3(kBgmvExpandThreads), 0, stream, d, token_adapter, num_tokens, am, units,
                       groups, v, (uint16_t *)y);
  else
    hipLaunchKernelGGL((bgmv_expand_kernel<float, kBgmvExpandThreads>), grid,
                       dim3(kBgmvExpandThreads), 0, stream, d, token_adapter, num_tokens, am, units,
                       groups, v, (float *)y);
  return check_launch("bgmv expand launch");
}
