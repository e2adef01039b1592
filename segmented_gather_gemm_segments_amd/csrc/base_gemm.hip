// Base projection y = x W^T for the layer the adapters modify: bf16 operands,
// fp32 accumulation on the matrix cores, bf16 output rounded to nearest even.
// It is computed once for every token of the batch, whatever the tokens'
// adapters ("Multi-LoRA serving: the single translator with a thousand
// glossaries", section "The bare mechanism"); the SGMV delta is then added to
// it.  Both operands are contiguous along k (x [m][k], W [n][k]), the layout in
// which every MFMA operand fragment is a run of 8 consecutive k.
//
// Two kernel families share one tiling: the register-staged kernel described
// here serves any shape (ragged edges read as zeros); whole-tile shapes take
// the direct-to-LDS kernels further down, which are faster.
//
// Tiling for gfx950: a workgroup of four waves computes a 128 x 128 tile of y
// over k in steps of 64; each wave owns a 64 x 64 sub-tile as 4 x 4 blocks of
// v_mfma_f32_16x16x32_bf16 with W rows as the A operand and x rows as the B
// operand, so D[n][m] leaves each lane holding 4 consecutive output columns of
// one token (one 8-byte store).  The k-tiles of both operands are staged in one
// LDS buffer with padded rows (72 elements, 36 KiB in all) and prefetched
// through registers: the global loads of tile t+1 are in flight while tile t is
// multiplied, then a barrier, the stores of tile t+1 into LDS, and a second
// barrier.  One buffer rather than two, and registers bounded to three waves
// per SIMD, let three workgroups share a compute unit instead of two; that
// hides more latency and, with 640-tile grids (1280 tokens x 8192 columns),
// runs them in one round of 768 slots instead of 1.25 rounds of 512.  Tiles
// are ordered so that the m-tiles sharing one W tile run on the same XCD
// (workgroup b runs on XCD b % 8) and share its L2.
//
// Grids of few tiles (1280 tokens x 1024 columns is 80 tiles, a third of the
// compute units) split k when the caller lends an fp32 workspace: S slices of
// each tile write fp32 partial tiles, and a second launch adds them in slice
// order and rounds once, so the result does not depend on scheduling.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "lora_internal.h"

using namespace lora;

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBM = 128;       // tokens per tile
constexpr int kBN = 128;       // output columns per tile
constexpr int kBK = 64;        // k per step
constexpr int kLd = kBK + 8;   // LDS row stride in elements (16-byte pad)
constexpr int kGemmThreads = 256;
constexpr int kChunks = kBM * kBK / 8 / kGemmThreads;  // 16-byte chunks per thread per operand
static_assert(kBM == kBN, "one chunk map serves both operands");

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Loads this thread's chunks of one k-tile of rows [row0, row0 + 128) of a
// [rows][ld] operand: chunk c = tid + 256 i is row c / 8, elements 8 (c % 8) ..
// +7 of the tile.  Rows past `rows` and k at or past `k_end` read as zero.
__device__ __forceinline__ void load_tile(const uint16_t *__restrict__ src, int rows, int ld, int k_end,
                                          int row0, int k0, uint4 (&r)[kChunks]) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = (int)threadIdx.x + kGemmThreads * i;
    const int row = row0 + (c >> 3), kk = k0 + (c & 7) * 8;
    if (row < rows && kk < k_end)
      r[i] = *reinterpret_cast<const uint4 *>(src + (int64_t)row * ld + kk);
    else
      r[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile(uint16_t *lds, const uint4 (&r)[kChunks]) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = (int)threadIdx.x + kGemmThreads * i;
    *reinterpret_cast<uint4 *>(lds + (c >> 3) * kLd + (c & 7) * 8) = r[i];
  }
}

__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void base_gemm_kernel(int m, int n, int k, int tiles_m, int tiles, int splits, int k_slice,
                      const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                      uint16_t *__restrict__ y, float *__restrict__ part) {
  __shared__ uint16_t sw[kBN * kLd];
  __shared__ uint16_t sx[kBM * kLd];
  // XCD-aware order: the grid is a multiple of 8; logical tile L = (b % 8) *
  // (grid / 8) + b / 8 gives each XCD a contiguous run, m fastest.
  const int b = blockIdx.x, g8 = gridDim.x >> 3;
  const int U = (b & 7) * g8 + (b >> 3);
  if (U >= tiles * splits) return;
  // unit U = (tile L, k slice sl), slices of a tile adjacent
  const int L = U / splits, sl = U - L * splits;
  const int kb = sl * k_slice, ke = min(k, kb + k_slice);
  const int tm = L % tiles_m, tn = L / tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;     // 2 x 2 waves, 64 x 64 each
  const int fr = lane & 15, fg = lane >> 4;    // fragment row, k group

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = ke > kb ? (ke - kb + kBK - 1) / kBK : 0;
  uint4 rw[kChunks], rx[kChunks];
  load_tile(w, n, k, ke, n0, kb, rw);
  load_tile(x, m, k, ke, m0, kb, rx);
  store_tile(sw, rw);
  store_tile(sx, rx);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      load_tile(w, n, k, ke, n0, kb + (kt + 1) * kBK, rw);
      load_tile(x, m, k, ke, m0, kb + (kt + 1) * kBK, rx);
    }
    const uint16_t *tw = sw + (wn * 64 + fr) * kLd + fg * 8;
    const uint16_t *tx = sx + (wm * 64 + fr) * kLd + fg * 8;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(tw + i * 16 * kLd + ks * 32));
        fb[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(tx + i * 16 * kLd + ks * 32));
      }
      // ask the scheduler to interleave the fragment reads with the MFMAs
      // (left to itself it waits for every read before each row of 4 MFMAs)
      __builtin_amdgcn_iglp_opt(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading tile kt
    if (more) {
      store_tile(sw, rw);
      store_tile(sx, rx);
    }
    __syncthreads();
  }
  // D[n][m] of block (i, j): lane (fg, fr) holds columns n0 + 64 wn + 16 i + 4 fg
  // .. +3 of token m0 + 64 wm + 16 j + fr
  float *pt = splits > 1 ? part + (int64_t)sl * m * n : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = n0 + wn * 64 + i * 16 + fg * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + wm * 64 + j * 16 + fr;
      if (row < m && col < n) {
        if (pt) {
          *reinterpret_cast<f32x4_t *>(pt + (int64_t)row * n + col) = acc[i][j];
        } else {
          uint2 o;
          o.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
          o.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2 *>(y + (int64_t)row * n + col) = o;
        }
      }
    }
  }
}

// Whole-tile shapes (m, n multiples of 128, k of the k-step): the same tile
// and wave layout, but the k-tiles go from global memory straight into LDS
// (global_load_lds_dwordx4: lane l of a wave's load writes 16 bytes at the
// load's LDS base + 16 l), so no registers stage them and no LDS stores are
// issued, and two LDS buffers alternate with one barrier per step.  Rows are
// unpadded; the 16-byte chunks of a row are permuted by an XOR of the row
// index so that the 8 lanes of an LDS read phase (8 consecutive rows, one
// chunk) hit 8 different bank groups.  A k-step of 64 (64 KiB of LDS, two
// workgroups per CU) does more work per barrier and suits large grids; a
// k-step of 32 (32 KiB, three per CU) suits grids of a few rounds, where the
// slot count decides how full the last round is.
template <int BK>
struct LdsTile {
  static constexpr int kCpr = BK / 8;         // 16-byte chunks per row
  static constexpr int kRows = 64 / kCpr;     // rows per wave load
  static constexpr int kLoads = 128 * kCpr / kGemmThreads;  // loads per thread per operand
  // LDS slot of chunk c of row r (an involution: also the chunk of slot c)
  __device__ static __forceinline__ int slot(int r, int c) {
    return BK == 64 ? c ^ (r & 7) : c ^ ((r >> 1) & 3);
  }
};

template <int BK>
__device__ __forceinline__ void issue_tile_lds(const uint16_t *__restrict__ src, int ld, int row0, int k0,
                                               uint16_t *lds) {
  using LT = LdsTile<BK>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / LT::kCpr, c = LT::slot(rl, lane % LT::kCpr);
#pragma unroll
  for (int i = 0; i < LT::kLoads; ++i) {
    const int g = i * (kGemmThreads / 64) + wave;  // this wave load's rows: g kRows .. +kRows-1
    const uint16_t *p = src + (int64_t)(row0 + g * LT::kRows + rl) * ld + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(p, (__attribute__((address_space(3))) void *)(lds + g * LT::kRows * BK),
                                     16, 0, 0);
  }
}

template <int BK>
__device__ __forceinline__ void base_gemm_lds_body(int m, int n, int k, int tiles_m, int tiles, int splits,
                                                   int k_slice, const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ w,
                                                   uint16_t *__restrict__ y, float *__restrict__ part) {
  using LT = LdsTile<BK>;
  // four separate arrays rather than two double buffers: the compiler keeps
  // apart accesses to different LDS variables, so it does not wait for the
  // loads into one buffer before reading the other
  __shared__ __attribute__((aligned(16))) uint16_t sw0[128 * BK], sw1[128 * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sx0[128 * BK], sx1[128 * BK];
  const int b = blockIdx.x, g8 = gridDim.x >> 3;
  const int U = (b & 7) * g8 + (b >> 3);
  if (U >= tiles * splits) return;
  const int L = U / splits, sl = U - L * splits;
  const int kb = sl * k_slice, ke = min(k, kb + k_slice);
  const int tm = L % tiles_m, tn = L / tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int fr = lane & 15, fg = lane >> 4;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = ke > kb ? (ke - kb) / BK : 0;
  if (nk > 0) {
    issue_tile_lds<BK>(w, k, n0, kb, sw0);
    issue_tile_lds<BK>(x, k, m0, kb, sx0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // every counter to zero: this wave's tile is in LDS
  __syncthreads();
  // one k-step: loads of step kt+1 into the other buffer, MFMAs on buffer B
  // (a compile-time constant: the loop below is unrolled by two)
  auto step = [&](auto bufc, int kt) {
    constexpr int B = decltype(bufc)::value;
    uint16_t *rw = B ? sw1 : sw0, *rx = B ? sx1 : sx0;  // read now
    uint16_t *nw = B ? sw0 : sw1, *nx = B ? sx0 : sx1;  // loaded for the next step
    if (kt + 1 < nk) {
      issue_tile_lds<BK>(w, k, n0, kb + (kt + 1) * BK, nw);
      issue_tile_lds<BK>(x, k, m0, kb + (kt + 1) * BK, nx);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t fa[4], fb[4];
      const int ch = ks * 4 + fg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wn * 64 + i * 16 + fr, rb = wm * 64 + i * 16 + fr;
        fa[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(rw + ra * BK + LT::slot(ra, ch) * 8));
        fb[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(rx + rb * BK + LT::slot(rb, ch) * 8));
      }
      if (BK == 32) __builtin_amdgcn_iglp_opt(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's loads (this wave's share) have landed
    __syncthreads();                // ... and every wave's, and nobody still reads buffer B
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
  }
  float *pt = splits > 1 ? part + (int64_t)sl * m * n : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = n0 + wn * 64 + i * 16 + fg * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + wm * 64 + j * 16 + fr;
      if (pt) {
        *reinterpret_cast<f32x4_t *>(pt + (int64_t)row * n + col) = acc[i][j];
      } else {
        uint2 o;
        o.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
        o.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2 *>(y + (int64_t)row * n + col) = o;
      }
    }
  }
}

__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void base_gemm_lds64_kernel(int m, int n, int k, int tiles_m, int tiles, int splits, int k_slice,
                            const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                            uint16_t *__restrict__ y, float *__restrict__ part) {
  base_gemm_lds_body<64>(m, n, k, tiles_m, tiles, splits, k_slice, x, w, y, part);
}
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void base_gemm_lds32_kernel(int m, int n, int k, int tiles_m, int tiles, int splits, int k_slice,
                            const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                            uint16_t *__restrict__ y, float *__restrict__ part) {
  base_gemm_lds_body<32>(m, n, k, tiles_m, tiles, splits, k_slice, x, w, y, part);
}

// y = round(sum over slices s = 0 .. splits-1 of part[s]), 4 outputs per thread.
__global__ __launch_bounds__(256) void base_gemm_reduce_kernel(int64_t mn, int splits,
                                                               const float *__restrict__ part,
                                                               uint16_t *__restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  f32x4_t a = *reinterpret_cast<const f32x4_t *>(part + i);
  for (int s = 1; s < splits; ++s) a += *reinterpret_cast<const f32x4_t *>(part + s * mn + i);
  uint2 o;
  o.x = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
  o.y = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
  *reinterpret_cast<uint2 *>(y + i) = o;
}

constexpr int kMaxSplits = 4;
constexpr int kSlotsPerCu = 3;       // workgroups of the GEMM kernel one compute unit holds
constexpr int kMinStepsPerSlice = 4;  // k steps each slice keeps at least

// Slices of k for an m x n x k problem on `cus` compute units: the largest
// S <= 4 (a power of two) whose S x tiles units still fit in one round of the
// device's slots (three workgroups per CU) and leave every slice at least 4
// k-steps of 64; 1 for grids of more than half the slots.
int pick_splits(int64_t tiles, int k, int cus) {
  const int64_t slots = (int64_t)kSlotsPerCu * cus;
  int s = 1;
  while (s < kMaxSplits && tiles * s * 2 <= slots && k >= 2 * s * kMinStepsPerSlice * kBK) s *= 2;
  return s;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Checks the arguments shared by both entry points (LORA_OK, or an error with
// its message); *tiles_m, *tiles get the grid's tile counts.
lora_status check_gemm(int32_t dtype, int32_t m, int32_t n, int32_t k, const void *x, const void *w,
                       const void *y, int64_t *tiles_m, int64_t *tiles) {
  if (dtype != LORA_BF16) return fail(LORA_EUNSUPPORTED, "base gemm supports bf16 only");
  if (m < 0 || n <= 0 || k <= 0) return fail(LORA_EINVAL, "base gemm sizes m=%d n=%d k=%d", m, n, k);
  if (n % 8 || k % 8) return fail(LORA_EUNSUPPORTED, "base gemm needs n and k multiples of 8");
  *tiles_m = (m + kBM - 1) / kBM;
  *tiles = *tiles_m * ((n + kBN - 1) / kBN);
  if (m == 0) return ok();
  if (!x || !w || !y) return fail(LORA_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y))
    return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  return ok();
}

// Enqueues the GEMM with k cut into `splits` slices (1: no split; more: their
// fp32 partial tiles go to `part`, splits * m * n floats, then the reduction).
lora_status launch_gemm(int32_t m, int32_t n, int32_t k, int64_t tiles_m, int64_t tiles, int splits,
                        const void *x, const void *w, void *y, float *part, hipStream_t stream) {
  if (tiles * splits > INT32_MAX - 8) return fail(LORA_EINVAL, "base gemm too large");
  // slice length in whole k-steps
  const int k_slice = (int)((((int64_t)k + splits - 1) / splits + kBK - 1) / kBK * kBK);
  const int grid = (int)((tiles * splits + 7) & ~int64_t(7));
  // whole tiles: direct-to-LDS kernels, a k-step of 64 for grids of at least
  // six tiles per CU (three rounds of two), else 32; otherwise the
  // register-staged kernel, which reads ragged edges as zeros
  const bool whole = m % kBM == 0 && n % kBN == 0 && k % 64 == 0;
  auto kern = base_gemm_kernel;
  if (whole) kern = tiles * splits >= 6 * (int64_t)device_cus() ? base_gemm_lds64_kernel : base_gemm_lds32_kernel;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), 0, stream, m, n, k, (int)tiles_m,
                     (int)tiles, splits, k_slice, (const uint16_t *)x, (const uint16_t *)w,
                     (uint16_t *)y, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "base gemm launch");
  if (splits > 1) {
    const int64_t mn = (int64_t)m * n;  // a multiple of 8
    const int64_t blocks = (mn / 4 + 255) / 256;
    if (blocks > INT32_MAX) return fail(LORA_EINVAL, "base gemm too large");
    hipLaunchKernelGGL(base_gemm_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mn,
                       splits, (const float *)part, (uint16_t *)y);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "base gemm reduce launch");
  }
  return ok();
}

}  // namespace

// ----------------------------------------------------------------- scratch
// Device memory of lora_base_gemm_noalloc's split-k partial tiles, held by
// the library on every device it runs on until the process ends.  Its size
// covers every split the rule in pick_splits asks for on a 256-CU device:
// S x tiles <= 1.5 x CUs units of 128 x 128 fp32 partials, 384 x 64 KiB.
constexpr int64_t kScratchBytes = LORA_BASE_GEMM_SCRATCH_BYTES;
static_assert(kScratchBytes == int64_t(24) << 20, "24 MiB");
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current (in host code the array's name is only a host-side
// stand-in, never a device address).
lora_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LORA_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LORA_EHIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ok();
}

}  // namespace

extern "C" lora_status lora_base_gemm_workspace(int32_t m, int32_t n, int32_t k, int64_t *bytes) {
  if (!bytes) return fail(LORA_EINVAL, "null pointer");
  *bytes = 0;
  if (m < 0 || n <= 0 || k <= 0) return fail(LORA_EINVAL, "base gemm sizes m=%d n=%d k=%d", m, n, k);
  if (m == 0) return ok();
  const int64_t tiles = ((m + kBM - 1) / kBM) * (int64_t)((n + kBN - 1) / kBN);
  const int s = pick_splits(tiles, k, device_cus());
  if (s > 1) *bytes = (int64_t)s * m * n * (int64_t)sizeof(float);
  return ok();
}

extern "C" lora_status lora_base_gemm(int32_t dtype, int32_t m, int32_t n, int32_t k,
                                      const void *x, const void *w, void *y, void *workspace,
                                      int64_t workspace_bytes, hipStream_t stream) {
  int64_t tiles_m = 0, tiles = 0;
  lora_status st = check_gemm(dtype, m, n, k, x, w, y, &tiles_m, &tiles);
  if (st != LORA_OK) return st;
  if (workspace_bytes < 0) return fail(LORA_EINVAL, "negative workspace size");
  if (m == 0) return ok();
  if (workspace && !aligned16(workspace)) return fail(LORA_EINVAL, "device arrays must be 16-byte aligned");
  // split k only into a workspace that holds every slice's partial tile
  int splits = 1;
  if (workspace) {
    const int s = pick_splits(tiles, k, device_cus());
    if (s > 1 && workspace_bytes >= (int64_t)s * m * n * (int64_t)sizeof(float)) splits = s;
  }
  return launch_gemm(m, n, k, tiles_m, tiles, splits, x, w, y, (float *)workspace, stream);
}

extern "C" lora_status lora_base_gemm_noalloc(int32_t dtype, int32_t m, int32_t n, int32_t k,
                                              const void *x, const void *w, void *y,
                                              hipStream_t stream) {
  int64_t tiles_m = 0, tiles = 0;
  lora_status st = check_gemm(dtype, m, n, k, x, w, y, &tiles_m, &tiles);
  if (st != LORA_OK || m == 0) return st;
  const int s = pick_splits(tiles, k, device_cus());
  void *part = nullptr;
  if (s > 1) {
    const int64_t need = (int64_t)s * m * n * (int64_t)sizeof(float);
    if (need > kScratchBytes)
      return fail(LORA_ENOMEM, "base gemm %dx%dx%d splits k %d ways into %lld bytes of partial "
                  "tiles; the library's scratch holds %lld", m, n, k, s, (long long)need,
                  (long long)kScratchBytes);
    if ((st = scratch_address(&part)) != LORA_OK) return st;
  }
  return launch_gemm(m, n, k, tiles_m, tiles, s, x, w, y, (float *)part, stream);
}
