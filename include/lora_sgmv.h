/*
 * lora_sgmv.h -- C ABI of the MI355X (gfx950) multi-LoRA delta path.
 *
 * What is computed.  For every token t of a batch whose tokens carry
 * different LoRA adapters, add the adapter's low-rank correction to the
 * layer's output:
 *
 *     y_t  <-  y_t + B_{a(t)} ( A_{a(t)} x_t )
 *
 * with A_a in R^{r_a x d_in}, B_a in R^{d_out x r_a}; the product B A is never
 * formed.  Sources: "Multi-LoRA serving: the single translator with a thousand
 * glossaries" (blog.lo0.es), section "The bare mechanism" (y = Wx + B(Ax), the
 * shapes of A and B) and section "SGMV: the kernel that holds it all up" (the
 * per-token equation y_t = W x_t + B_{a(t)} A_{a(t)} x_t, its two phases
 * shrink d_in -> r and expand r -> d_out, grouping tokens by adapter, one
 * launch for every adapter of the batch, tensor cores for large segments and a
 * batched gather path for small ones).  y_t enters holding the base term W x_t.
 *
 * Storage conventions (shared by every entry point):
 *   - x [T, d_in] and y [T, d_out] are row-major device arrays indexed by the
 *     token's ORIGINAL position in the batch; element type = lora_weights.dtype.
 *   - v [T, r_max] is a row-major fp32 device array (the rank-space
 *     intermediate A x, never rounded to bf16).  Entries j >= r_{a(t)} and rows
 *     of tokens without an adapter are not written.
 *   - A_a is stored as r_a rows of length d_in ("A rows"); B_a as its transpose,
 *     r_a rows of length d_out ("B^T rows").  Rows live in pages of page_rows
 *     rows each; a per-adapter page table names the pages (S-LoRA-style unified
 *     paging: "Multi-LoRA serving ..." TL;DR and section "Operational pitfalls",
 *     memory fragmentation; and the glossary entry "Multi-LoRA Serving",
 *     skillsintelligence.tools, intro paragraph).  Dense per-adapter stacks are
 *     the special case page_rows >= r_max with a NULL page table (page a holds
 *     adapter a).
 *   - No alpha/r scale is applied: a caller that wants one pre-scales B.
 *   - Adapter id LORA_NO_ADAPTER (-1) means the token has no adapter: its y row
 *     is left bit-unchanged ("Multi-LoRA Inference Serving", clusterbid.com,
 *     paragraph on vLLM's adapter pool: only a request that names an adapter
 *     gets one).
 *   - bf16 arithmetic: products and sums in fp32; y is rounded once, to nearest
 *     even, when stored.  fp32 workloads compute in fp32 throughout.
 *
 * Calls and errors.
 *   - Every function returns a lora_status; LORA_OK == 0.  On any error nothing
 *     is launched and no output is touched; lora_last_error() gives a message
 *     (thread-local, valid until the thread's next call into the library).
 *   - Host-side functions (segments, plan, pool bookkeeping) are synchronous
 *     and need no GPU.  Device-side functions enqueue work on `stream` (the
 *     caller's HIP stream; 0 = default) and return without synchronising.
 *   - The library allocates no device memory on any call below; every buffer
 *     is caller-owned, except the fixed scratch array that the library's code
 *     object holds for lora_base_gemm_noalloc.  Pointers to device arrays must
 *     be 16-byte aligned, and d_in and d_out multiples of 8.
 *   - Each y element is written by exactly one GPU thread, with no atomics, so
 *     results are bit-identical from run to run.
 *   - Device-resident indices (token_perm, plan items, page tables, per-token
 *     adapter ids, ranks) are checked by the kernels: an out-of-range value
 *     makes the affected token or row contribute nothing instead of reading
 *     out of bounds.  Outputs for such tokens are then unspecified.  The debug
 *     build of the library reports such values (lora_debug_flags below).
 */
#ifndef LORA_SGMV_H
#define LORA_SGMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 2

typedef int32_t lora_status;
#define LORA_OK 0
#define LORA_EINVAL (-1)        /* null pointer, negative size, misalignment, inconsistent sizes */
#define LORA_ERANGE (-2)        /* a host-visible adapter id outside {-1} U [0, num_adapters) */
#define LORA_EUNSUPPORTED (-3)  /* rank outside 1..LORA_MAX_RANK, d not a multiple of 8, unknown dtype */
#define LORA_ENOMEM (-4)        /* page pool exhausted, or an output array too small */
#define LORA_EHIP (-5)          /* a HIP runtime error; its text is in lora_last_error() */

#define LORA_F32 0
#define LORA_BF16 1

/* Storage formats of the adapter rows (lora_weights.weight_format). */
#define LORA_WFMT_PLAIN 0     /* elements of type lora_weights.dtype */
#define LORA_WFMT_FP8_E4M3 1  /* OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7,
                                 3 mantissa bits; 0x7f / 0xff are NaN, no infinities),
                                 one byte per element */
#define LORA_WFMT_INT4 2      /* two's-complement 4-bit integers in -8..7, two per
                                 byte, element 2i in the low nibble of byte i */

#define LORA_NO_ADAPTER (-1)
#define LORA_MAX_RANK 128

int32_t lora_abi_version(void);
const char *lora_last_error(void);
const char *lora_status_name(lora_status status);

/* ------------------------------------------------------------------------ */
/* Segment build (host).  Groups the batch's tokens by adapter: ascending
 * adapter id, original token order inside a segment, tokens with id -1
 * skipped ("SGMV: the kernel that holds it all up": SGMV groups the batch's
 * tokens by adapter; TL;DR: one pass grouping requests by adapter).  Stable
 * counting sort, O(T + N).
 *   token_adapter [num_tokens]     in : adapter per token (-1 = none)
 *   token_perm    [num_tokens]     out: the T' adapted tokens, segment by segment
 *   seg_starts    [num_tokens + 1] out: segment s is token_perm[seg_starts[s] ..
 *                                       seg_starts[s+1]); seg_starts[S] = T'
 *   seg_adapter   [num_tokens]     out: adapter of segment s (strictly increasing)
 *   num_segments                   out: S
 * All arrays are caller-owned host memory with the capacities shown.
 * Errors: LORA_EINVAL (null pointer with num_tokens > 0, negative sizes),
 * LORA_ERANGE (an id outside {-1} U [0, num_adapters)); outputs untouched. */
lora_status lora_segments_build(const int32_t *token_adapter, int32_t num_tokens,
                                int32_t num_adapters, int32_t *token_perm,
                                int32_t *seg_starts, int32_t *seg_adapter,
                                int32_t *num_segments);

/* ------------------------------------------------------------------------ */
/* Work plan (host).  One launch per phase covers every segment of the batch
 * ("SGMV ..." section: the correct delta for every token in a single kernel
 * pass; "Multi-LoRA Inference Serving": blocks from several adapters
 * dispatched onto different compute units by one launch).  Each segment takes
 * the MFMA path when it holds at least `mfma_min_tokens` tokens and the
 * gather/GEMV path otherwise (the page's size-dependent choice: tensor cores
 * for large segments, batched gather for one-request segments).  The plan is a
 * flat list of work items, heaviest first, that covers every (token, output)
 * pair of the batch exactly once; item k is executed by workgroup k.
 *
 * Items:
 *   shrink, gather path: up to LORA_SHRINK_GATHER_TOKENS tokens x one group of
 *     LORA_SHRINK_GATHER_ROWS rows of A (block = row group); one item per row
 *     group the adapter's rank needs;
 *   shrink, MFMA path: up to LORA_SHRINK_MFMA_TOKENS tokens x every row (block 0);
 *   expand, gather path: up to LORA_EXPAND_GATHER_TOKENS tokens x one block of
 *     LORA_EXPAND_GATHER_COLS columns of y;
 *   expand, MFMA path: up to 64 tokens x one block of LORA_EXPAND_MFMA_COLS
 *     columns; up to LORA_EXPAND_MFMA_TOKENS (128) tokens for output widths
 *     near 8192 columns (a width takes the choice measured on MI355X for the
 *     nearest of 1024, 4096, 8192, 14336 and 28672 columns; 128 ran faster
 *     only at 8192), and only while the plan then still holds at least
 *     LORA_EXPAND_LONG_TILE_MIN_ITEMS MFMA items.
 * A shrink plan depends on the adapters' ranks (host_rank, or r_max for every
 * adapter when host_rank is NULL) but not on d_in; an expand plan depends on
 * d_out but not on the ranks.  A plan stays valid for every projection with
 * the same segments, ranks (shrink) and d_out (expand): build once per batch,
 * upload once, launch many.                                                  */
typedef struct {
  int32_t perm_begin;  /* first token of the item, as an index into token_perm */
  int32_t adapter;     /* adapter of the item's segment */
  int32_t count_path;  /* token count (bits 0..15) | path << 16 */
  int32_t block;       /* shrink: row group (gather) or 0 (MFMA); expand: column block */
} lora_item;

#define LORA_PHASE_SHRINK 0
#define LORA_PHASE_EXPAND 1

#define LORA_PATH_AUTO 0    /* policy: choose per segment by length */
#define LORA_PATH_GATHER 1  /* policy: every segment on the gather/GEMV path */
#define LORA_PATH_MFMA 2    /* policy: every segment on the MFMA path */

#define LORA_DEFAULT_MFMA_MIN_TOKENS 16

/* Tokens, rows and columns per item, by path.  */
#define LORA_SHRINK_GATHER_TOKENS 4
#define LORA_SHRINK_GATHER_ROWS 4
#define LORA_SHRINK_MFMA_TOKENS 16
#define LORA_EXPAND_GATHER_TOKENS 4
#define LORA_EXPAND_MFMA_TOKENS 128
#define LORA_EXPAND_GATHER_COLS 2048
#define LORA_EXPAND_MFMA_COLS 256
#define LORA_EXPAND_LONG_TILE_MIN_ITEMS 256   /* one per compute unit of an MI355X */

/* Builds the plan for `phase` from the host copies of segment_build's output.
 *   host_rank      shrink: host [num_adapters] ranks (1..r_max), or NULL (every
 *                  adapter planned at r_max); expand: ignored
 *   dim            shrink: r_max (1..LORA_MAX_RANK); expand: d_out (> 0, a
 *                  multiple of 8)
 *   path_policy    LORA_PATH_AUTO / _GATHER / _MFMA
 *   mfma_min_tokens  AUTO threshold (<= 0 selects LORA_DEFAULT_MFMA_MIN_TOKENS)
 *   items, capacity  caller-owned host array; with items == NULL only the item
 *                    count is returned (in *num_items)
 * Errors: LORA_EINVAL (bad sizes, non-increasing seg_starts, unknown policy or
 * phase), LORA_ERANGE (a segment adapter outside [0, num_adapters), a rank
 * outside 1..r_max), LORA_EUNSUPPORTED (dim out of range), LORA_ENOMEM
 * (capacity too small; *num_items still holds the needed count).            */
lora_status lora_sgmv_plan(int32_t phase, const int32_t *seg_starts,
                           const int32_t *seg_adapter, int32_t num_segments,
                           int32_t num_adapters, const int32_t *host_rank, int32_t dim,
                           int32_t path_policy, int32_t mfma_min_tokens, lora_item *items,
                           int32_t capacity, int32_t *num_items);
/* lora_sgmv_plan with the expand's MFMA token tile given: expand_tile_tokens
 * 0 takes the width table above (what lora_sgmv_plan does), 64 or
 * LORA_EXPAND_MFMA_TOKENS forces that tile (a shrink plan ignores it); for
 * other devices or shapes, and to reproduce the table's measurements.  The
 * kernels give every token the same bits under either tile.  Errors as
 * lora_sgmv_plan, and LORA_EINVAL for another expand_tile_tokens.          */
lora_status lora_sgmv_plan_tile(int32_t phase, const int32_t *seg_starts,
                                const int32_t *seg_adapter, int32_t num_segments,
                                int32_t num_adapters, const int32_t *host_rank, int32_t dim,
                                int32_t path_policy, int32_t mfma_min_tokens,
                                int32_t expand_tile_tokens, lora_item *items, int32_t capacity,
                                int32_t *num_items);

/* ------------------------------------------------------------------------ */
/* Adapter weights as the kernels read them (the adapter-row gather through the
 * page table).  Row j of adapter a's A is stored row
 *     s = a_page_table[a*max_pages + j/page_rows] * page_rows + j % page_rows
 * of a_pages, at byte offset s * row_bytes(d_in), and row j of its B^T likewise
 * in b_pages with width d_out.  With a NULL page table the page index is the
 * adapter id (dense stack: page_rows >= r_max, max_pages ignored).  Rows
 * j >= rank[a] of a page are never read.
 *
 * Quantized rows (weight_format FP8_E4M3 or INT4, with dtype LORA_BF16): each
 * stored row s holds codes q and has an fp32 scale sc[s] (a_scales, b_scales,
 * indexed by the same stored-row number s); its values are q * sc[s].  FP8
 * storage halves an adapter's bytes and INT4 storage quarters them ("Multi-LoRA
 * Inference Serving: Serving Thousands of Fine-Tuned Models on One GPU",
 * clusterbid.com, the paragraphs on the adapter memory budget and on adapter
 * weight quantization); the codes are dequantized inside the kernels, so the
 * rows cross HBM in their stored size.  The scales factor out of both phases:
 * v[j] is the row-j sum of codes times x, times A's row scale; the expand uses
 * v[j] times B^T's row scale.  row_bytes(d) = 2d (bf16), 4d (fp32), d (FP8),
 * d/2 (INT4).  */
typedef struct {
  int32_t dtype;         /* LORA_F32 or LORA_BF16: element type of x, y, A, B */
  int32_t d_in, d_out;   /* multiples of 8 */
  int32_t num_adapters;  /* N: valid adapter ids are 0..N-1 */
  int32_t r_max;         /* every rank <= r_max <= LORA_MAX_RANK; row stride of v */
  int32_t page_rows;     /* rows per page (> 0) */
  int32_t max_pages;     /* page-table row length (pages per adapter) */
  int32_t num_pages_a;   /* pages in a_pages (bounds for page ids) */
  int32_t num_pages_b;   /* pages in b_pages */
  int32_t weight_format; /* LORA_WFMT_PLAIN, or (dtype LORA_BF16 only) LORA_WFMT_FP8_E4M3
                            or LORA_WFMT_INT4 */
  const void *a_pages;   /* device [num_pages_a][page_rows] rows of row_bytes(d_in) */
  const void *b_pages;   /* device [num_pages_b][page_rows] rows of row_bytes(d_out) (B^T) */
  const int32_t *rank;   /* device [N]: rank of each adapter (1..r_max) */
  const int32_t *a_page_table; /* device [N][max_pages] or NULL (dense) */
  const int32_t *b_page_table; /* device [N][max_pages] or NULL (dense) */
  const int32_t *host_rank;    /* host [N] copy of rank, or NULL; when given it is
                                  validated (1..r_max) before launch */
  const float *a_scales;       /* device [num_pages_a * page_rows] row scales; quantized
                                  formats only (NULL for LORA_WFMT_PLAIN) */
  const float *b_scales;       /* device [num_pages_b * page_rows] */
} lora_weights;

/* ------------------------------------------------------------------------ */
/* Segmented (SGMV) mode: the batch arrives grouped by lora_segments_build and
 * planned by lora_sgmv_plan (items uploaded to device memory by the caller).
 *
 * Shrink ("SGMV ..." section, phase 1, projection d_in -> r through A_{a(t)}):
 *     v[t][j] = sum_k A_{a(t)}[j][k] * x[t][k]        for j < r_{a(t)}
 * Expand (phase 2, projection r -> d_out through B_{a(t)}, added into y):
 *     y[t][i] = round( y[t][i] + sum_j B_{a(t)}[i][j] * v[t][j] )
 *   token_perm [num_perm]   device; token indices in [0, num_tokens)
 *   items      [num_items]  device; a plan of the matching phase
 * num_items == 0 or num_tokens == 0 is a no-op.  Errors: LORA_EINVAL,
 * LORA_EUNSUPPORTED, LORA_ERANGE (host_rank out of 1..r_max), LORA_EHIP.   */
lora_status lora_sgmv_shrink(const lora_weights *w, const int32_t *token_perm, int32_t num_perm,
                             const lora_item *items, int32_t num_items, int32_t num_tokens,
                             const void *x, float *v, hipStream_t stream);
lora_status lora_sgmv_expand(const lora_weights *w, const int32_t *token_perm, int32_t num_perm,
                             const lora_item *items, int32_t num_items, int32_t num_tokens,
                             const float *v, void *y, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Tiled segmented shrink: the v of lora_sgmv_shrink for bf16 activations and
 * bf16, FP8 E4M3 or INT4 rows (dequantised to bf16 MFMA operands as they leave
 * LDS; a row's scale multiplies its sums), planned for segments whose shrink
 * is a real dense product
 * ("SGMV ..." section: the shrink phase, d_in -> r through A_{a(t)}; tensor
 * cores for the long segments).  A tile item is up to LORA_SHRINK_TILE_TOKENS
 * tokens of one segment and one slice of d_in: its workgroup streams the
 * tokens' x rows and the adapter's A rows of the slice into LDS once (so A
 * crosses the compute unit once per 64 tokens instead of once per 16) and
 * runs the products on MFMA.  With more than one slice the items write fp32
 * partial products to a caller-owned workspace and a second launch on the
 * same stream adds each token's partials in slice order (a fixed order:
 * repeated runs are bit-identical).  Short low-rank segments keep gather
 * items.
 *
 * lora_sgmv_plan_tiled: as lora_sgmv_plan's shrink phase, plus d_in (a
 * multiple of LORA_SHRINK_TILE_K) and max_splits (1..LORA_MAX_K_SPLITS; <= 0:
 * no bound but d_in's).  Segments of at least tile_min_tokens tokens (<= 0:
 * LORA_DEFAULT_TILE_MIN_TOKENS), and shorter ones of rank at least
 * LORA_TILE_MIN_RANK_SHORT (whose gather items would read each x row r / 4
 * times), take tile items (path LORA_PATH_TILE, block = slice); the others
 * gather items as in lora_sgmv_plan (policy GATHER: none tiled; MFMA: all
 * tiled).  *k_splits receives the number of slices, chosen so
 * that the heaviest tile item reads about LORA_SHRINK_TILE_ITEM_BYTES; every
 * slice is a non-empty multiple of LORA_SHRINK_TILE_K elements.  Items
 * heaviest first.  Errors as lora_sgmv_plan, LORA_EUNSUPPORTED for a d_in
 * that is not a positive multiple of LORA_SHRINK_TILE_K, or r_max above 64.
 *
 * lora_sgmv_shrink_tiled_workspace: bytes of workspace for k_splits
 * (k_splits * num_perm * r_max floats; 0 when k_splits == 1).
 *
 * lora_sgmv_shrink_tiled: runs the plan; k_splits must be the plan's (the
 * slices are recomputed from d_in and k_splits).  workspace: caller-owned
 * device memory, 16-byte aligned, of at least the size above (contents on
 * entry do not matter; NULL with 0 bytes when k_splits == 1); calls that
 * share it must not overlap (on one stream they do not).  Errors: as
 * lora_sgmv_shrink; LORA_EUNSUPPORTED unless activations are bf16, r_max <=
 * 64 and d_in is a multiple of LORA_SHRINK_TILE_K; LORA_EINVAL for
 * k_splits out of range or leaving an empty slice, or a missing, misaligned
 * or short workspace.                                                        */
#define LORA_PATH_TILE 3                    /* plan items only: a tiled shrink item */
#define LORA_SHRINK_TILE_TOKENS 64
#define LORA_SHRINK_TILE_K 64               /* slices are multiples of this many elements */
#define LORA_SHRINK_TILE_ITEM_BYTES 262144  /* bytes of x and A an item aims to read */
#define LORA_DEFAULT_TILE_MIN_TOKENS 16
#define LORA_TILE_MIN_RANK_SHORT 32
#define LORA_MAX_K_SPLITS 64
#define LORA_TILE_PAYS_BYTES (24 << 20)    /* compute-unit bytes a tiled shrink must save */
lora_status lora_sgmv_plan_tiled(const int32_t *seg_starts, const int32_t *seg_adapter,
                                 int32_t num_segments, int32_t num_adapters,
                                 const int32_t *host_rank, int32_t r_max, int32_t d_in,
                                 int32_t path_policy, int32_t tile_min_tokens, int32_t max_splits,
                                 lora_item *items, int32_t capacity, int32_t *num_items,
                                 int32_t *k_splits);
lora_status lora_sgmv_shrink_tiled_workspace(int32_t num_perm, int32_t r_max, int32_t k_splits,
                                             int64_t *bytes);
/* lora_sgmv_tiled_pays: whether to prefer the tiled shrink for a batch (host
 * only).  *pays = 1 when lora_sgmv_shrink_tiled accepts the weights (dtype
 * LORA_BF16, any weight_format, r_max <= 64, d_in a positive multiple of
 * LORA_SHRINK_TILE_K) and its tile items, planned under the AUTO
 * policy, would read at least LORA_TILE_PAYS_BYTES fewer bytes through the
 * compute units than the items of lora_sgmv_plan (A rows once per 64 tokens
 * instead of once per 16, x rows once instead of once per row group): about
 * what the second launch costs.  Else 0 (batches of short low-rank segments,
 * such as decode tokens, or short d_in).  Arguments as lora_sgmv_plan_tiled
 * (host_rank may be NULL: every adapter at r_max); errors as lora_sgmv_plan. */
lora_status lora_sgmv_tiled_pays(const int32_t *seg_starts, const int32_t *seg_adapter,
                                 int32_t num_segments, int32_t num_adapters, const int32_t *host_rank,
                                 int32_t r_max, int32_t d_in, int32_t dtype, int32_t weight_format,
                                 int32_t tile_min_tokens, int32_t *pays);
lora_status lora_sgmv_shrink_tiled(const lora_weights *w, const int32_t *token_perm,
                                   int32_t num_perm, const lora_item *items, int32_t num_items,
                                   int32_t num_tokens, int32_t k_splits, const void *x, float *v,
                                   void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Per-token (BGMV, decode) mode: adapter ids stay on the device, no host
 * planning and no host synchronisation; every token takes the gather/GEMV path
 * (S-LoRA's decode kernel, MBGMV, in the same section: mixed ranks in one
 * batch).  Same arithmetic as the segmented calls.
 *   token_adapter [num_tokens]  device; ids outside [0, N) (and -1) are skipped
 *   order  LORA_BGMV_TOKEN_MAJOR: workgroups per token (shrink: one per
 *          group of 2 rows of A; expand: one per block of 1024 columns);
 *          LORA_BGMV_ADAPTER_MAJOR: the same split per adapter, each workgroup
 *          scanning token_adapter for its adapter's tokens, so each adapter's
 *          rows are read once however many tokens use it;
 *          LORA_BGMV_AUTO: shrink adapter-major when num_adapters <= num_tokens
 *          <= 4 num_adapters, otherwise token-major; expand token-major.
 *          Every order gives bit-identical results.                        */
#define LORA_BGMV_AUTO 0
#define LORA_BGMV_TOKEN_MAJOR 1
#define LORA_BGMV_ADAPTER_MAJOR 2
lora_status lora_bgmv_shrink(const lora_weights *w, const int32_t *token_adapter,
                             int32_t num_tokens, int32_t order, const void *x, float *v,
                             hipStream_t stream);
lora_status lora_bgmv_expand(const lora_weights *w, const int32_t *token_adapter,
                             int32_t num_tokens, int32_t order, const float *v, void *y,
                             hipStream_t stream);

/* Per-token (BGMV) delta in ONE launch: shrink and expand of each token fused
 * in one workgroup (S-LoRA's decode kernel MBGMV in "Multi-LoRA serving ...",
 * section "SGMV: the kernel that holds it all up"; the launch and gather
 * overhead per adapted layer that the glossary entry "Multi-LoRA Serving",
 * section "Limits and open questions", attributes to unmerged adapters).
 * Computes y[t] += B_{a(t)} (A_{a(t)} x[t]) for every token with the same
 * arithmetic as lora_bgmv_shrink + lora_bgmv_expand (fp32 v, one rounding of
 * y); v [num_tokens, r_max] receives the rank-space values when non-NULL.
 * The fused and two-launch paths sum in different orders, so their results
 * agree to rounding, not bit for bit; the fused path's orders and placements
 * all give identical bits.  token_adapter, x, y as for lora_bgmv_shrink/expand.
 *   token_order [num_ordered]  device, or NULL.  Token-major order only: the
 *          tokens to process, in placement order (each an index in
 *          [0, num_tokens); others are skipped; tokens not listed keep their y).
 *          Each token may be listed at most once: a token listed twice is
 *          updated by two workgroups that race on its y row (the token_perm
 *          of lora_segments_build lists every token once).
 *          Consecutive entries run on the same XCD and share its L2, so an
 *          order that groups the tokens of each adapter -- the token_perm of
 *          lora_segments_build, built once per batch on the host and reused by
 *          every layer, like a plan -- reads each adapter's rows from memory
 *          about once instead of once per token.  NULL: every token, in index
 *          order (no host step; adapter ids stay on the device).
 *   order  LORA_BGMV_TOKEN_MAJOR (and LORA_BGMV_AUTO): one workgroup per
 *          token and column block;
 *          LORA_BGMV_ADAPTER_MAJOR: one workgroup per adapter and column block,
 *          finding its tokens by scanning token_adapter and processing them
 *          four at a time (for few tokens per adapter); token_order ignored.
 * Errors as for lora_bgmv_shrink, and LORA_EINVAL for num_ordered outside
 * 0..num_tokens with a token_order.                                        */
lora_status lora_bgmv_fused(const lora_weights *w, const int32_t *token_adapter,
                            int32_t num_tokens, const int32_t *token_order,
                            int32_t num_ordered, int32_t order, const void *x, float *v,
                            void *y, hipStream_t stream);

/* Several projections of the same input in ONE fused launch: the q, k and v
 * (or gate and up) projections of a layer, each with its own adapter matrices
 * (w[p]) and output (y[p] [num_tokens, w[p]->d_out]; v[p] optional, as for
 * lora_bgmv_fused), all reading x ("Multi-LoRA serving ...", section "The
 * maths that matters": every targeted projection of a layer carries its own
 * A and B; x is shared).  The work units of one token are placed on one XCD,
 * so x crosses the fabric once for all projections, and one launch replaces
 * num_proj.  Per projection the arithmetic is lora_bgmv_fused's (token-major),
 * so the bits equal those of separate lora_bgmv_fused calls.  It pays where
 * launches dominate (small decode batches: 2.6x for q/k/v of a 70B layer at
 * 32 tokens); at 256 tokens separate launches balance better (0.97x).
 *   w [num_proj]  host array of descriptors with equal dtype, weight_format,
 *                 d_in and num_adapters (their d_out may differ); num_proj in 1..4
 *   v [num_proj]  host array of device pointers (entries may be NULL), or NULL
 *   y [num_proj]  host array of device pointers
 *   token_adapter, token_order, num_ordered, x as for lora_bgmv_fused.
 * Errors: as lora_bgmv_fused; LORA_EINVAL for num_proj or mismatched
 * descriptors.                                                            */
lora_status lora_bgmv_fused_multi(const lora_weights *const *w, int32_t num_proj,
                                  const int32_t *token_adapter, int32_t num_tokens,
                                  const int32_t *token_order, int32_t num_ordered, const void *x,
                                  float *const *v, void *const *y, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Paged adapter pool (host bookkeeping over caller-owned device storage of
 * [num_pages][page_rows] rows of row_width elements in the given dtype and
 * weight_format (row bytes as for lora_weights), plus, for the quantized
 * formats, caller-owned device row scales [num_pages * page_rows] that must be
 * NULL otherwise).  Pages are handed out from a
 * free list shuffled by `shuffle_seed` (0 = in order), so an adapter's pages
 * are scattered through the pool as they are after churn; freed pages return
 * to the back of the list.  Sources: the unified paging of adapter weights
 * ("Multi-LoRA serving ..." TL;DR; section "Operational pitfalls", memory
 * fragmentation) and the fixed-size adapter pool of "Multi-LoRA Inference
 * Serving" (clusterbid.com).  A lora_pool object is not thread-safe.        */
typedef struct lora_pool lora_pool;
lora_status lora_pool_create(int32_t num_pages, int32_t page_rows, int32_t row_width,
                             int32_t dtype, int32_t weight_format, void *device_storage,
                             float *device_scales, uint64_t shuffle_seed, lora_pool **out);
/* Takes ceil(rows / page_rows) pages; ids written to page_ids.  LORA_ENOMEM if
 * too few pages are free (nothing taken). */
lora_status lora_pool_alloc(lora_pool *pool, int32_t rows, int32_t *page_ids);
/* Returns pages to the pool.  LORA_EINVAL on an id that is not currently taken
 * (nothing freed). */
lora_status lora_pool_free(lora_pool *pool, const int32_t *page_ids, int32_t num_pages);
lora_status lora_pool_num_free(const lora_pool *pool, int32_t *num_free);
/* Copies `rows` stored rows from src (host or device memory) into the pages,
 * page_rows rows per page, and for a quantized pool their `rows` scales from
 * src_scales (NULL for a plain pool), asynchronously on `stream`.  Host
 * sources must stay valid until the stream has passed this point. */
lora_status lora_pool_write_rows(lora_pool *pool, const int32_t *page_ids, int32_t rows,
                                 const void *src, const float *src_scales, hipStream_t stream);
void lora_pool_destroy(lora_pool *pool);
/* The pool's geometry as created (any output may be NULL). */
lora_status lora_pool_info(const lora_pool *pool, int32_t *num_pages, int32_t *page_rows,
                           int32_t *row_width, int32_t *dtype, int32_t *weight_format);

/* ------------------------------------------------------------------------ */
/* Adapter residency: an LRU cache of adapters over two page pools (A rows and
 * B^T rows; the same pool twice when d_in == d_out), filled from caller-owned
 * host copies -- the hot HBM pool and warm host tier of "Multi-LoRA serving
 * ..." (TL;DR; section "Operational pitfalls": cold start, fragmentation; its
 * figure of the serving stack: LRU eviction, asynchronous host-to-device copy
 * on use) and the fixed-size adapter pool of "Multi-LoRA Inference Serving"
 * (clusterbid.com, vLLM paragraph: adapters swapped in and out as requests
 * arrive).  The cache owns the contents of three caller-owned device arrays
 * that a lora_weights descriptor then names: page tables [num_ids][max_pages]
 * (max_pages = ceil(r_max / page_rows)) and ranks [num_ids], where num_ids is
 * the size of the adapter id space (resident or not).  Non-resident adapters
 * have page ids -1 and rank 0 there.  A lora_cache is not thread-safe.
 *
 * lora_cache_prepare makes every adapter of a batch resident before the
 * batch's kernels run on `compute`: misses take pages (evicting the least
 * recently used adapters the batch does not use, those whose last batch has
 * completed before those still in flight), their rows, row scales,
 * page-table rows and ranks are copied on the cache's own stream, and
 * `compute` waits for those copies with an event (the call itself does not
 * block).  A page freed by an eviction is rewritten only once the last batch
 * that used the evicted adapter has completed on `compute`; use one compute
 * stream per cache.  Host rows must stay valid and unchanged while their
 * adapter is registered; pinned host memory (hipHostMalloc) lets the copies
 * run on the DMA engines alongside the kernels.                             */
#define LORA_CACHE_HOST_ONLY 1  /* flag: bookkeeping only, no device work (tests) */
typedef struct lora_cache lora_cache;
typedef struct {
  int64_t hits;            /* batch adapters found resident (cumulative) */
  int64_t misses;          /* batch adapters uploaded (cumulative) */
  int64_t evictions;       /* adapters evicted (cumulative) */
  int64_t bytes_uploaded;  /* rows and row scales copied to the pools (cumulative) */
  int32_t resident;        /* adapters resident now */
  int32_t scattered;       /* resident adapters whose pages are not consecutive ids */
  int32_t free_pages_a, free_pages_b;
} lora_cache_stats;
/* Errors: LORA_EINVAL (null pointer, unknown flag, pools of different page
 * size, dtype or format), LORA_EUNSUPPORTED (r_max), LORA_EHIP. */
lora_status lora_cache_create(lora_pool *pool_a, lora_pool *pool_b, int32_t num_ids, int32_t r_max,
                              int32_t *device_page_table_a, int32_t *device_page_table_b,
                              int32_t *device_rank, int32_t flags, lora_cache **out);
/* Host copies of adapter `id`: rank rows of A (d_in) and of B^T (d_out) in the
 * pools' format, and for quantized pools their row scales (else NULL).
 * Errors: LORA_ERANGE (id or rank), LORA_EINVAL (null rows, scales that do
 * not match the format, a resident adapter). */
lora_status lora_cache_register(lora_cache *cache, int32_t id, int32_t rank,
                                const void *host_a_rows, const void *host_b_rows,
                                const float *host_a_scales, const float *host_b_scales);
/* ids [n] host (-1 entries skipped).  Errors: LORA_ERANGE (an id outside the
 * space or not registered), LORA_ENOMEM (the batch's adapters alone exceed
 * the pools; nothing changed), LORA_EHIP. */
lora_status lora_cache_prepare(lora_cache *cache, const int32_t *ids, int32_t n, hipStream_t compute);
lora_status lora_cache_get_stats(const lora_cache *cache, lora_cache_stats *stats);
/* Page ids of a resident adapter (capacity max_pages each; NULL allowed);
 * *num_pages = 0 when it is not resident. */
lora_status lora_cache_pages(const lora_cache *cache, int32_t id, int32_t *pages_a,
                             int32_t *pages_b, int32_t *num_pages);
/* Waits for the cache's copies, then frees it (not the pools or arrays). */
void lora_cache_destroy(lora_cache *cache);

/* ------------------------------------------------------------------------ */
/* Base projection y = x W^T computed once for every token of the batch, the
 * term the adapters' deltas are added to ("Multi-LoRA serving ...", section
 * "The bare mechanism": Wx is computed only once for all the tokens; W in
 * R^{d_out x d_in}).  bf16 in, fp32 accumulation (MFMA), bf16 out rounded to
 * nearest even.
 *   x [m][k], w [n][k], y [m][n]: row-major device arrays; k, n multiples of 8.
 *   workspace, workspace_bytes: optional device memory owned by the caller
 *     (NULL / 0: none; 16-byte aligned).  When it holds the size that
 *     lora_base_gemm_workspace reports for the shape (grids too small to fill
 *     the device), k is cut into up to 4 slices whose fp32 partial tiles go
 *     there and are added in slice order by a second launch on the same
 *     stream; otherwise, or for a smaller workspace, k is not split.  The
 *     workspace must not be in use by other work on the device until the
 *     call's work on `stream` is done.
 * Errors: LORA_EINVAL (sizes, null or misaligned pointers, negative
 * workspace_bytes), LORA_EUNSUPPORTED (dtype other than LORA_BF16; n or k not
 * multiples of 8), LORA_EHIP. */
lora_status lora_base_gemm(int32_t dtype, int32_t m, int32_t n, int32_t k, const void *x,
                           const void *w, void *y, void *workspace, int64_t workspace_bytes,
                           hipStream_t stream);
/* Workspace bytes with which lora_base_gemm splits k for an m x n x k problem
 * on the current device (0: it would not split).  *bytes host.  Errors:
 * LORA_EINVAL (sizes, null bytes). */
lora_status lora_base_gemm_workspace(int32_t m, int32_t n, int32_t k, int64_t *bytes);

/* lora_base_gemm for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, arithmetic and results as
 * lora_base_gemm called with the workspace lora_base_gemm_workspace reports
 * (bit for bit: the same kernels and the same k split), but the split-k
 * partial tiles go to a scratch array the library holds in device memory:
 * LORA_BASE_GEMM_SCRATCH_BYTES (24 MiB) on every device it is called on, kept
 * until the process ends.  Nothing is allocated by the call (no hipMalloc, no
 * hipFree, no allocating library routine); the scratch's device address is
 * looked up once per device on the first call there.  Every call on one
 * device shares that device's scratch, and each split call overwrites every
 * partial it reads before reading it (nothing needs clearing), so calls that
 * overlap on one device -- on different streams, or on one stream from
 * several host threads without ordering -- race and give wrong results.
 * Errors: as lora_base_gemm, and LORA_ENOMEM when the shape's split needs
 * more partial-tile bytes than the scratch holds (not for any shape on a
 * device of up to 256 compute units, where the split rule stays within 24 MiB). */
#define LORA_BASE_GEMM_SCRATCH_BYTES (24 << 20)
lora_status lora_base_gemm_noalloc(int32_t dtype, int32_t m, int32_t n, int32_t k, const void *x,
                                   const void *w, void *y, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Debug build.  The library is also built as liblora_sgmv_debug.so, with
 * LORA_DEBUG: its kernels record the bad device-side values that every build
 * skips (see "Device-resident indices" above) as bits of a device word, and
 * still exit normally.  lora_debug_flags waits for the device's work (it reads
 * the word with a synchronous copy), stores the word in *flags and, when clear
 * is non-zero, resets it.  The word covers every call on the current device
 * since the last clear.  Release builds return LORA_EUNSUPPORTED (and *flags =
 * 0).  Errors: LORA_EINVAL (null flags), LORA_EHIP. */
#define LORA_DEBUG_BAD_PAGE 1u      /* a page id outside the pool for a row below the rank */
#define LORA_DEBUG_BAD_ADAPTER 2u   /* a device adapter id outside {-1} U [0, num_adapters) */
#define LORA_DEBUG_BAD_RANK 4u      /* a used adapter's rank outside 1..r_max */
#define LORA_DEBUG_BAD_TOKEN 8u     /* a token_perm entry outside [0, num_tokens) */
#define LORA_DEBUG_BAD_ITEM 16u     /* a plan item that names no valid tokens or adapter */
lora_status lora_debug_flags(uint32_t *flags, int32_t clear);

/* ------------------------------------------------------------------------ */
/* Measurement helper, not part of the delta path: a bare streaming read of
 * `groups` consecutive regions of bytes_per_group bytes of src, one workgroup
 * of `threads` threads per region (16-byte loads), writing nothing to sink
 * [groups] in practice.  The benchmark times it to show the floor that
 * launches of a given size and workgroup count cannot beat on the device.
 * src 16-byte aligned with groups * bytes_per_group readable bytes;
 * bytes_per_group a multiple of 16; threads a multiple of 64 in 64..1024;
 * nontemporal 1: the loads carry the non-temporal hint (0: plain loads).
 * Errors: LORA_EINVAL, LORA_EHIP. */
lora_status lora_probe_stream_read(const void *src, int64_t bytes_per_group, int32_t groups,
                                   int32_t threads, int32_t nontemporal, uint32_t *sink,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_SGMV_H */
