/*
 * sel_attn.h - C ABI of libselattn.so: prompt-phase selection attention over
 * INT8 paged K/V, hand-written HIP kernels for gfx950 (MI355X).
 *
 * Page cited: #2808 "sycl: prompt attention over 8-query selection unions on
 * XMX (opt-in STRATA_PROMPT_ATTN_UNION=1)".
 *
 * The method (section Summary): each query position attends only to the cells
 * it selected. Groups of 8 neighbouring positions share one sorted union of
 * their selections; every union cell carries a byte whose bit i says whether
 * position i of the group chose it (section Extra Notes: an int32 cell plus a
 * separate mask byte). K and V are INT8 behind a page table; 64-cell chunks of
 * the union are dequantised once and multiplied on matrix cores with FP32 sums
 * for all 96 rows of a group (8 positions x 12 query heads of one KV head); in
 * the online softmax a cell counts as -inf for the positions that did not
 * choose it, so every position attends to exactly its own cells.
 *
 * One pass of the path is two calls on one stream:
 *   sel_attn_build_union  selections + page table -> per-group union, masks,
 *                         pool rows (each cell's page resolved once), lengths
 *   sel_attn_prefill      union rows and masks + q + INT8 K/V pools -> output
 * (sel_attn_prefill_split: the same attention for grids too small to fill the
 * GPU, over a caller-owned workspace)
 * and the step before it, when the selections come from block scores:
 *   sel_attn_select_blocks  block scores -> per-position selections
 * For batches whose neighbouring selections hardly overlap, one call does the
 * same attention without a union:
 *   sel_attn_prefill_positions  selections + q + paged INT8 K/V -> output
 * and for decode (one position, or a short speculative verify window), the
 * same attention split over each position's cells:
 *   sel_attn_decode             selections + q + paged INT8 K/V -> output
 * (sel_attn_decode_noalloc: the same for callers that cannot allocate).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array pointers are DEVICE pointers owned by the caller. The library
 *   allocates no device memory, keeps no state between calls except a cached
 *   per-device architecture check (and, for sel_attn_decode_noalloc, a static
 *   device array and its per-device address), and enqueues its kernels
 *   asynchronously on `stream` (NULL = the null stream). Inputs are only read.
 * - Return value: SEL_ATTN_OK when the kernels were enqueued; a negative code
 *   when nothing was enqueued. sel_attn_last_error() then describes why.
 * - Errors that need the data to detect (a cell out of range, a bad length, a
 *   page-table entry past the pool) cannot be returned synchronously. The
 *   kernels OR SEL_ATTN_STATUS_* bits into *status (a device uint32 that the
 *   caller zeroes beforehand and reads after synchronising the stream). Outputs
 *   of the groups concerned are then unspecified, but every access stays in
 *   bounds.
 * - Calls are deterministic: identical inputs give bitwise-identical outputs.
 *   Calls on different streams that write different outputs may overlap.
 */
#ifndef SEL_ATTN_H_
#define SEL_ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SEL_ATTN_OK 0
#define SEL_ATTN_EINVAL (-1)       /* null or misaligned pointer, or a size out of range */
#define SEL_ATTN_EUNSUPPORTED (-2) /* a shape the library does not implement, or a device that is not gfx950 */
#define SEL_ATTN_ELAUNCH (-3)      /* a HIP call failed (device query or kernel launch) */

/* Bits the kernels OR into *status. */
#define SEL_ATTN_STATUS_CELL_RANGE 1u  /* a selected cell outside [0, n_ctx) */
#define SEL_ATTN_STATUS_SEL_LEN 2u     /* sel_len[j] outside [0, sel_cap] */
#define SEL_ATTN_STATUS_PAGE_RANGE 4u  /* page_table entry >= n_pages (or < -1), or a union
                                          row past the pools */
#define SEL_ATTN_STATUS_UNION_LEN 8u   /* union_len[g] outside [0, 8*sel_cap] */
#define SEL_ATTN_STATUS_V_SCALE 16u    /* a v_scale of a used cell with |v_scale| >= 4 or not finite */

/* Shapes the library implements. */
#define SEL_ATTN_HEAD_DIM 128
#define SEL_ATTN_PAGE_SIZE 64
#define SEL_ATTN_Q_PER_KV 12
#define SEL_ATTN_GROUP 8           /* positions per union group */
#define SEL_ATTN_SINKS 3           /* sink cells 0, 1, 2 in every selection */
#define SEL_ATTN_TOP_BLOCKS 31     /* earlier blocks a selection takes by score */
#define SEL_ATTN_SEL_MAX 2051      /* 3 + 31*64 + 64: cells in a full selection */
#define SEL_ATTN_SELECT_MAX_CTX 262144 /* n_ctx limit of sel_attn_select_blocks */
#define SEL_ATTN_POSITIONS_MAX_CAP 2560  /* sel_cap limit of sel_attn_prefill_positions and decode */
#define SEL_ATTN_DECODE_MAX_Q 65535      /* n_q limit of sel_attn_decode (one grid dimension) */
#define SEL_ATTN_DECODE_NOALLOC_MAX_BYTES 8388608 /* static scratch of sel_attn_decode_noalloc (8 MiB) */

typedef struct sel_attn_dims {
  int32_t n_ctx;     /* logical context length in cells, >= 1; page_table has
                        ceil(n_ctx / page_size) entries */
  int32_t n_q;       /* query positions in this call, >= 0 (0 = nothing to do).
                        Group g holds query indices [8g, 8g+8) clipped to n_q; the
                        last group may be ragged. Groups start at query index 0. */
  int32_t n_kv;      /* KV heads, >= 1 */
  int32_t q_per_kv;  /* query heads per KV head; must be 12. Query head h reads
                        KV head h / 12 */
  int32_t head_dim;  /* must be 128 */
  int32_t page_size; /* cells per page; must be 64 */
  int32_t sel_cap;   /* row stride of sel, >= 1 (2051 in the headline workloads);
                        each group's union rows have stride 8 * sel_cap */
  int32_t n_pages;   /* physical pages in each pool, >= 1; a pool
                        (n_pages * n_kv * 64 * 128 bytes) must stay under 4 GiB */
} sel_attn_dims;

/*
 * sel_attn_select_blocks - the selection step before the path (section What
 * changed: the selection, block scores then top-k, which the page leaves as it
 * is; the accuracy list in section Summary: a selection holds at most 2,051
 * cells). The page does
 * not say how blocks are scored; the scores are an input.
 *
 *   first_pos     position of query index 0; query index j is at position
 *                 p = first_pos + j, and 0 <= first_pos, first_pos + n_q <= n_ctx
 *   block_scores  const float [n_q][ceil(n_ctx/64)]  row j scores the blocks
 *                 before p's own block, floor(p/64); later entries are not read
 *   sel           int32 [n_q][sel_cap]   out: row j in ascending order
 *   sel_len       int32 [n_q]            out: cells in row j
 *   Row j is the sink cells {0, 1, 2}, the 31 earlier blocks (64 cells each)
 *   with the highest scores, and the own block's cells up to p. A position with
 *   at most 31 earlier blocks takes all of them: its row is [0, p]. Equal scores
 *   go to the lower block index first; a NaN score counts as -inf; -0.0 equals
 *   +0.0. Each cell appears once (the sinks lie inside block 0 when it is
 *   chosen), so sel_len[j] <= 2051. Entries past sel_len[j] are left untouched.
 *   The output feeds sel_attn_build_union with the same dims.
 *   Errors (nothing enqueued): sel_cap < 2051 or positions outside [0, n_ctx)
 *   give EINVAL; n_ctx > SEL_ATTN_SELECT_MAX_CTX gives EUNSUPPORTED. The
 *   n_kv and n_pages fields are checked as for the other calls but not used.
 *   Alignment: 4 bytes for every array.
 */
int sel_attn_select_blocks(const sel_attn_dims* d, int32_t first_pos, const float* block_scores,
                           int32_t* sel, int32_t* sel_len, hipStream_t stream);

/*
 * sel_attn_build_union - the union step (section Summary: per group of 8
 * adjacent positions, one sorted list of every cell any of them selected, each
 * entry tagged with which of the 8 selected it; section What changed: one
 * work-group per 8 positions with local bitmaps; section Extra Notes: cells of
 * pages that are not resident are masked). Each union cell is also resolved
 * through the page table here, once, rather than by every KV head's work-group
 * of sel_attn_prefill.
 *
 *   sel          const int32 [n_q][sel_cap]   selected logical cells of each
 *                                             query index; any order, repeats
 *                                             allowed (a cell counts once)
 *   sel_len      const int32 [n_q]            valid entries of each row
 *   page_table   const int32 [ceil(n_ctx/64)] physical page of each logical
 *                                             page; -1 = not resident
 *   union_cells  int32 [G][8*sel_cap]         out: ascending distinct cells of
 *                                             group g in [0, union_len[g])
 *   union_mask   uint8 [G][8*sel_cap]         out: bit i set iff query index
 *                                             8g+i chose the cell
 *   union_rows   int32 [G][8*sel_cap]         out: the cell's pool row for KV
 *                                             head 0, p * n_kv * 64 + c % 64
 *                                             with p = page_table[c / 64]
 *                                             (KV head h's row is that + 64 h,
 *                                             in the [n_pages][n_kv][64] order
 *                                             of the pools and scales); -1 when
 *                                             the page is not resident
 *   union_len    int32 [G]                    out: size of group g's union
 *   status       uint32 [1]                   in/out: OR of SEL_ATTN_STATUS_*
 *   G = ceil(n_q / 8). Entries past union_len[g] are left untouched. The cells
 *   and masks depend on the selections alone; only the rows read the table.
 *   Errors: a cell outside [0, n_ctx) is dropped and sets CELL_RANGE; a length
 *   outside [0, sel_cap] is clamped and sets SEL_LEN; a page-table entry of a
 *   union cell outside [-1, n_pages) sets PAGE_RANGE and gives row -1.
 *   Alignment: 4 bytes for the int32 arrays.
 */
int sel_attn_build_union(const sel_attn_dims* d, const int32_t* sel, const int32_t* sel_len,
                         const int32_t* page_table, int32_t* union_cells, uint8_t* union_mask,
                         int32_t* union_rows, int32_t* union_len, uint32_t* status,
                         hipStream_t stream);

/*
 * sel_attn_prefill - the attention step over each group's union (section
 * Summary: INT8 K/V of 64-cell chunks of the union dequantised once, S^T = K Q^T
 * and O += P V on matrix cores with FP32 sums for the group's 96 rows, cells the
 * row's position did not choose set to -inf in the online softmax; section
 * What changed: one work-group per group of 8 positions and KV head; section
 * Extra Notes: cells of pages that are not resident are masked for everyone).
 *
 *   q            const float [n_q][n_kv*12][128]        queries (rounded to
 *                                                       FP16 for the products)
 *   k_pool       const int8  [n_pages][n_kv][64][128]   keys, page-major, then
 *   v_pool       const int8  [n_pages][n_kv][64][128]   KV head, cell, dim
 *   k_scale      const float [n_pages][n_kv][64]        per cell and KV head:
 *   v_scale      const float [n_pages][n_kv][64]        k = k_int8 * k_scale
 *   union_rows, union_mask, union_len                   as written by
 *                                                       sel_attn_build_union
 *                                                       with the same dims; a
 *                                                       row of -1 is masked for
 *                                                       everyone
 *   softmax_scale                                       multiplies q.k (e.g.
 *                                                       1/sqrt(128))
 *   out          float [n_q][n_kv*12][128]              out: softmax-weighted
 *                                                       sum of dequantised V
 *                                                       over the position's own
 *                                                       resident cells; 0 when
 *                                                       it has none
 *   status       uint32 [1]                             in/out, as above
 *   Precision: both matrix products take their operands (Q, dequantised K, V
 *   and the probabilities) in FP16 (round to nearest even); scores, softmax and sums are FP32. K and V
 *   integers are exact in FP16; k_scale is applied to the FP32 score, v_scale
 *   as an FP16 factor (v_scale * 2^6) on the FP16 probability.
 *   Supported scales: |v_scale| < 4 (other values set V_SCALE); k_scale any
 *   finite value.
 *   Errors: UNION_LEN and V_SCALE as listed above; PAGE_RANGE for a row r
 *   other than -1 whose KV-head rows r + 64 h would leave the pools
 *   (r < 0 or r >= (n_pages * n_kv - n_kv + 1) * 64), and such a cell is
 *   treated as not resident. A row inside that range is read as given.
 *   Alignment: q, out, k_pool, v_pool 16 bytes; the rest 4 bytes (mask 1).
 */
int sel_attn_prefill(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                     const int8_t* v_pool, const float* k_scale, const float* v_scale,
                     const int32_t* union_rows, const uint8_t* union_mask,
                     const int32_t* union_len, float softmax_scale, float* out, uint32_t* status,
                     hipStream_t stream);

/*
 * sel_attn_prefill_workspace_bytes - device workspace that sel_attn_prefill_split
 * needs for these dims: groups x KV heads x splits x 49,920 bytes, with
 * splits = min(16, ceil(512 / (groups x KV heads)), floor(C / 12)), where
 * C = ceil(min(8 sel_cap, n_ctx) / 32) is the number of 32-cell chunks of the
 * longest union the dims allow; 0 when splits <= 1 (groups x KV heads already
 * give the GPU 512 work-groups, or the unions are too short to share out), and
 * the call then runs exactly as sel_attn_prefill.
 */
size_t sel_attn_prefill_workspace_bytes(const sel_attn_dims* d);

/*
 * sel_attn_prefill_split - sel_attn_prefill for grids too small to fill the GPU
 * (the same attention over the same unions, section Summary). Each group's
 * union is divided at 32-cell chunk boundaries over `splits` work-groups, each
 * of which runs the same online softmax over its share and writes its
 * unnormalised state (running maximum, probability sum, O) to the workspace; a
 * second kernel merges the shares of every row (weights exp2(m_s - max m)) and
 * writes out. Results agree with sel_attn_prefill's to rounding, not bitwise
 * (the sums are grouped differently); they are deterministic.
 *
 *   arguments    as for sel_attn_prefill, plus:
 *   workspace    device memory of at least workspace_bytes =
 *                sel_attn_prefill_workspace_bytes(d), 16-byte aligned, owned by
 *                the caller; may be NULL when that size is 0. Calls that run
 *                at the same time need workspaces of their own.
 *   Errors: as sel_attn_prefill; a workspace that is NULL, too small or
 *   misaligned while one is needed gives EINVAL.
 */
int sel_attn_prefill_split(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                           const int8_t* v_pool, const float* k_scale, const float* v_scale,
                           const int32_t* union_rows, const uint8_t* union_mask,
                           const int32_t* union_len, float softmax_scale, float* out,
                           uint32_t* status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * sel_attn_prefill_positions - the same attention as sel_attn_build_union +
 * sel_attn_prefill, computed per position with no union: every position
 * gathers its own selected cells (section Summary: the FP32 kernel in which
 * every position gathers its own ~2,051 cells defines what is computed;
 * section Extra Notes: the union path wins only where adjacent positions'
 * selections share cells, and gains nothing when they are unrelated). Pick this call
 * when the union of 8 neighbours is several times one selection.
 *
 *   q, k_pool, v_pool, k_scale, v_scale, softmax_scale, out, status
 *                as for sel_attn_prefill
 *   page_table   const int32 [ceil(n_ctx/64)]: physical page of each logical
 *                page; -1 = not resident
 *   sel, sel_len as for sel_attn_build_union: any order, repeats count once
 *   Precision: the products take Q, K, V and P' = p * v_scale * 2^6 in FP16
 *   (round to nearest even); scores, softmax and sums are FP32. Results agree
 *   with sel_attn_prefill's to rounding, not bitwise; they depend on the order
 *   of each row's entries only through rounding, and identical inputs give
 *   bitwise-identical outputs.
 *   Errors: CELL_RANGE (the cell is dropped), SEL_LEN (clamped), PAGE_RANGE
 *   (treated as not resident), V_SCALE (|v_scale| >= 4: the cell's value
 *   counts as 0). sel_cap > SEL_ATTN_POSITIONS_MAX_CAP gives EUNSUPPORTED.
 *   Alignment: q, out, k_pool, v_pool 16 bytes; the rest 4 bytes.
 */
int sel_attn_prefill_positions(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                               const int8_t* v_pool, const float* k_scale, const float* v_scale,
                               const int32_t* page_table, const int32_t* sel,
                               const int32_t* sel_len, float softmax_scale, float* out,
                               uint32_t* status, hipStream_t stream);

/*
 * sel_attn_decode_workspace_bytes - device workspace that sel_attn_decode needs
 * for these dims: n_q * n_kv * ceil(sel_cap / 64) records of 6,272 bytes.
 * Returns 0 when the dims are invalid (sel_attn_decode then says why).
 */
size_t sel_attn_decode_workspace_bytes(const sel_attn_dims* d);

/*
 * sel_attn_decode - the attention of sel_attn_prefill_positions for a few
 * positions (decode, or a speculative verify window), each position's cells
 * split into pieces of 64 so that one position occupies dozens of work-groups.
 * The page leaves decode as it is (section Summary: decode tok/s and the verify
 * window's time are unchanged); this is the same definition as the prompt path
 * (section Summary: every position attends to exactly its own cells), for the
 * decode workload.
 *
 *   arguments as for sel_attn_prefill_positions, plus
 *   workspace        device memory of at least workspace_bytes =
 *                    sel_attn_decode_workspace_bytes(d), 16-byte aligned,
 *                    owned by the caller; overwritten by the call, so calls
 *                    that run at the same time need workspaces of their own
 *   Two kernels on `stream`: the splits, then their merge. Results agree with
 *   sel_attn_prefill_positions to rounding; identical inputs give identical
 *   bits. Meant for small n_q: every split repeats its position's dedup.
 *   Errors: as sel_attn_prefill_positions; a workspace that is NULL, too small
 *   or misaligned, or n_q > SEL_ATTN_DECODE_MAX_Q, gives EINVAL.
 */
int sel_attn_decode(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                    const int8_t* v_pool, const float* k_scale, const float* v_scale,
                    const int32_t* page_table, const int32_t* sel, const int32_t* sel_len,
                    float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                    uint32_t* status, hipStream_t stream);

/*
 * sel_attn_decode_noalloc - sel_attn_decode for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. It allocates nothing and
 * calls no allocating routine; the split records go to a static device array
 * of SEL_ATTN_DECODE_NOALLOC_MAX_BYTES that the library holds on every GPU it
 * runs on until the process ends (its address is looked up once per device,
 * on the first call there).
 *
 *   arguments as for sel_attn_decode, without the workspace
 *   The caller still provides q, the pools, scales, page table, selections,
 *   out and status. Outputs are bitwise identical to sel_attn_decode's for the
 *   same inputs (same kernels). Every call on one GPU shares that GPU's array
 *   and finds it as the last call left it (nothing in it has to start at
 *   zero): calls that overlap on one GPU (different streams, or several host
 *   threads) race and must be serialised by the caller.
 *   Errors: as sel_attn_decode; dims whose split records exceed the array
 *   (sel_attn_decode_workspace_bytes(d) > SEL_ATTN_DECODE_NOALLOC_MAX_BYTES,
 *   e.g. more than 8 positions x 4 KV heads at sel_cap 2,560) give EINVAL
 *   with nothing enqueued.
 */
int sel_attn_decode_noalloc(const sel_attn_dims* d, const float* q, const int8_t* k_pool,
                            const int8_t* v_pool, const float* k_scale, const float* v_scale,
                            const int32_t* page_table, const int32_t* sel, const int32_t* sel_len,
                            float softmax_scale, float* out, uint32_t* status,
                            hipStream_t stream);

/*
 * sel_attn_last_error - text describing the last nonzero return of an entry
 * point on the calling thread ("" if none). The pointer stays valid until the
 * thread's next call into the library.
 */
const char* sel_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SEL_ATTN_H_ */
