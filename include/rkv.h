/*
 * rkv.h -- C ABI of the retrieval-sparse paged decode attention library
 * for AMD MI355X (gfx950).
 *
 * The method (openGauss DataVec docs, "KV Cache Query-Based Computation
 * Inference Acceleration", section "Overall Solution"): each sequence's KV
 * cache is split into initial tokens, a sliding window and offload tokens;
 * every offload block of 128 tokens carries one key representation vector per
 * KV head; at each decode step the current query is scored against those
 * representations by inner product, the top ceil(ratio * n_offload) blocks are
 * kept, and softmax(q K^T / sqrt(d)) V runs over the initial, window and kept
 * blocks only.  The defaults come from the same page, section "Configuration
 * Parameters".  Paged K/V read through a block table follows the rkmt.cn ATB
 * KV-cache article, section 2.2 (PageAttention with a page table).
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless a parameter says "host".  The caller
 *    owns every buffer; the library allocates nothing and keeps no state
 *    between calls except the calling thread's last error text and, per
 *    device, its compute-unit count (queried once), the address of the
 *    static scratch array of rkv_decode_step_static and, once a copy-engine
 *    staging call asks for them (rkv_params.copy_lanes), its copy streams.
 *  - bf16 values travel as their 16-bit patterns (uint16_t).
 *  - All work is enqueued asynchronously on the given HIP stream; a call
 *    returns once the work is enqueued.  Arguments are validated on the host
 *    first: on any error status nothing is enqueued.
 *  - Outputs must not alias inputs.
 *  - Device-side values (lengths, page ids, counts) are clamped into range
 *    by the kernels so that bad values never cause an out-of-bounds access:
 *    a length above max_blocks * 128 is treated as max_blocks * 128, a
 *    negative length as 0, and a page id outside [0, n_pages) makes its block
 *    contribute nothing.  The debug build of the library (built with
 *    RKV_DEBUG) also reports the first such value: see rkv_debug_check.
 *
 * Memory layouts (part of the ABI):
 *  - k_pages: [n_pages][n_kv_heads][128 tokens][128 dims] bf16.  Each
 *    (page, head) slice is one contiguous 32 KiB tile, token-major.
 *  - v_pages: [n_pages][n_kv_heads][128 dims][128 tokens] bf16.  Each
 *    (page, head) slice is one contiguous 32 KiB tile, dim-major (the value
 *    tile is stored transposed so that the attention kernel reads the same
 *    token range of one dimension as 16 contiguous bytes).
 *  - block_table: [batch][max_blocks] int32, logical block -> page id.
 *  - lens: [batch] int32, current length L_b of each sequence, counting the
 *    token being decoded.
 *  - q: [batch][n_q_heads][128] bf16.  Query head g belongs to KV head
 *    g / (n_q_heads / n_kv_heads) (contiguous groups, as in grouped-query
 *    attention; CSDN "KV cache" survey, section "Share--KV cache共享").
 *  - reps: [batch][n_kv_heads][max_blocks][128] fp32, logical-indexed.
 *  - out: [batch][n_q_heads][128] fp32.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RKV_ABI_VERSION 6
#define RKV_BLOCK_SIZE 128
#define RKV_HEAD_DIM 128
#define RKV_PPM_ONE 1000000
#define RKV_MAX_GROUP 16        /* query heads per KV head */
#define RKV_MAX_COPY_LANES 8    /* rkv_params.copy_lanes */
#define RKV_MAX_BLOCKS 8192     /* blocks per sequence (1M tokens) */
/* Extent of one call, so that every launch grid fits the 32-bit work-item
 * count of a dispatch: batch * n_q_heads query rows, and batch * n_kv_heads
 * lists times the longest per-list row the call takes (max_blocks, m_cap,
 * k_cap, slot_cap).  Larger calls fail with RKV_ERR_UNSUPPORTED. */
#define RKV_MAX_QUERY_ROWS (1 << 18)
#define RKV_MAX_LIST_ENTRIES (1 << 23)

typedef enum rkv_status {
  RKV_OK = 0,
  RKV_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad value */
  RKV_ERR_UNSUPPORTED = 2,  /* block/head size != 128, group > 16, ... */
  RKV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  RKV_ERR_HIP = 4,          /* a HIP launch or copy failed; see rkv_last_error */
  RKV_ERR_BOUNDS = 5        /* debug builds: a kernel met an out-of-range device
                               value (see rkv_debug_check) */
} rkv_status;

/* Selection modes (rkv_params.select_mode, see rkv_select). */
#define RKV_SELECT_PER_HEAD 0
#define RKV_SELECT_PER_SEQUENCE 1

/* Attention kernel variants. */
#define RKV_ATTN_AUTO 0
#define RKV_ATTN_MFMA 1   /* query heads of a group packed against K tiles */
#define RKV_ATTN_VALU 2   /* vector-ALU dot products, same memory schedule */

/*
 * Method parameters.  Names follow the page's environment variables
 * (openGauss page, "Configuration Parameters").
 */
typedef struct rkv_params {
  int32_t block_size;      /* tokens per block; must be 128 */
  int32_t head_dim;        /* must be 128 */
  int32_t n_q_heads;       /* > 0, multiple of n_kv_heads */
  int32_t n_kv_heads;      /* > 0; n_q_heads / n_kv_heads <= 16 */
  int32_t init_tokens;     /* VLLM_RETRIEVAL_INIT_TOKENS_NUM, default 1024, >= 0 */
  int32_t local_tokens;    /* VLLM_RETRIEVAL_LOCAL_TOKENS_NUM, default 7192, >= 0 */
  int32_t topk_ppm;        /* VLLM_RETRIEVAL_TOPK_PERCENT in parts per million,
                              default 200000 (0.2); 0 .. 1000000 */
  int32_t dense_boundary;  /* VLLM_RETRIEVAL_DENSE_BOUNDARY, default 32768;
                              prompt_len < boundary attends to every block;
                              0 disables the dense switch */
  float scale;             /* softmax scale, default 1/sqrt(128) */
  int32_t attn_impl;       /* RKV_ATTN_AUTO / _MFMA / _VALU */
  int32_t split_waves;     /* waves the attention split is spread over,
                              at most 65536; 0 = auto (two per compute
                              unit: 512 on MI355X) */
  int32_t select_mode;     /* RKV_SELECT_PER_HEAD (default) or
                              RKV_SELECT_PER_SEQUENCE, see rkv_select */
  int32_t copy_lanes;      /* streams the copy-engine staging calls spread
                              their copies over: 0 or 1 (default 0) = the
                              caller's side stream only; 2 ..
                              RKV_MAX_COPY_LANES = that many streams of the
                              library's own, see rkv_stage_blocks_async */
} rkv_params;

/* Defaults of the page (init 1024, local 7192, ratio 0.2, dense boundary
 * 32K, block 128) for the given head counts; automatic attention variant
 * and split, per-head selection, copies on the side stream only. */
rkv_params rkv_params_default(int32_t n_q_heads, int32_t n_kv_heads);

int32_t rkv_abi_version(void);
const char* rkv_status_string(rkv_status status);
/* Text of the calling thread's last error ("" if none).  Valid until the
 * thread's next failing call. */
const char* rkv_last_error(void);

/*
 * rkv_build_reps -- block representation vectors (openGauss page, "Feature
 * Description" and "Overall Solution": representation vectors are extracted
 * block by block).  The representation of block j of sequence b at KV head h
 * is the fp32 mean of the block's 128 keys:
 *     reps[b][h][j][:] = (1/128) * sum_t K[block_table[b][j]][h][t][:]
 * It is written for every COMPLETE block j in [block_begin[b], floor(L_b/128));
 * the trailing partial block gets none.  Other entries of reps are untouched.
 *   k_pages      bf16 pool, layout above; n_pages pages
 *   block_table  [batch][max_blocks]
 *   lens         [batch] lengths L_b
 *   block_begin  [batch] first block to (re)build, or NULL for 0
 *   reps         [batch][n_kv_heads][max_blocks][128] fp32 output
 * Idempotent.  Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_HIP.
 */
rkv_status rkv_build_reps(const rkv_params* params, const uint16_t* k_pages,
                          int64_t n_pages, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* lens,
                          const int32_t* block_begin, int32_t batch,
                          float* reps, hipStream_t stream);

/*
 * rkv_append_kv -- write the decoded token's K and V (one autoregressive
 * step adds one token to the cache; rkmt.cn ATB article, section 1.1) into
 * slot L_b - 1 of its page, and, when that token completes its block and
 * reps is not NULL, write the block's representation as rkv_build_reps
 * would.  Sequences with L_b <= 0 are skipped.
 *   k_new, v_new [batch][n_kv_heads][128] bf16
 *   k_pages, v_pages updated in place; reps optional (NULL: no rep)
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_HIP.
 */
rkv_status rkv_append_kv(const rkv_params* params, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* k_pages,
                         uint16_t* v_pages, int64_t n_pages,
                         const int32_t* block_table, int32_t max_blocks,
                         const int32_t* lens, int32_t batch, float* reps,
                         hipStream_t stream);

/*
 * Workspace bytes rkv_select needs for these sizes (may be 0).
 */
size_t rkv_select_workspace_size(const rkv_params* params, int32_t batch,
                                 int32_t max_blocks);

/*
 * The smallest k_cap (kept ids per list) rkv_select and the calls built on
 * it accept for max_blocks blocks per sequence: max_blocks when a list can
 * be dense (dense_boundary > 0, or topk_ppm = RKV_PPM_ONE), otherwise
 * ceil(max_blocks * topk_ppm / RKV_PPM_ONE) (openGauss page, "Configuration
 * Parameters": the top-k ratio of the offload blocks, which never exceed
 * max_blocks).  0 for a NULL params or max_blocks < 0.
 */
int32_t rkv_topk_capacity(const rkv_params* params, int32_t max_blocks);

/*
 * rkv_select -- inner-product retrieval and block-table merge (openGauss
 * page, "Overall Solution": the IP between the current token's query and
 * every representation, the top-K closest blocks, joined with the initial
 * tokens and the sliding window).  For every (sequence b, KV head h):
 *   nb          = ceil(L/128)
 *   n_init      = min(ceil(init_tokens/128), nb)
 *   local_start = min(floor(max(L - local_tokens, 0)/128), nb - 1)
 *   offload     = blocks [n_init, local_start)  (n_off of them, maybe 0)
 *   score s_j   = sum over the group's query heads g of q[b][g] . reps[b][h][j]
 *   k           = n_off if prompt_len < dense_boundary or topk_ppm = 10^6,
 *                 else ceil(n_off * topk_ppm / 10^6)
 *   selected    = the k offload blocks with the largest s_j, ties to the
 *                 smaller block index, written in ascending order
 * With select_mode = RKV_SELECT_PER_SEQUENCE (the other reading of the
 * page's one record per block), s_j is summed over all KV heads of the
 * sequence (fp32, heads in order), one top-k runs per sequence and every
 * KV head gets the same selected blocks and the same merged list.
 * Outputs:
 *   sel_ids  [batch][n_kv_heads][k_cap] logical block ids (first n_sel valid);
 *            may be NULL only when k_cap is 0
 *   n_sel    [batch][n_kv_heads]
 *   merged   [batch][n_kv_heads][m_cap] PAGE ids of the attended blocks in
 *            ascending logical order: init, selected, then local blocks
 *            (optional: NULL skips the merge)
 *   n_merged [batch][n_kv_heads] (required when merged is given)
 * prompt_lens [batch] may be NULL (then the dense switch uses lens).
 * workspace >= rkv_select_workspace_size(params, batch, max_blocks) bytes
 * (the scores, one fp32 per (b, h, block)); calls that overlap on one
 * workspace race.  Two launches: a scoring pass spread over many compute
 * units, then one top-k + merge workgroup per (b, h) (per b in the
 * per-sequence mode).
 * Capacity rules, checked on the host: k_cap >= max_blocks when the dense
 * switch can fire (dense_boundary > 0 or topk_ppm = 10^6), else
 * k_cap >= ceil(max_blocks * topk_ppm / 10^6); m_cap >= max_blocks.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
rkv_status rkv_select(const rkv_params* params, const uint16_t* q,
                      const float* reps, const int32_t* block_table,
                      const int32_t* lens, const int32_t* prompt_lens,
                      int32_t batch, int32_t max_blocks, int32_t* sel_ids,
                      int32_t* n_sel, int32_t k_cap, int32_t* merged,
                      int32_t* n_merged, int32_t m_cap, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * rkv_append_select -- rkv_append_kv followed by rkv_select, with the
 * append folded into the selection's scoring launch (same arguments and
 * results as the two calls in that order; reps is written for a block the
 * appended token completes).  The selection never reads the appended token
 * or that block's representation: the block holding slot L - 1 is the
 * sequence's last, which is always local.  For a decode step this saves one
 * launch and its memory round trips.
 * Errors: as rkv_append_kv and rkv_select.
 */
rkv_status rkv_append_select(const rkv_params* params, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* k_pages,
                             uint16_t* v_pages, int64_t n_pages,
                             const uint16_t* q, float* reps,
                             const int32_t* block_table, const int32_t* lens,
                             const int32_t* prompt_lens, int32_t batch,
                             int32_t max_blocks, int32_t* sel_ids,
                             int32_t* n_sel, int32_t k_cap, int32_t* merged,
                             int32_t* n_merged, int32_t m_cap, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * rkv_merge_table -- the merge step of rkv_select on its own: builds merged /
 * n_merged from given selections (sel_ids / n_sel, logical ids ascending,
 * all inside the offload range) with the region rule above.  Init and local
 * blocks come from block_table.  host_table ([batch][max_blocks] device
 * int32, or NULL) marks blocks kept in host memory (entry >= 0): the r-th
 * kept block of sequence b, when it is such a block, is taken to live at
 * page stage_page0 + b * k_cap + r (the staging pages rkv_stage_blocks
 * fills); every other block comes from block_table.  Ids outside the offload
 * range are written as page -1, which rkv_decode_attn skips.
 * Same capacity rule for m_cap.  Errors as rkv_select.
 */
rkv_status rkv_merge_table(const rkv_params* params, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* lens,
                           const int32_t* sel_ids, const int32_t* n_sel,
                           int32_t k_cap, int32_t batch,
                           const int32_t* host_table, int64_t stage_page0,
                           int32_t* merged, int32_t* n_merged, int32_t m_cap,
                           hipStream_t stream);

/*
 * rkv_stage_blocks -- host tier (openGauss page, "Feature Description" and
 * "Overall Solution": the offload part of the KV cache is kept in host DDR
 * and the blocks selected at a decode round are loaded into HBM before
 * attention; "Configuration Parameters": prompts beyond the offload boundary
 * keep their offload region on the host).
 * For every (b, h) and r < min(n_sel[b][h], k_cap): copies the K tile and the
 * V tile of head h of logical block j = sel_ids[b][h][r] from host page
 * host_table[b][j] of the host pools to page stage_page0 + b * k_cap + r of
 * the device pools (head h's slice only).  One kernel reads the host pools
 * directly over the bus; no host round trip is needed for the ids.
 *   host_k, host_v  HOST pointers to pinned, device-mapped memory (e.g.
 *                   hipHostMalloc), n_host_pages pages, same tile layouts as
 *                   k_pages / v_pages; checked on the host
 *   host_table      [batch][max_blocks] device int32: host page of each
 *                   block, -1 when the block is not in host memory (such
 *                   entries, and ids outside [0, max_blocks), copy nothing)
 *   sel_ids, n_sel  as written by rkv_select
 *   k_pages, v_pages device pools of n_pages pages; pages
 *                   [stage_page0, stage_page0 + batch * k_cap) are the
 *                   staging area and must lie inside the pool
 * Errors: RKV_ERR_INVALID_ARG (including host pools that are not pinned and
 * mapped), RKV_ERR_UNSUPPORTED, RKV_ERR_HIP.
 */
rkv_status rkv_stage_blocks(const rkv_params* params, const uint16_t* host_k,
                            const uint16_t* host_v, int64_t n_host_pages,
                            const int32_t* host_table, int32_t max_blocks,
                            const int32_t* sel_ids, const int32_t* n_sel,
                            int32_t k_cap, int32_t batch, uint16_t* k_pages,
                            uint16_t* v_pages, int64_t n_pages,
                            int64_t stage_page0, hipStream_t stream);

/*
 * rkv_offload_blocks -- prefill-time move of the offload region into the
 * host tier (openGauss page, "Feature Description" and "Configuration
 * Parameters": beyond the offload boundary the offload part of the KV cache
 * is kept in host DDR; "Overall Solution": representations are extracted
 * block by block at prefill, so rkv_build_reps over the same pages may run
 * on another stream meanwhile -- both only read the device pages -- though
 * on MI355X that is slower than running them one after the other: while a
 * kernel writes host memory over the bus, HBM reads elsewhere stall).
 * For every sequence b and every block j of its offload range
 * [n_init, local_start) (region rule of rkv_select, from lens[b]) with
 * host_table[b][j] >= 0: copies all KV heads of device page
 * block_table[b][j] (K and V) to host page host_table[b][j] of the pinned
 * pools.  Other host pages are not touched.
 *   host_k, host_v  HOST pointers to pinned, device-mapped memory (e.g.
 *                   hipHostMalloc), n_host_pages pages, same layouts as the
 *                   device pools; written by the device over the bus
 * The copies are complete when the stream's work is (synchronize before the
 * host reads the pools or the device pages are reused).
 * Errors: RKV_ERR_INVALID_ARG (including host pools that are not pinned and
 * mapped), RKV_ERR_UNSUPPORTED, RKV_ERR_HIP.
 */
rkv_status rkv_offload_blocks(const rkv_params* params, const uint16_t* k_pages,
                              const uint16_t* v_pages, int64_t n_pages,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* lens, int32_t batch,
                              const int32_t* host_table, uint16_t* host_k,
                              uint16_t* host_v, int64_t n_host_pages,
                              hipStream_t stream);

/*
 * Workspace bytes rkv_stage_resident needs for these sizes.
 */
size_t rkv_stage_workspace_size(const rkv_params* params, int32_t batch,
                                int32_t k_cap);

/*
 * rkv_stage_resident -- host tier with residency across decode steps
 * (openGauss page, "Feature Description" and "Overall Solution": the
 * offload part of the KV cache stays in host DDR and the blocks retrieved at
 * each decode round are loaded into HBM before attention).  Consecutive
 * rounds keep many of the same blocks, so a block already held in HBM is
 * not loaded again: the result is that of rkv_stage_blocks followed by
 * rkv_merge_table with the same host table, with fewer bytes over the bus.
 * Staging slot r (0 <= r < slot_cap) of (sequence b, KV head h) is the
 * head-h slice of device page stage_page0 + b * slot_cap + r.  slot_cap must
 * be at least the number of host-resident blocks a list keeps in one call
 * (k_cap always suffices; ceil(n_off * topk_ppm / 10^6) suffices when no
 * prompt is below the dense boundary).  A list that keeps more gives the
 * blocks that found no slot page -1 (not attended) and reports
 * n_staged = -1.
 * For every (b, h):
 *   slot_ids [batch][n_kv_heads][slot_cap] device int32, IN/OUT: the
 *            logical block each slot holds (-1: none);
 *   slot_cursor [batch][n_kv_heads] device int32, IN/OUT: the next slot to
 *            fill.  Fill slot_ids with -1 and slot_cursor with 0 before the
 *            first call for a sequence (and whenever the host pools, the
 *            host table or the staging pages are changed by anyone else);
 *            leave both untouched between calls.
 *   A kept host-resident block already held by a slot keeps that slot; the
 *   kept host-resident blocks not held take, in ascending block order, the
 *   slots holding no kept block, first-in first-out (in slot order from the
 *   cursor, which then moves past the last slot filled), and are copied
 *   there (K and V tiles of head h, 32 KiB each).  A slot not reused keeps
 *   its block, which then costs no copy if kept again later: with slot_cap
 *   above the number of kept blocks, recently dropped blocks stay resident.
 *   merged / n_merged: as rkv_merge_table (init blocks, kept blocks, local
 *   blocks; kept host-resident blocks at their slot's page, other kept
 *   blocks at their block-table page).
 *   n_staged [batch][n_kv_heads] (optional, may be NULL): blocks copied
 *   (-1: slot_cap was too small for the kept blocks, see above).
 * host_table, host_k, host_v, n_host_pages, sel_ids, n_sel, k_cap: as
 * rkv_stage_blocks; lens as rkv_select.  1 <= slot_cap <= 8192,
 * m_cap >= max_blocks; pages [stage_page0, stage_page0 + batch * slot_cap)
 * must lie inside the device pools.
 * Two launches on `stream` (slot planner, then the copies); calls that
 * overlap on one slot state / workspace race.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
rkv_status rkv_stage_resident(const rkv_params* params, const uint16_t* host_k,
                              const uint16_t* host_v, int64_t n_host_pages,
                              const int32_t* host_table,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* lens, const int32_t* sel_ids,
                              const int32_t* n_sel, int32_t k_cap, int32_t batch,
                              int32_t slot_cap, int32_t* slot_ids,
                              int32_t* slot_cursor, uint16_t* k_pages,
                              uint16_t* v_pages, int64_t n_pages,
                              int64_t stage_page0, int32_t* merged,
                              int32_t* n_merged, int32_t m_cap, int32_t* n_staged,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * rkv_stage_plan / rkv_stage_copy -- rkv_stage_resident's two launches as
 * separate calls, so that the copies can run on a side stream while the
 * attention over the blocks already in HBM runs on the main one (the
 * openGauss page, "Overall Solution": each round loads the retrieved blocks
 * into HBM; here the round's attention starts on the blocks that are
 * there).  rkv_stage_plan is the residency planner: slot state, merged table
 * and the copy list in `workspace`.  With merged_new non-NULL (split mode)
 * the merged table keeps only the entries whose pages are in HBM before
 * this call's copies -- init and window blocks, kept blocks on device or
 * already held in a slot -- in order, and merged_new [batch][n_kv_heads]
 * [k_cap] receives, n_new [batch][n_kv_heads] per list, the staging pages
 * of the blocks this call copies (whole blocks; attend them with
 * rkv_decode_attn_lse and lengths that are multiples of 128).  Kept host
 * blocks left without a slot (n_staged = -1) are in neither table.
 * rkv_stage_copy copies the list the last rkv_stage_plan left in the same
 * workspace (the caller orders it after that call).  Arguments, workspace
 * (rkv_stage_workspace_size) and errors as rkv_stage_resident; n_pages is
 * the device pool's page count.
 */
rkv_status rkv_stage_plan(const rkv_params* params, const int32_t* host_table,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* lens, const int32_t* sel_ids,
                          const int32_t* n_sel, int32_t k_cap, int32_t batch,
                          int32_t slot_cap, int32_t* slot_ids, int32_t* slot_cursor,
                          int64_t n_pages, int64_t stage_page0, int32_t* merged,
                          int32_t* n_merged, int32_t m_cap, int32_t* merged_new,
                          int32_t* n_new, int32_t* n_staged, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);
rkv_status rkv_stage_copy(const rkv_params* params, const uint16_t* host_k,
                          const uint16_t* host_v, int64_t n_host_pages,
                          const int32_t* host_table, int32_t max_blocks, int32_t k_cap,
                          int32_t batch, int32_t slot_cap, uint16_t* k_pages,
                          uint16_t* v_pages, int64_t n_pages, int64_t stage_page0,
                          const void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Bytes of pinned host memory (host_list) the copy-engine staging calls
 * below need for these sizes.
 */
size_t rkv_stage_host_list_size(const rkv_params* params, int32_t batch,
                                int32_t k_cap);

/*
 * rkv_stage_blocks_async -- rkv_stage_blocks through the copy engines (same
 * source, page and staging-page rules, same results): the kept ids and
 * counts (device sel_ids / n_sel as rkv_select wrote them) are copied to the
 * pinned host buffer host_list on `stream`, the calling thread waits for
 * them, and the K and V tiles of every kept host-resident block are copied
 * with hipMemcpy2DAsync / hipMemcpyAsync on `side`: one copy per run of
 * consecutive blocks on consecutive host pages going to consecutive staging
 * pages (per KV head, a 2-D copy with a one-page pitch; in the per-sequence
 * selection mode, where every head keeps the same blocks, whole pages in one
 * contiguous copy).  `done` (may be NULL) is recorded on `side` after the
 * last copy: make the attention's stream wait for it.
 * Copy lanes: each copy command costs the copy engines about 10 us however
 * small it is, and the commands of one stream run one after another.  With
 * params->copy_lanes = n >= 2 the copies go instead to n streams the
 * library creates on the current device at the first such call (default
 * priority, kept until the process ends), each command to the one with the
 * least work queued by this call; they start after the work queued on
 * `side` so far (an event) and `side` waits for them (one event per lane),
 * so `done` and everything later on `side` still follow every copy.  On
 * MI355X four lanes copy whole pages about 2x and 32 KiB tiles about 3x
 * faster than one stream.  The lanes are streams of the calling process:
 * when it has more streams than the runtime has hardware queues
 * (GPU_MAX_HW_QUEUES), streams share queues and work on them can no
 * longer overlap, so lanes are off by default.  Calls that use lanes are
 * serialized by a lock inside the library.  The merged table
 * comes from rkv_merge_table with the device host table, as for
 * rkv_stage_blocks.  The call blocks the calling thread until the ids are
 * on the host, so it cannot be captured in a graph.
 *   host_table_host [batch][max_blocks] HOST int32: the same table as the
 *                   device host_table of rkv_stage_blocks
 *   host_list       pinned host memory, >= rkv_stage_host_list_size bytes
 * Other arguments as rkv_stage_blocks.
 * Errors: RKV_ERR_INVALID_ARG (including host pools or host_list that are
 * not pinned host memory), RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
rkv_status rkv_stage_blocks_async(const rkv_params* params, const uint16_t* host_k,
                                  const uint16_t* host_v, int64_t n_host_pages,
                                  const int32_t* host_table_host, int32_t max_blocks,
                                  const int32_t* sel_ids, const int32_t* n_sel,
                                  int32_t k_cap, int32_t batch, uint16_t* k_pages,
                                  uint16_t* v_pages, int64_t n_pages,
                                  int64_t stage_page0, void* host_list,
                                  size_t host_list_bytes, hipStream_t stream,
                                  hipStream_t side, hipEvent_t done);

/*
 * rkv_stage_resident_async -- rkv_stage_resident with the copies through the
 * copy engines (same slot policy, slot state, merged table and results): the
 * slot planner runs on `stream`, its (block, slot) copy list and counts go
 * to the pinned host buffer host_list, the calling thread waits for them,
 * and the copies are issued on `side` as for rkv_stage_blocks_async (runs
 * of consecutive blocks, host pages and slots; whole pages in the
 * per-sequence mode; over params->copy_lanes lanes when that is 2 or
 * more).  `done` (may be NULL) is recorded on `side` after the last copy.
 * Blocks the calling thread until the list is on the host.
 *   host_table      [batch][max_blocks] DEVICE int32 (read by the planner)
 *   host_table_host the same table in HOST memory (read by the copy issue)
 *   host_list       pinned host memory, >= rkv_stage_host_list_size bytes
 * Other arguments as rkv_stage_resident.
 * Errors: as rkv_stage_resident, and RKV_ERR_INVALID_ARG / RKV_ERR_WORKSPACE
 * for host_list.
 */
rkv_status rkv_stage_resident_async(
    const rkv_params* params, const uint16_t* host_k, const uint16_t* host_v,
    int64_t n_host_pages, const int32_t* host_table, const int32_t* host_table_host,
    const int32_t* block_table, int32_t max_blocks, const int32_t* lens,
    const int32_t* sel_ids, const int32_t* n_sel, int32_t k_cap, int32_t batch,
    int32_t slot_cap, int32_t* slot_ids, int32_t* slot_cursor, uint16_t* k_pages,
    uint16_t* v_pages, int64_t n_pages, int64_t stage_page0, int32_t* merged,
    int32_t* n_merged, int32_t m_cap, int32_t* n_staged, void* workspace,
    size_t workspace_bytes, void* host_list, size_t host_list_bytes,
    hipStream_t stream, hipStream_t side, hipEvent_t done);

/*
 * Workspace bytes rkv_decode_attn needs for these sizes.
 */
size_t rkv_attn_workspace_size(const rkv_params* params, int32_t batch,
                               int32_t m_cap);

/*
 * rkv_decode_attn -- paged decode attention over a merged block table
 * (rkmt.cn ATB article, section 1.1: softmax(Q K^T / sqrt(d_k)) V with one
 * query token; section 2.2: K/V read through a page table).  For query head
 * g of KV head h:
 *     out[b][g] = sum_t softmax_t(scale * q[b][g] . K_t) V_t
 * over every token t of the pages merged[b][h][0 .. n_merged-1].  Every entry
 * holds 128 tokens except the LAST one, taken to be the sequence's trailing
 * block, which holds L - 128 * (ceil(L/128) - 1) tokens.  A (b, h) with
 * n_merged = 0 writes zeros.
 * The work is split over the merged blocks (split-K, the Flash-Decoding
 * idiom named in the CSDN survey's references): the 64-token halves of all
 * merged blocks of the batch are spread evenly over split_waves waves (for
 * a batch of one, whose lists are all equally long, each list's halves are
 * dealt round robin over split_waves / n_kv_heads waves), and the partial
 * softmax results are merged by their log-sum-exp (the survey's
 * cascade-inference paragraph: partial results merged the FlashDecoding
 * way) by a second kernel.  Extent limits: RKV_MAX_QUERY_ROWS and
 * RKV_MAX_LIST_ENTRIES with m_cap as the row.
 *   merged [batch][n_kv_heads][m_cap], n_merged [batch][n_kv_heads]
 *   out [batch][n_q_heads][128] fp32
 *   workspace >= rkv_attn_workspace_size(params, batch, m_cap) bytes of
 *   scratch (partials); calls that overlap on one workspace race.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
rkv_status rkv_decode_attn(const rkv_params* params, const uint16_t* q,
                           const uint16_t* k_pages, const uint16_t* v_pages,
                           int64_t n_pages, const int32_t* merged,
                           const int32_t* n_merged, int32_t m_cap,
                           const int32_t* lens, int32_t batch, float* out,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * rkv_decode_attn_lse -- rkv_decode_attn for one part of each row's tokens,
 * merged with a part attended before (prev_out / prev_lse) and leaving the
 * row's log-sum-exp for a part after it.  Softmax over a union of token
 * sets merges exactly from each set's normalized output and log-sum-exp
 * (the CSDN survey's cascade-inference paragraph: partial results merged
 * the FlashDecoding way), so a step's attention can start on the blocks
 * already in HBM while the rest are still being copied (rkv_stage_plan in
 * split mode): out = softmax over (this call's tokens and the previous
 * part's) of V.
 *   prev_out [batch][n_q_heads][128] fp32, prev_lse [batch][n_q_heads]: a
 *            previous call's out and lse, or both NULL; must not be out
 *   lse      [batch][n_q_heads] fp32 or NULL: log2 of sum_t e^{z_t} over
 *            every token folded into out (z_t = scale * q . K_t), -inf
 *            for none
 *   lens     as rkv_decode_attn: the last entry of a list holds
 *            L - 128 (ceil(L/128) - 1) tokens; to attend every entry as a
 *            whole block (the newly staged part of a split table), pass
 *            lengths that are multiples of 128 (e.g. 128 * m_cap)
 * Other arguments, workspace and errors as rkv_decode_attn.
 */
rkv_status rkv_decode_attn_lse(const rkv_params* params, const uint16_t* q,
                               const uint16_t* k_pages, const uint16_t* v_pages,
                               int64_t n_pages, const int32_t* merged,
                               const int32_t* n_merged, int32_t m_cap,
                               const int32_t* lens, int32_t batch,
                               const float* prev_out, const float* prev_lse,
                               float* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
/*
 * rkv_decode_attn_cascade -- rkv_decode_attn for a batch whose sequences
 * share a prefix of pages (CSDN survey, section "Share--KV cache共享":
 * cascade inference attends a shared prefix once for all requests and
 * merges its partial results with each request's own part the
 * FlashDecoding way; ATB article, section 2.1: pages shared by reference
 * count).  The first shared_blocks logical blocks of every sequence are
 * taken to sit on sequence 0's pages (block_table[b][j] == block_table[0][j]);
 * a sequence's shared range also ends before its last block (which holds
 * the decoded token) and at its first block whose page is not sequence
 * 0's.  Every (page, KV head) tile of the shared range that some sequence
 * attends (an init, kept or window block of its merged list) is read once
 * for a group of 16 / group sequences, whose query heads fill the MFMA tile
 * together (a sequence that did not keep the block is masked out), instead
 * of once per sequence; the rest of each list is attended as by
 * rkv_decode_attn, and the partial results of both parts are merged by
 * log-sum-exp.  The result is rkv_decode_attn's up to floating-point
 * rounding (the partials are merged in another grouping).  Launches: one
 * preparation (shared-block masks and private merged tables, in the
 * workspace), the split, the combine.  With shared_blocks = 0 or a batch of
 * one, exactly rkv_decode_attn's launches.
 *   merged, n_merged, m_cap  as rkv_decode_attn, over device pages (not the
 *                            host tier's staging pages)
 *   sel_ids [batch][n_kv_heads][k_cap], n_sel [batch][n_kv_heads]
 *                            the kept ids that merged was built from
 *   block_table [batch][max_blocks], shared_blocks in [0, max_blocks]
 *   workspace >= rkv_attn_cascade_workspace_size(params, batch, m_cap,
 *                shared_blocks) bytes, 16-byte aligned; calls that overlap on
 *                one workspace race.
 * MFMA only: attn_impl = RKV_ATTN_VALU gives RKV_ERR_UNSUPPORTED.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
size_t rkv_attn_cascade_workspace_size(const rkv_params* params, int32_t batch,
                                       int32_t m_cap, int32_t shared_blocks);
rkv_status rkv_decode_attn_cascade(const rkv_params* params, const uint16_t* q,
                                   const uint16_t* k_pages, const uint16_t* v_pages,
                                   int64_t n_pages, const int32_t* merged,
                                   const int32_t* n_merged, int32_t m_cap,
                                   const int32_t* sel_ids, const int32_t* n_sel,
                                   int32_t k_cap, const int32_t* block_table,
                                   int32_t max_blocks, int32_t shared_blocks,
                                   const int32_t* lens, int32_t batch, float* out,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);


/*
 * rkv_select_attend -- the top-k and merge of rkv_select from given scores,
 * followed by rkv_decode_attn over the merged table (openGauss page,
 * "Overall Solution": the top-K blocks by inner product joined with the
 * initial and window blocks; rkmt.cn ATB article, sections 1.1 and 2.2: the
 * attention over those pages).  Same results, bit for bit, as those two
 * steps: sel_ids / n_sel / merged / n_merged as rkv_select writes them and
 * out as rkv_decode_attn writes it.
 *   scores [batch][n_kv_heads][max_blocks] device fp32, 4-byte aligned:
 *          entry j of (b, h) is the inner-product score of block j (the
 *          group's query heads summed; per-sequence mode: summed over the
 *          heads by the top-k as in rkv_select); the whole [max_blocks] row of a list may be
 *          read, but only its offload blocks' entries affect the result,
 *          and only for lists with 0 < k < n_off.  rkv_select,
 *          rkv_append_select and rkv_decode_step leave exactly these scores
 *          in the first batch * n_kv_heads * max_blocks * 4 bytes of their
 *          select workspace.
 * For a batch of one sequence with per-head selection, MFMA attention
 * (attn_impl != RKV_ATTN_VALU) and max_blocks <= 1024, the top-k and merge
 * run inside the attention launch: each of the P attention waves of a
 * (sequence, KV head) list finds the list's selection from the scores
 * itself (the same set; the list's first wave writes the selection and
 * merged outputs), so the step has no separate top-k launch.  Other shapes
 * take the top-k launch and then rkv_decode_attn's launches.
 * Other arguments as rkv_select (prompt_lens, k_cap, m_cap >= max_blocks,
 * merged and n_merged required) and rkv_decode_attn (workspace:
 * rkv_attn_workspace_size(params, batch, m_cap) bytes; calls that overlap
 * on one workspace race).
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
rkv_status rkv_select_attend(const rkv_params* params, const uint16_t* q,
                             const uint16_t* k_pages, const uint16_t* v_pages,
                             int64_t n_pages, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* lens,
                             const int32_t* prompt_lens, int32_t batch,
                             const float* scores, int32_t* sel_ids,
                             int32_t* n_sel, int32_t k_cap, int32_t* merged,
                             int32_t* n_merged, int32_t m_cap, float* out,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * rkv_decode_step -- one decode step of one layer: rkv_append_select
 * (append the decoded token, score the offload blocks) and then
 * rkv_select_attend on the scores it left in select_workspace.  Same
 * results, bit for bit, as rkv_append_select (with the merged table)
 * followed by rkv_decode_attn.  For a batch of one sequence (see
 * rkv_select_attend) that is three launches: scoring with the append, the
 * attention with the selection folded in, the combine.
 *   select_workspace >= rkv_select_workspace_size(params, batch, max_blocks)
 *   attn_workspace   >= rkv_attn_workspace_size(params, batch, m_cap),
 *                       16-byte aligned, not the select workspace.
 * Other arguments as rkv_append_select and rkv_decode_attn.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP.
 */
rkv_status rkv_decode_step(const rkv_params* params, const uint16_t* k_new,
                           const uint16_t* v_new, uint16_t* k_pages,
                           uint16_t* v_pages, int64_t n_pages, const uint16_t* q,
                           float* reps, const int32_t* block_table,
                           const int32_t* lens, const int32_t* prompt_lens,
                           int32_t batch, int32_t max_blocks, int32_t* sel_ids,
                           int32_t* n_sel, int32_t k_cap, int32_t* merged,
                           int32_t* n_merged, int32_t m_cap, float* out,
                           void* select_workspace, size_t select_workspace_bytes,
                           void* attn_workspace, size_t attn_workspace_bytes,
                           hipStream_t stream);

/*
 * rkv_decode_step_static -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): rkv_decode_step with both workspaces taken from a scratch
 * array the library keeps in device memory, RKV_STATIC_SCRATCH_BYTES per
 * GPU, held from the library's first use on that GPU until the process ends.
 * The call allocates nothing and gives the same results as rkv_decode_step,
 * bit for bit (the same kernels run).  The select workspace takes the first
 * rkv_select_workspace_size bytes (rounded up to 256), the attention
 * workspace the following rkv_attn_workspace_size bytes; a shape that needs
 * more than RKV_STATIC_SCRATCH_BYTES in all fails with RKV_ERR_UNSUPPORTED
 * before anything is enqueued.  Nothing in the scratch has to start at zero.
 * Every call on one GPU uses that GPU's one scratch array and leaves its
 * contents there, so calls that overlap on one GPU (other streams, other
 * host threads) race: the caller must order them.
 * Other arguments and errors as rkv_decode_step.
 */
#define RKV_STATIC_SCRATCH_BYTES (64u << 20)
rkv_status rkv_decode_step_static(const rkv_params* params, const uint16_t* k_new,
                                  const uint16_t* v_new, uint16_t* k_pages,
                                  uint16_t* v_pages, int64_t n_pages,
                                  const uint16_t* q, float* reps,
                                  const int32_t* block_table, const int32_t* lens,
                                  const int32_t* prompt_lens, int32_t batch,
                                  int32_t max_blocks, int32_t* sel_ids,
                                  int32_t* n_sel, int32_t k_cap, int32_t* merged,
                                  int32_t* n_merged, int32_t m_cap, float* out,
                                  hipStream_t stream);

/*
 * Bounds reports (memory isolation of the pages one sequence may touch:
 * rkmt.cn ATB article, section 3.3).  In a library built with RKV_DEBUG,
 * every kernel that clamps or skips an out-of-range device value -- a
 * length outside [0, max_blocks * 128], a page id outside the device pool
 * (other than the merge's own -1 for a block it leaves out), a kept block id
 * outside its list's offload range or [0, max_blocks), a count above its
 * list's capacity, a host page id outside the host pool -- records the first
 * one into *word (device uint64_t, zero-filled by the caller) and goes on as
 * the release build does, so every kernel still exits normally.
 *   rkv_debug_set_report(word): route the reports of kernels launched from
 *     now on, on the current device, to word (NULL: stop reporting).  A
 *     release build returns RKV_ERR_UNSUPPORTED.
 *   rkv_debug_check(word, stream): waits for `stream`, reads and clears
 *     *word; RKV_OK if nothing was reported, else RKV_ERR_BOUNDS with the
 *     kind and value in rkv_last_error.
 */
rkv_status rkv_debug_set_report(uint64_t* word);
rkv_status rkv_debug_check(uint64_t* word, hipStream_t stream);

/*
 * rkv_debug_wave_stamps -- measurement helper, not part of the method.  In
 * a library built with RKV_WAVE_STAMPS, every wave of the folded-selection
 * attention launch (rkv_select_attend / rkv_decode_step for a batch of one)
 * records RKV_WAVE_STAMP_SLOTS 64-bit values, kept by the wave until it
 * ends and then written to a device array (row = the wave's workgroup id,
 * first RKV_WAVE_STAMP_WAVES waves; each launch overwrites the rows of its
 * waves): slot 0 the wave's start, 1 its scores and table row arrived, 2
 * its selection found, 3 its first unit's V tile requested, 4 its merged
 * list in LDS, 5 its partials written, 6 (XCC_ID << 32) | HW_ID (where it
 * ran), 7 + i its i-th unit attended (i < RKV_WAVE_STAMP_SLOTS - 7); times
 * are s_memrealtime ticks (100 MHz), 0 for an event the wave did not
 * reach.  This call copies the first `waves` rows to dst (host memory,
 * waves * RKV_WAVE_STAMP_SLOTS values), blocking; call it after the
 * launches have finished.  The stamps themselves cost the waves a few
 * instructions each.
 * Errors: RKV_ERR_INVALID_ARG (dst NULL with waves > 0, waves outside
 * [0, RKV_WAVE_STAMP_WAVES]), RKV_ERR_UNSUPPORTED (a library built without
 * RKV_WAVE_STAMPS), RKV_ERR_HIP.
 */
#define RKV_WAVE_STAMP_SLOTS 16
#define RKV_WAVE_STAMP_WAVES 4096
rkv_status rkv_debug_wave_stamps(uint64_t* dst, int32_t waves);

/*
 * rkv_read_probe -- measurement helper, not part of the method: reads
 * `bytes` (rounded down to 16) of device memory once with 16-byte loads from
 * every compute unit and XORs the data into *sink (a device uint32), so that
 * a caller can time the achievable streaming-read bandwidth next to the
 * nominal HBM peak.  buffer must be 16-byte aligned.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_HIP.
 */
rkv_status rkv_read_probe(const void* buffer, size_t bytes, uint32_t* sink,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
