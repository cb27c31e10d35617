/*
 * zr.h - C ABI of libzr, the MI355X (gfx950) library for one decode step of
 * hierarchical sparse KV attention ("zoom-in" over reasoning thoughts).
 *
 * One step, for every sequence b of a batch and every KV head g:
 *   1. zr_coarse_score   score the decode query against one mean summary key
 *                        per generated thought (ZoomR, Sec. 3.3 "Per-Head
 *                        Importance Scoring", eq. alpha).
 *   2. zr_select_topk    keep the k best-scoring thoughts (ZoomR, Sec. 3.3,
 *                        eq. I_top-k).
 *   3. zr_sparse_decode_attn
 *                        exact softmax attention over the tokens of the kept
 *                        thoughts plus a recent window (ZoomR, Sec. 3.3 eq. I_f,
 *                        Sec. 2 eq. A), read from a paged block pool through a
 *                        per-sequence block table (KV-cache management page,
 *                        "Paged KV cache (PagedAttention)").
 *   zr_sparse_decode_step runs steps 1-3 as one call (fewer launches and
 *   dependent memory round trips; same results as the three calls).
 *   zr_sparse_decode_attn_cached repeats step 3 on the selection kept in
 *   the workspace, for the decode steps between semantic boundaries, where
 *   ZoomR keeps the attended set and only the recent tokens grow (ZoomR
 *   Sec. 3.4 and Appendix A.3; Algorithm 1 rebuilds it at boundaries only).
 *   zr_sparse_decode_attn_partials and zr_attn_combine are its two passes
 *   (split-K attention, then the log-sum-exp merge) as separate calls.
 *   zr_dense_paged_decode_attn is the dense baseline: attention over every
 *   cached token through the same block table (same page, eq. 4).
 *   zr_consensus and zr_zoom_decode_attn are ZoomR's full multi-granularity
 *   selection: votes over every (layer, KV head) top-k set, the consensus
 *   set, and attention over prompt + window + consensus thoughts at full
 *   resolution + the other voted thoughts' summaries (ZoomR Sec. 3.3,
 *   "Global Aggregation and Consensus" and "Constructing the Final
 *   Multi-Granularity Context").
 *   zr_append_kv and zr_summary_keys are the append path that precedes a
 *   step: the new token's K/V into the paged cache (with on-demand block
 *   allocation) and the mean summary key of a thought once it is complete.
 *   zr_score_topk is steps 1-2 as one call (a semantic boundary's per-layer
 *   work before the consensus step).
 *   zr_reuse_plan and zr_sparse_decode_attn_reuse are step 3 between
 *   semantic boundaries with the work split made once per boundary (segment
 *   records), instead of planned by every call.
 *   zr_stage_selected moves a step's attended tiles from pools in pinned host
 *   memory into a device staging pool (ZoomR Sec. 3.4, the cache kept in
 *   host memory and only I_f loaded per step).
 *   zr_sparse_decode_step_noalloc is zr_sparse_decode_step on a device array
 *   built into the library, for callers that cannot allocate.
 *   zr_summary_prefetch_rule reports how the step kernel loads summary-key
 *   rows for a geometry (ahead of the thought range or not), for tests.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers (memory of the current HIP
 *     device); the zr_geom / zr_thoughts structs themselves are host memory
 *     and are read during the call only.
 *   - The caller owns every buffer (except the built-in device array of
 *     zr_sparse_decode_step_noalloc). The library never allocates, frees or
 *     synchronizes; each call only enqueues kernels on `stream` (a hipStream_t
 *     passed as void*, NULL = the legacy default stream) and returns.
 *   - Host-visible arguments are validated before anything is enqueued; on a
 *     non-ZR_OK status nothing was enqueued and no output was touched.
 *     ZR_E_LAUNCH reports a HIP launch error (work may be partially enqueued).
 *   - Device-resident integer data is the caller's contract (block ids in
 *     [0, num_blocks), thought spans inside [0, seq_len), seq_len <=
 *     16 * max_blocks_per_seq, sel entries in [-1, N_b)). The kernels clamp
 *     or skip entries outside these ranges so that no access leaves the
 *     buffers, but the result for such entries is unspecified.
 *   - q, k_pool, v_pool, summary_keys and out must be 16-byte aligned
 *     (ZR_E_ALIGN otherwise), the workspace too (ZR_E_WORKSPACE).
 *   - Calls on one stream run in order; calls that write the same buffers on
 *     different streams race.
 *
 * Data layouts (row-major, innermost last; dtype = zr_geom.dtype)
 *   q            [batch][n_q_heads][head_dim]                    dtype
 *   k_pool       [num_blocks][n_kv_heads][16][head_dim]          dtype
 *                token j of sequence b, KV head g is the key row
 *                k_pool[block_table[b][j/16]][g][j%16][:]
 *   v_pool       [num_blocks][n_kv_heads][head_dim][16]          dtype
 *                values are stored dimension-major inside a block: the
 *                value of token j is v_pool[block_table[b][j/16]][g][:][j%16]
 *                (each dimension's 16 slots are contiguous, so a block's
 *                values load directly as matrix-core operands)
 *   block_table  [batch][max_blocks_per_seq]                     int32
 *   seq_lens     [batch]  cached tokens T_b                      int32
 *   thoughts     CSR by sequence: thoughts of sequence b are rows
 *                seq_ptr[b] .. seq_ptr[b+1]-1; a thought is the logical
 *                token span [start, start+len) (ZoomR's regular segment R_i)
 *   summary_keys [n_total][n_kv_heads][head_dim]                 dtype
 *   scores       [n_total][n_kv_heads]                           float32
 *   sel          [batch][n_kv_heads][k] local thought index, ascending,
 *                -1 padded                                       int32
 *   out          [batch][n_q_heads][head_dim]                    float32
 * Query head h reads KV head h / (n_q_heads / n_kv_heads).
 */
#ifndef ZR_H
#define ZR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZR_OK = 0,
  ZR_E_NULL = 1,        /* a required pointer is NULL */
  ZR_E_SHAPE = 2,       /* sizes inconsistent or out of range */
  ZR_E_UNSUPPORTED = 3, /* valid request the library has no kernel for */
  ZR_E_WORKSPACE = 4,   /* workspace NULL or smaller than zr_workspace_bytes() */
  ZR_E_LAUNCH = 5,      /* the HIP runtime reported an error */
  ZR_E_ALIGN = 6,       /* q, pools, out or summary keys not 16-byte aligned */
  ZR_E_SCRATCH = 7      /* zr_sparse_decode_step_noalloc: more than ZR_NOALLOC_SCRATCH_BYTES needed */
} zr_status;

typedef enum { ZR_F32 = 0, ZR_BF16 = 1 } zr_dtype;

/* Built limits. */
#define ZR_BLOCK_SIZE 16
#define ZR_MAX_K 1024                 /* k of zr_select_topk / zr_sparse_decode_attn */
#define ZR_MAX_THOUGHTS_PER_SEQ 8192  /* zr_thoughts.max_per_seq */
#define ZR_MAX_PAIRS 4096             /* batch * n_kv_heads of the attention and step calls */
#define ZR_NOALLOC_SCRATCH_BYTES (16u << 20) /* device scratch of zr_sparse_decode_step_noalloc */

/* Per-sequence results of zr_append_kv. */
#define ZR_APPEND_OK 0              /* token appended, seq_lens[b] grew by one */
#define ZR_APPEND_NO_FREE_BLOCK 1   /* a new block was needed and the free stack was empty */
#define ZR_APPEND_TABLE_FULL 2      /* block_table[b] has no column for the token */
#define ZR_APPEND_BAD_BLOCK 3       /* a block id outside [0, num_blocks) was met */

typedef struct {
  int32_t batch;              /* B >= 0 (B = 0: every call is a no-op) */
  int32_t n_q_heads;          /* Hq > 0, multiple of n_kv_heads */
  int32_t n_kv_heads;         /* Hkv > 0; Hq / Hkv in {1, 2, 4, 8, 16} */
  int32_t head_dim;           /* 64 or 128 */
  int32_t block_size;         /* must be ZR_BLOCK_SIZE (16) */
  int32_t max_blocks_per_seq; /* columns of block_table, >= 1 */
  int32_t num_blocks;         /* physical blocks in each pool, >= 1 */
  int32_t dtype;              /* zr_dtype of q, pools and summary keys */
} zr_geom;

typedef struct {
  const int32_t* seq_ptr;     /* device [batch + 1], non-decreasing, seq_ptr[0] = 0 */
  const int32_t* start;       /* device [n_total] first logical token of each thought */
  const int32_t* len;         /* device [n_total] tokens in each thought (>= 1) */
  const void* summary_keys;   /* device [n_total][n_kv_heads][head_dim], dtype */
  int32_t n_total;            /* = seq_ptr[batch] */
  int32_t max_per_seq;        /* >= max_b (seq_ptr[b+1] - seq_ptr[b]) */
} zr_thoughts;

/*
 * Coarse scorer (ZoomR, Sec. 3.3, eq. alpha, with grouped-query heads):
 *   scores[i][g] = sum over the query heads h of KV group g of q[b][h] . kbar[i][g]
 * for every thought i of sequence b. The sum over the group is the plain
 * GQA reading of a per-head score (one score per KV head). Accumulated in
 * float64, rounded once to float32. Reads q and summary keys; writes every
 * row of `scores`.
 * Errors: ZR_E_NULL (geom, q, th or its pointers, scores), ZR_E_SHAPE,
 * ZR_E_UNSUPPORTED, ZR_E_ALIGN, ZR_E_LAUNCH.
 */
zr_status zr_coarse_score(const zr_geom* geom, const void* q, const zr_thoughts* th,
                          float* scores, void* stream);

/*
 * Per-(sequence, KV head) top-k (ZoomR, Sec. 3.3, eq. I_top-k): among the
 * thoughts of sequence b, keep the min(k, N_b) best under the order
 * (score descending, then thought index ascending; NaN below every number,
 * -0 equal to +0), written in ascending thought index to sel[b][g][0..),
 * the rest of the row filled with -1. k >= N_b keeps every thought; k = 0
 * writes nothing (sel may then be NULL).
 * Errors: ZR_E_NULL, ZR_E_SHAPE (k < 0 or > ZR_MAX_K, max_per_seq out of
 * range), ZR_E_LAUNCH.
 */
zr_status zr_select_topk(const zr_geom* geom, const zr_thoughts* th, const float* scores,
                         int32_t k, int32_t* sel, void* stream);

/*
 * zr_coarse_score then zr_select_topk in one call (one kernel; scores and
 * sel bit-identical to the two calls): the per-layer work of a semantic
 * boundary before the consensus step (ZoomR Algorithm 1, scores and top-k of
 * every head; Sec. 3.3). k = 0 writes the scores only (sel may be NULL).
 * Errors: those of zr_coarse_score and zr_select_topk, and ZR_E_UNSUPPORTED
 * when max_per_seq and k do not fit the kernel's on-chip memory.
 */
zr_status zr_score_topk(const zr_geom* geom, const void* q, const zr_thoughts* th, int32_t k,
                        float* scores, int32_t* sel, void* stream);

/*
 * Zoomed-in sparse decode attention (ZoomR, Sec. 3.3 eq. I_f restricted to
 * the recent window and the selected thoughts' full-resolution spans; Sec. 2
 * eq. A). For sequence b, KV head g the attended tokens are
 *   [T_b - window, T_b)  union  [start_i, start_i + len_i) for i in sel[b][g]
 * each token once (window clipped at 0). Every query head h of group g gets
 *   out[b][h] = softmax(scale * q[b][h] . K_j) weighted sum of V_j
 * over those tokens, with float32 accumulation; an empty token set gives 0.
 * `sel` rows are read as written by zr_select_topk (k columns, -1 = none;
 * any order, repeats count once); k = 0 means window only (sel may then be
 * NULL).
 * Work split: one pair kernel lists each (b, g)'s attended 16-token blocks
 * with slot masks; the attention kernel's workgroups take equal ranges of
 * all (b, g) lists laid end to end (the grid is sized from `max_attended`,
 * the caller's bound on tokens per (b, g); a larger count is still handled
 * correctly, only with a coarser split); a combine kernel merges the
 * partial softmax states by log-sum-exp. `workspace` holds the block lists
 * (kept for zr_sparse_decode_attn_cached) and the partial results; it must
 * be at least zr_workspace_bytes(geom, max_attended) bytes and 16-byte
 * aligned, and calls that share a workspace must not run concurrently.
 * Errors: ZR_E_NULL, ZR_E_SHAPE (k, window, max_attended < 0; k > ZR_MAX_K),
 * ZR_E_UNSUPPORTED (also: the per-(b, g) lists do not fit the kernel's
 * on-chip memory, roughly max_blocks_per_seq > 20000, or batch * n_kv_heads
 * * (2 max_blocks_per_seq + 1) > INT32_MAX, the list entries the work split
 * counts), ZR_E_WORKSPACE, ZR_E_ALIGN, ZR_E_LAUNCH.
 */
zr_status zr_sparse_decode_attn(const zr_geom* geom, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* seq_lens, const zr_thoughts* th,
                                const int32_t* sel, int32_t k, int32_t window, float scale,
                                int32_t max_attended, float* out, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * Sparse attention on a cached selection. `workspace` must hold the block
 * lists written by the last zr_sparse_decode_attn, zr_sparse_decode_step or
 * zr_zoom_decode_attn that used it (same geom; the block-table rows of those spans unchanged):
 * the selected thoughts' spans, clipped below that call's window start
 * T0 - window0. This call attends those spans plus its own window
 * [max(T - window, T0 - window0), T) of the current seq_lens: a window that
 * would reach below T0 - window0 starts there instead, so that no token is
 * attended twice (the lists keep T0 - window0 per (b, g) in the workspace).
 * Between semantic boundaries pass
 * window = window0 + (T - T0), so that the window keeps the start it had at
 * the boundary and every token decoded since is attended (ZoomR Sec. 3.4:
 * the attended set is recomputed only at semantic boundaries); the result
 * then equals zr_sparse_decode_attn with the same selection and that window.
 * A smaller window leaves the tokens between the two window starts out.
 * Workspace and errors as zr_sparse_decode_attn (ws_bytes >=
 * zr_workspace_bytes(geom, max_attended); the lists do not depend on
 * max_attended).
 */
zr_status zr_sparse_decode_attn_cached(const zr_geom* geom, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       const int32_t* seq_lens, int32_t window, float scale,
                                       int32_t max_attended, float* out, void* workspace,
                                       size_t ws_bytes, void* stream);

/*
 * Attention between semantic boundaries with the work split fixed at the
 * boundary (ZoomR Sec. 3.4 and Appendix A.3: the attended set is rebuilt
 * only at semantic boundaries; between them the selected spans stay and the
 * recent window grows by one token per step).
 *
 * zr_reuse_plan, called once after the boundary call (zr_sparse_decode_attn,
 * zr_sparse_decode_step or zr_zoom_decode_attn) that left its block lists in
 * `workspace`, with that call's geom, window and max_attended and the
 * lengths T0 = seq_lens at the boundary: it splits the attention over the
 * lists' spans and the window [T0 - window, T0 + horizon) (starting no
 * earlier than the lists' own window start) among the
 * attention workgroups and keeps, per workgroup, a record of its share with
 * the list entries resolved, in `workspace`.
 * zr_sparse_decode_attn_reuse, called at every step after that with the
 * current lengths T (T0 <= T <= T0 + horizon) and a new query: attention over
 * the spans and [T0 - window, T), i.e. zr_sparse_decode_attn_cached with
 * window + (T - T0), each workgroup starting from its record rather than
 * planning: before its first K/V loads it reads the record's header and then
 * the entries in it, instead of every pair's list length, the plan and then
 * the list entries. Tokens past T0 + horizon are left out. out = NULL runs the
 * attention pass only (its partial states stay in the workspace for
 * zr_attn_combine, called with the same geom and max_attended).
 * Block ids of the boundary's blocks are taken when the records are made;
 * blocks appended later are read from the block table. Another
 * zr_sparse_decode_attn, zr_sparse_decode_step or zr_zoom_decode_attn on the
 * workspace replaces the lists: call zr_reuse_plan again (calls that only
 * attend, such as zr_sparse_decode_attn_cached, leave the records valid).
 * With horizon = 0 and T = T0 the output equals zr_sparse_decode_attn_cached
 * with `window` bit for bit.
 * A horizon above 16 * max_blocks_per_seq (the table's capacity) plans the
 * same records as that capacity: no window reaches past it.
 * Errors: ZR_E_NULL, ZR_E_SHAPE (window, horizon, max_attended < 0),
 * ZR_E_UNSUPPORTED, ZR_E_WORKSPACE, and for zr_sparse_decode_attn_reuse those
 * of zr_sparse_decode_attn_cached.
 */
zr_status zr_reuse_plan(const zr_geom* geom, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t window, int32_t horizon, int32_t max_attended, void* workspace,
                        size_t ws_bytes, void* stream);
zr_status zr_sparse_decode_attn_reuse(const zr_geom* geom, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_table,
                                      const int32_t* seq_lens, float scale, int32_t max_attended,
                                      float* out, void* workspace, size_t ws_bytes,
                                      void* stream);

/*
 * The two passes of zr_sparse_decode_attn_cached as separate calls: the
 * split-K attention and the log-sum-exp combine (ZoomR Sec. 2 eq. A computed
 * as a sum over blocks, KV-cache management page eq. 4, in pieces whose
 * softmax states are merged afterwards).
 *
 * zr_sparse_decode_attn_partials runs the attention kernel only, on the block
 * lists and with the arguments of zr_sparse_decode_attn_cached (no `out`): for
 * every piece of the (b, g) lists it leaves the running maximum, sum and
 * weighted value sum of each query head in the workspace.
 * zr_attn_combine merges the partial states the last attention call on
 * `workspace` left (this one, or any attention call, which combines them
 * itself as well) into out[b][h] ([batch][n_q_heads][head_dim] float32,
 * 16-byte aligned). It must get the geom and max_attended of that call, which
 * fix the workspace layout (zr_dense_paged_decode_attn lays it out for
 * max_attended = 16 * max_blocks_per_seq; with other values the output is
 * wrong, but nothing outside the workspace is read); the workspace is only
 * read.
 * partials followed by combine give bit for bit the output of
 * zr_sparse_decode_attn_cached with the same arguments. Workspace ownership
 * and concurrency as zr_sparse_decode_attn.
 * Errors: those of zr_sparse_decode_attn_cached; for zr_attn_combine
 * ZR_E_NULL (out), ZR_E_ALIGN (out), ZR_E_SHAPE (max_attended < 0),
 * ZR_E_UNSUPPORTED (geometry, batch * n_kv_heads > ZR_MAX_PAIRS),
 * ZR_E_WORKSPACE, ZR_E_LAUNCH.
 */
zr_status zr_sparse_decode_attn_partials(const zr_geom* geom, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_table,
                                         const int32_t* seq_lens, int32_t window, float scale,
                                         int32_t max_attended, void* workspace,
                                         size_t ws_bytes, void* stream);
zr_status zr_attn_combine(const zr_geom* geom, int32_t max_attended, float* out,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * One whole sparse decode step: zr_coarse_score, zr_select_topk and
 * zr_sparse_decode_attn with the same arguments, fused so that the scores,
 * the selection and the block lists of each (b, g) come from one kernel.
 * Writes `scores` ([n_total][n_kv_heads]), `sel` ([batch][n_kv_heads][k];
 * may be NULL when k = 0) and `out`, bit-identical to the three calls.
 * Needs summary keys (16-byte aligned) and the workspace of
 * zr_sparse_decode_attn.
 * Errors: as the three calls.
 */
zr_status zr_sparse_decode_step(const zr_geom* geom, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* seq_lens, const zr_thoughts* th, int32_t k,
                                int32_t window, float scale, int32_t max_attended,
                                float* scores, int32_t* sel, float* out, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * The per-step host-to-device move of the attended set, for pools kept in
 * host memory (ZoomR Sec. 3.4, "Decoding Stage": the full cache stays in CPU
 * memory and each generation step loads only the entries of I_f to the GPU).
 * k_pool / v_pool may be device-mapped pinned host memory (or device memory).
 * The call
 *   1. builds each (sequence b, KV head g) pair's block list from `sel` and
 *      `th` into `workspace`, as zr_sparse_decode_attn does (selected spans
 *      clipped below T - window; the same lists zr_sparse_decode_attn_cached
 *      reads);
 *   2. copies, for every pair, the key and value tiles of the listed blocks
 *      and then of the window [T - window, T) into the staging pools:
 *      entry j of pair (b, g) goes to staging block b * stage_blocks + j,
 *      KV head g (k_stage [batch * stage_blocks][n_kv_heads][16][head_dim],
 *      v_stage [batch * stage_blocks][n_kv_heads][head_dim][16], device
 *      memory, 16-byte aligned);
 *   3. writes the pairs' lists again with staging block ids into
 *      `stage_workspace` (at least zr_workspace_bytes(geom_stage,
 *      max_attended) bytes, geom_stage = geom with num_blocks = batch *
 *      stage_blocks and max_blocks_per_seq + 1: a staged list also holds
 *      the window's blocks, so it can be one entry longer than a row of the
 *      block table).
 * zr_sparse_decode_attn_cached(geom_stage, q, k_stage, v_stage, block_table,
 * seq_lens, 0, scale, max_attended, out, stage_workspace, ...) then gives,
 * bit for bit, zr_sparse_decode_attn on the original pools with the same
 * sel and window (with window 0 it reads no block-table entry, so the
 * original block_table serves). Entries past stage_blocks of a pair are not
 * staged (that attention then leaves them out): dropped[p] ([batch *
 * n_kv_heads] int32) receives their number, 0 when the pair fits. A pair
 * lists at most ceil(max_attended / 16) + 2 k + 2 blocks when max_attended
 * bounds its attended tokens (a span of L tokens can touch ceil(L / 16) + 1
 * blocks, and so can the window), and never more than max_blocks_per_seq + 1
 * (every block attended, the block where the spans stop and the window
 * starts listed for both), so stage_blocks = max_blocks_per_seq + 1 never
 * drops an entry.
 * Errors: ZR_E_NULL, ZR_E_SHAPE (k, window, max_attended < 0; k > ZR_MAX_K;
 * stage_blocks outside [1, max_blocks_per_seq + 1]), ZR_E_ALIGN, ZR_E_WORKSPACE
 * (either workspace), ZR_E_UNSUPPORTED, ZR_E_LAUNCH.
 */
zr_status zr_stage_selected(const zr_geom* geom, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const zr_thoughts* th, const int32_t* sel, int32_t k, int32_t window,
                            int32_t max_attended, void* workspace, size_t ws_bytes,
                            int32_t stage_blocks, void* k_stage, void* v_stage,
                            void* stage_workspace, size_t stage_ws_bytes, int32_t* dropped,
                            void* stream);

/*
 * zr_sparse_decode_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step with the same arguments minus the workspace,
 * whose role a device array built into the library takes, ZR_NOALLOC_SCRATCH_BYTES
 * (16 MiB) on each GPU the library runs on, held until the process ends.
 * The call allocates nothing. Results are bit-identical to
 * zr_sparse_decode_step with a workspace of its own. The array's address is
 * looked up on the first call on each device (with that device current).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race, and the block lists a call
 * leaves there are overwritten by the next call (zr_sparse_decode_attn_cached
 * cannot reuse them).
 * Errors: those of zr_sparse_decode_step; ZR_E_SCRATCH when
 * zr_workspace_bytes(geom, max_attended) exceeds ZR_NOALLOC_SCRATCH_BYTES
 * (checked before anything is enqueued); ZR_E_LAUNCH also when the array's
 * address cannot be obtained.
 */
zr_status zr_sparse_decode_step_noalloc(const zr_geom* geom, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* block_table,
                                        const int32_t* seq_lens, const zr_thoughts* th,
                                        int32_t k, int32_t window, float scale,
                                        int32_t max_attended, float* scores, int32_t* sel,
                                        float* out, void* stream);

/*
 * Dense paged decode attention (the baseline): softmax attention of every
 * query head over all T_b cached tokens of its sequence, read block by block
 * through the block table (KV-cache management page, eq. 4; ZoomR Sec. 2
 * eq. A). Same split and combine as the sparse call (every block of the
 * sequence, no pair kernel) with max_attended = 16 * max_blocks_per_seq;
 * workspace >= zr_workspace_bytes(geom, 16 * max_blocks_per_seq).
 * Errors: as zr_sparse_decode_attn.
 */
zr_status zr_dense_paged_decode_attn(const zr_geom* geom, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table,
                                     const int32_t* seq_lens, float scale, float* out,
                                     void* workspace, size_t ws_bytes, void* stream);

/*
 * Append one decode token per sequence to the paged cache (ZoomR Algorithm 1:
 * the new k_t, v_t enter the cache before scoring; KV-cache management page,
 * paged KV cache: a block is allocated on demand, only when the sequence's
 * last block is full). For every sequence b with T = seq_lens[b]:
 *   - if T % 16 == 0, pop the top of the free stack (free_blocks[*free_count
 *     - 1], then *free_count decreases) into block_table[b][T / 16];
 *   - write k_new[b][g][:] to key slot T % 16 and v_new[b][g][:] to value
 *     slot T % 16 of block block_table[b][T / 16], every KV head g;
 *   - seq_lens[b] = T + 1; status[b] = ZR_APPEND_OK.
 * On ZR_APPEND_NO_FREE_BLOCK / TABLE_FULL / BAD_BLOCK nothing of sequence b
 * changes (a BAD_BLOCK pop still consumes the stack entry). When several
 * sequences need a block in one call, which of the popped blocks each gets
 * is unspecified (they pop concurrently); each popped block goes to exactly
 * one sequence. Blocks are returned to the stack by the caller (writing
 * free_blocks and *free_count between calls).
 * Layouts: k_new, v_new [batch][n_kv_heads][head_dim] dtype (16-byte
 * aligned, like the pools); free_blocks [capacity] int32; free_count [1]
 * int32; status [batch] int32; block_table and seq_lens are updated in place.
 * Errors: ZR_E_NULL, ZR_E_SHAPE, ZR_E_UNSUPPORTED, ZR_E_ALIGN, ZR_E_LAUNCH.
 */
zr_status zr_append_kv(const zr_geom* geom, void* k_pool, void* v_pool, int32_t* block_table,
                       int32_t* seq_lens, const void* k_new, const void* v_new,
                       const int32_t* free_blocks, int32_t* free_count, int32_t* status,
                       void* stream);

/*
 * Mean summary keys of completed thoughts (ZoomR, Sec. 3.3, eq. for the mean
 * summary key; computed over the thought's own cached keys). For every
 * w < n_which, i = which[w] (a global thought index of `th`), b its sequence
 * and every KV head g:
 *   summary_keys[i][g][:] = mean over j in [start_i, start_i + len_i) of the
 *                           cached key K[b][g][j]
 * summed in float64, divided once, rounded to float32 and then, for bf16
 * caches, to bf16 (nearest even). Reads k_pool through block_table; writes
 * only the rows `which` of summary_keys ([n_total][n_kv_heads][head_dim]
 * dtype, 16-byte aligned; th->summary_keys is not read). An index outside
 * [0, n_total) is skipped.
 * Errors: ZR_E_NULL, ZR_E_SHAPE (n_which < 0), ZR_E_UNSUPPORTED, ZR_E_ALIGN,
 * ZR_E_LAUNCH.
 */
zr_status zr_summary_keys(const zr_geom* geom, const void* k_pool, const int32_t* block_table,
                          const zr_thoughts* th, const int32_t* which, int32_t n_which,
                          void* summary_keys, void* stream);

/*
 * Votes and consensus (ZoomR, Sec. 3.3, eqs. for I_all and v_i; Sec. 4, the
 * agreeability metric AG). sel holds n_layers stacked selections, [n_layers]
 * [batch][n_kv_heads][k], each row a set of local thought indices (-1 =
 * none; any order, as zr_select_topk writes them or otherwise). For every
 * sequence b:
 *   votes[i] = number of (layer, KV head) rows holding thought i, a row
 *              counting once however often it lists i  ([n_total]);
 *   cons[b][0..) = the min(c, |I_all|) thoughts with the most votes among those
 *                  with at least one, ties to the lower index, ascending, -1
 *                  padded to c  ([batch][c]);
 *   agree[b] = sum of the consensus thoughts' votes / sum of all votes (0 if
 *              there are none)  ([batch] float32).
 * Indices outside [0, N_b) in sel are ignored. n_layers = 0 or k = 0 gives
 * no votes.
 * Errors: ZR_E_NULL, ZR_E_SHAPE (n_layers, k, c < 0; k, c > ZR_MAX_K),
 * ZR_E_UNSUPPORTED (max_per_seq too large for on-chip memory), ZR_E_LAUNCH.
 */
zr_status zr_consensus(const zr_geom* geom, const zr_thoughts* th, const int32_t* sel,
                       int32_t n_layers, int32_t k, int32_t c, int32_t* votes, int32_t* cons,
                       float* agree, void* stream);

/*
 * Attention over ZoomR's multi-granularity set (ZoomR, Sec. 3.3, eq. for
 * I_f), one set per sequence shared by all heads:
 *   I_f = [0, n_prompt)  union  [T_b - window, T_b)
 *         union  R_i = [start_i, start_i + len_i)          for i in cons[b]
 *         union  S_i = [sum_start_i, sum_start_i + sum_len_i)  for the other
 *                                                 thoughts with votes[i] > 0
 * (th->start/len are the regular segments R_i; sum_start/sum_len [n_total]
 * the summary segments S_i), each token once, clipped to [0, T_b). Every
 * query head gets softmax(scale * q . K) V over I_f, float32 accumulation.
 * Like zr_sparse_decode_attn it leaves the block lists in `workspace`, so
 * zr_sparse_decode_attn_cached can repeat the attention between semantic
 * boundaries. Workspace, alignment and errors as zr_sparse_decode_attn
 * (ZR_E_SHAPE also for c or n_prompt < 0).
 */
zr_status zr_zoom_decode_attn(const zr_geom* geom, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, const zr_thoughts* th,
                              const int32_t* sum_start, const int32_t* sum_len,
                              const int32_t* votes, const int32_t* cons, int32_t c,
                              int32_t n_prompt, int32_t window, float scale,
                              int32_t max_attended, float* out, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * How the scorer of zr_coarse_score, zr_score_topk and zr_sparse_decode_step
 * schedules its summary-key loads (introspection for tests and tuning; no
 * passage of the pages defines it, the results never depend on it). On even
 * batches it loads a batch of `rows` summary-key rows before sequence b's
 * thought range [seq_ptr[b], seq_ptr[b+1]) is known, starting at row
 *   max(0, (int)((float)b * per_seq) - margin)
 * and uses them when they hold the whole range (else it loads the range's
 * rows once it is known). Host pointers; *rows = *margin = 0 and
 * *per_seq = 0 when the rule is off for this geometry and thought counts.
 * Errors: ZR_E_NULL, ZR_E_SHAPE (n_total or max_per_seq < 0), and the
 * geometry errors of the other calls.
 */
zr_status zr_summary_prefetch_rule(const zr_geom* geom, int32_t n_total, int32_t max_per_seq,
                                   int32_t* rows, float* per_seq, int32_t* margin);

/* Workspace bytes the attention calls need for a grid sized for
 * `max_attended` tokens per (sequence, KV head): per-(b, g) block lists
 * (8 bytes per block-table column) and the partial softmax states (one per
 * piece of a (b, g) list that one workgroup takes). 0 if geom is invalid or
 * batch * n_kv_heads > ZR_MAX_PAIRS. */
size_t zr_workspace_bytes(const zr_geom* geom, int32_t max_attended);

/* Static, NUL-terminated description of a status code. */
const char* zr_status_string(zr_status s);

#ifdef __cplusplus
}
#endif

#endif /* ZR_H */
