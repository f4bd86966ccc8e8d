/*
 * ds_rows.h -- C ABI of the MI355X (gfx950) multi-row sparse-attention
 * decode core.
 *
 * One call of each entry point serves up to DS_ROWS_MAX independent decode
 * requests ("rows"), each with its own key caches, in a single launch
 * sequence. Per row the path is
 *
 *   ds_rows_indexer_score  lightning-indexer score of every cached key
 *   ds_rows_topk           deterministic causal top-512 of those scores
 *   ds_rows_gather         copy of the selected rows of the shared KV
 *   ds_rows_sparse_attn    attention over the gathered rows with a learned
 *                          per-head sink
 *
 * and two fused forms of it: ds_rows_indexer_topk (score and top-512 in one
 * call, the first selection stage in the indexer's epilogue) and
 * ds_rows_sparse_attn_direct (gather and attention in one call). The step
 * before them, ds_rows_compressor, turns each row's decode token into its
 * next compressed cache row.
 *
 * Source pages (docs.rs source views of the Rust crate mlx-native):
 *   [shader 0.18] "mlx-native 0.18.0 src/shaders/deepseek_rows.metal"
 *   [host 0.21]   "mlx-native 0.21.0 src/ops/deepseek_rows.rs"
 * Each entry point names the kernels and dispatch function whose
 * computation and argument checks it provides.
 *
 * Conventions shared by every call
 *   - Device pointers are plain HIP device addresses owned by the caller.
 *     The library allocates nothing and keeps no state between calls.
 *   - bf16 buffers hold raw bfloat16 bit patterns (uint16).
 *   - Every `*_elems` / `*_bytes` argument is the capacity of the buffer
 *     it follows; a call checks that each buffer is large enough.
 *   - All argument checks run before anything is enqueued. A failed check
 *     returns DS_ERR_INVALID_ARGUMENT, enqueues nothing and leaves a
 *     message readable through ds_rows_last_error(). After the arguments,
 *     a call that would launch checks the current HIP device (DS_ERR_DEVICE
 *     if there is none or it is not a gfx950). A failed launch returns
 *     DS_ERR_HIP.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream) of the current HIP device and the call returns without
 *     waiting for it. Calls on one stream run in order, so the four calls
 *     chain without extra synchronisation.
 *   - Bad data is not a call error: it is handled fail-closed (outputs are
 *     zeroed), as described per call.
 *   - Row r of a multi-row call produces, bit for bit, what a one-row call
 *     on row r alone produces.
 */
#ifndef DS_ROWS_H
#define DS_ROWS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS_ROWS_MAX 8          /* rows per call */
#define DS_HEADS 64            /* indexer and attention heads */
#define DS_INDEXER_DIM 128     /* indexer query/key width */
#define DS_HEAD_DIM 512        /* attention query/KV width */
#define DS_TOP_K 512           /* indices selected per row */
#define DS_RATIO 4             /* query positions per compressed key */

typedef enum {
  DS_OK = 0,
  DS_ERR_INVALID_ARGUMENT = 1,  /* a check on the arguments failed */
  DS_ERR_HIP = 2,               /* the HIP runtime refused a launch */
  DS_ERR_DEVICE = 3             /* no current HIP device, or it is not a
                                   gfx950 (the kernels are built for it
                                   alone); nothing was enqueued */
} ds_status;

/* Largest kv_len of a row: the selection kernels address a row's entries
 * with 32-bit byte offsets of 8-byte keys. */
#define DS_KV_LEN_MAX ((1u << 30) - 1)

/* Per-row table of the indexer calls; the fields of the pages'
 * DeepSeekIndexerRow ([host 0.21] DeepSeekIndexerRow,
 * dispatch_deepseek_indexer_rows). Entries [rows, DS_ROWS_MAX) are ignored. */
typedef struct {
  uint32_t rows;                        /* 1..DS_ROWS_MAX */
  uint32_t kv_len[DS_ROWS_MAX];         /* cached compressed keys, in
                                           [1, DS_KV_LEN_MAX] */
  uint32_t start_pos[DS_ROWS_MAX];      /* absolute query position; keys
                                           j >= min(kv_len, (start_pos+1)/4)
                                           are causally hidden; requires
                                           kv_len >= (start_pos+1)/4 */
  int32_t offset[DS_ROWS_MAX];          /* >= 0, added to every emitted index;
                                           offset + visible - 1 <= INT32_MAX */
  uint32_t q_row[DS_ROWS_MAX];          /* row of q [_,64,128] and weights [_,64] */
  uint32_t output_offset[DS_ROWS_MAX];  /* element offset of the row's 512
                                           output indices; the ranges of all
                                           rows must be disjoint */
  const void *keys[DS_ROWS_MAX];        /* device, bf16 [kv_len, 128] */
  uint64_t keys_elems[DS_ROWS_MAX];     /* capacity of keys[r] in elements */
} ds_indexer_rows;

/* Per-row table of the gather and attention calls; the fields of the pages'
 * DeepSeekSparseAttentionRow ([host 0.21] DeepSeekSparseAttentionRow,
 * dispatch_deepseek_sparse_attention_flash_rows). */
typedef struct {
  uint32_t rows;                        /* 1..DS_ROWS_MAX */
  uint32_t kv_len[DS_ROWS_MAX];         /* rows of the row's KV, > 0 */
  uint32_t width[DS_ROWS_MAX];          /* selected slots of the row, > 0 */
  uint32_t index_offset[DS_ROWS_MAX];   /* element offset of the row's `width`
                                           indices in the indices buffer */
  uint32_t q_row[DS_ROWS_MAX];          /* row of q/out [_,64,512]; unique */
  const void *kv[DS_ROWS_MAX];          /* device, bf16 [kv_len, 512]; keys
                                           and values are the same tensor */
  uint64_t kv_elems[DS_ROWS_MAX];       /* capacity of kv[r] in elements */
} ds_sparse_rows;

/* ---- sizes --------------------------------------------------------------
 * Each returns 0 if the table itself is invalid (see ds_rows_last_error).
 * Layouts: row r's scores start at r * max(kv_len); the gathered rows and
 * mask entries of all rows are concatenated in row order, row r starting at
 * the sum of the widths of rows 0..r-1 (times 512 for the gathered rows). */
size_t ds_rows_scores_elems(const ds_indexer_rows *rows);        /* rows * max kv_len */
size_t ds_rows_topk_workspace_bytes(const ds_indexer_rows *rows);
size_t ds_rows_indexer_topk_workspace_bytes(const ds_indexer_rows *rows);
size_t ds_rows_gathered_elems(const ds_sparse_rows *rows);       /* sum(width) * 512 */
size_t ds_rows_mask_elems(const ds_sparse_rows *rows);           /* sum(width) */
size_t ds_rows_attn_workspace_bytes(const ds_sparse_rows *rows);

/* ---- ds_rows_indexer_score ----------------------------------------------
 * Lightning-indexer score of one query per row against the row's keys
 * ([shader 0.18] deepseek_indexer_score_mma_rows_bf16):
 *   scores[r*S + j] = sum_h w[h] * max(0, sum_d q[h,d] * keys_r[j,d])
 * for j < kv_len[r], where S = max kv_len, q = q[q_row[r]] (bf16 [64,128]),
 * w = weights[q_row[r]] (f32 [64]). The products are exact and accumulate in
 * f32. The score is -inf for j >= min(kv_len, (start_pos+1)/4) and when it is
 * not finite. Entries j >= kv_len[r] of row r are not written.
 *   q        device bf16 [q_rows, 64, 128], q_elems >= (max q_row + 1) * 8192
 *   weights  device f32  [q_rows, 64],      weights_elems >= (max q_row + 1) * 64
 *   scores   device f32, scores_elems >= ds_rows_scores_elems(rows)
 * Checks: those of [host 0.21] dispatch_deepseek_indexer_rows on the table,
 * keys capacity >= kv_len * 128, and non-null pointers. */
ds_status ds_rows_indexer_score(const ds_indexer_rows *rows,
                                const void *q, size_t q_elems,
                                const float *weights, size_t weights_elems,
                                float *scores, size_t scores_elems,
                                void *stream);

/* ---- ds_rows_topk -------------------------------------------------------
 * Deterministic causal top-512 of each row's scores ([shader 0.18]
 * index_rows_better and deepseek_indexer_topk_{block,merge,finalize}_rows_i32):
 * among keys j < min(kv_len, (start_pos+1)/4) with a finite score, ranked
 * by score (higher first; equal scores, including -0 and +0, by lower index
 * first), writes the first min(512, candidates) as j + offset[r] in rank
 * order to indices[output_offset[r] + t], and -1 to the remaining slots of
 * the row's 512.
 *   scores     device f32 as written by ds_rows_indexer_score
 *   workspace  device scratch, workspace_bytes >= ds_rows_topk_workspace_bytes
 *              (contents on entry do not matter; clobbered)
 *   indices    device i32, indices_elems >= max(output_offset + 512)
 * Checks: as ds_rows_indexer_score (keys pointers are not used here). */
ds_status ds_rows_topk(const ds_indexer_rows *rows,
                       const float *scores, size_t scores_elems,
                       void *workspace, size_t workspace_bytes,
                       int32_t *indices, size_t indices_elems,
                       void *stream);

/* ---- ds_rows_indexer_topk -----------------------------------------------
 * ds_rows_indexer_score followed by ds_rows_topk, with the first selection
 * stage moved into the indexer ([shader 0.18] deepseek_indexer_score_mma_
 * rows_bf16 and deepseek_indexer_topk_{block,merge,finalize}_rows_i32; the
 * pages' block stage keeps each 1024-key block's best 512). Writes the same
 * scores and the same indices as the two calls, bit for bit.
 * Each wave of the indexer keeps, of its 256 keys, those at or above a
 * threshold that keeps 24 to 32 of them (6 to 8 when every row has at least
 * 262144 visible keys; every valid key when it has at most that many) and a
 * floor below which lie all of its other keys; the top-k levels then
 * select from those candidates, and a row's result stands only if no floor
 * lies above its 512th key. Otherwise (heavy ties, scores sorted by
 * position) the row is selected again from its scores in the same call,
 * which is exact but slower. A call with a row of fewer than 16384 visible
 * keys (too few for its waves' candidates to hold its top 512 reliably)
 * runs the separate score and top-k kernels instead, with the same result.
 *   q, weights, scores  as ds_rows_indexer_score
 *   workspace  device scratch, workspace_bytes >=
 *              ds_rows_indexer_topk_workspace_bytes (enough for either
 *              path; contents on entry do not matter; clobbered)
 *   indices    device i32, indices_elems >= max(output_offset + 512)
 * Checks: those of ds_rows_indexer_score and of ds_rows_topk. */
ds_status ds_rows_indexer_topk(const ds_indexer_rows *rows,
                               const void *q, size_t q_elems,
                               const float *weights, size_t weights_elems,
                               float *scores, size_t scores_elems,
                               void *workspace, size_t workspace_bytes,
                               int32_t *indices, size_t indices_elems,
                               void *stream);

/* ---- ds_rows_indexer_candidates -----------------------------------------
 * The first kernel of ds_rows_indexer_topk alone: writes the scores (as
 * ds_rows_indexer_score) and leaves the waves' candidates and floors in the
 * workspace, where nothing else reads them. For timing the fused indexer
 * kernel on its own; arguments and checks as ds_rows_indexer_topk, without
 * the indices. */
ds_status ds_rows_indexer_candidates(const ds_indexer_rows *rows,
                                     const void *q, size_t q_elems,
                                     const float *weights, size_t weights_elems,
                                     float *scores, size_t scores_elems,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/* ---- ds_rows_indexer_score_mq -------------------------------------------
 * Lightning-indexer scores of query_len (1..8) consecutive queries per row,
 * e.g. speculative or multi-token decode ([shader 0.18]
 * deepseek_indexer_score_mma_rows_bf16: its loop over the query rows of a
 * group, each with its own causal count; the pages' rows dispatch runs it
 * with one query). Query t of row r is q[q_row[r] + t] (bf16 [64,128]) with
 * weights[q_row[r] + t], at absolute position start_pos[r] + t:
 *   scores[(r*query_len + t)*S + j] = sum_h w[h] * max(0, q[h] . keys_r[j])
 * for j < kv_len[r], S = max kv_len, and -inf for
 * j >= min(kv_len, (start_pos + t + 1)/4) or a non-finite score. Arithmetic
 * per key as ds_rows_indexer_score (query_len = 1 gives its bits).
 * The scores of query t of row r sit where ds_rows_topk expects row
 * e = r*query_len + t of a table with kv_len[r] and start_pos[r] + t, so a
 * ds_rows_topk call on such a table (rows*query_len <= 8) selects each
 * query's top 512.
 *   q        device bf16, q_elems >= (max q_row + query_len) * 8192
 *   weights  device f32, weights_elems >= (max q_row + query_len) * 64
 *   scores   device f32, scores_elems >= ds_rows_indexer_mq_scores_elems
 * Checks: rows 1..8, query_len 1..8, kv_len > 0, start_pos + query_len
 * <= UINT32_MAX, kv_len >= (start_pos + query_len)/4 (the last query's causal
 * length), key capacities, operand capacities, non-null pointers. The
 * table's offset and output_offset are not used. */
size_t ds_rows_indexer_mq_scores_elems(const ds_indexer_rows *rows, uint32_t query_len);
ds_status ds_rows_indexer_score_mq(const ds_indexer_rows *rows, uint32_t query_len,
                                   const void *q, size_t q_elems,
                                   const float *weights, size_t weights_elems,
                                   float *scores, size_t scores_elems,
                                   void *stream);

/* ---- ds_rows_gather -----------------------------------------------------
 * Gathers, for slot t < width[r] of row r with i = indices[index_offset[r]+t]
 * ([shader 0.18] deepseek_sparse_attention_gather_rows_bf16):
 *   i == -1               gathered row = 0, mask = -inf   (sentinel)
 *   i < -1 or i >= kv_len gathered row = 0, mask = 0, invalid[r] = 1
 *   otherwise             gathered row = kv_r[i] bit for bit, with every
 *                         non-finite element replaced by +0 (and then
 *                         invalid[r] = 1); mask = 0
 * invalid[r] (entry r of the call's table, not q_row) is written for every
 * row: 1 if any of its slots was bad, else 0. The caller need not clear it.
 *   indices   device i32, indices_elems >= max(index_offset + width)
 *   gathered  device bf16 [sum(width), 512], rows concatenated in row order
 *   mask      device bf16 [sum(width)]
 *   invalid   device u32 [rows], invalid_elems >= rows
 * Checks: those of [host 0.21] sparse_params / sparse_io_checks on the table
 * (rows, kv_len and width non-zero, unique q_row, kv capacity, index range),
 * output capacities, and non-null pointers. */
ds_status ds_rows_gather(const ds_sparse_rows *rows,
                         const int32_t *indices, size_t indices_elems,
                         void *gathered, size_t gathered_elems,
                         void *mask, size_t mask_elems,
                         uint32_t *invalid, size_t invalid_elems,
                         void *stream);

/* ---- ds_rows_sparse_attn ------------------------------------------------
 * Attention of each row's query over its gathered rows, keys = values, with
 * a learned sink logit per head shared by all rows ([shader 0.18]
 * deepseek_sparse_attention_score_rows_bf16 / _reduce_rows_bf16 /
 * _sanitize_rows_bf16; [host 0.21] dispatch_deepseek_sparse_attention_flash_rows,
 * whose flash kernel takes the gathered rows, an additive mask and the
 * per-row invalid flags):
 *   l[h,t]  = scale * q[h] . G[t] + mask[t]   for slots t whose mask is not -inf
 *   m       = max(sink[h], max_t l[h,t])
 *   Z       = exp(sink[h]-m) + sum_t exp(l[h,t]-m)
 *   out[h]  = sum_t exp(l[h,t]-m)/Z * G[t]       (f32 [64,512] per row)
 * out[q_row[r], h, :] is zeroed when invalid[r] != 0, when sink[h] or a
 * live logit l[h,t] is not finite, or when Z is not in (0,inf); any other
 * non-finite output element is zeroed. Logits accumulate in f32 from exact
 * bf16 products; the softmax weights enter the weighted sum as a bf16 hi+lo
 * pair (relative error ~2^-16) with f32 accumulation.
 *   q          device bf16 [q_rows, 64, 512], q_elems >= (max q_row+1)*32768
 *   sinks      device f32 [64]
 *   gathered   device bf16, as written by ds_rows_gather
 *   mask       device bf16 [sum(width)]: 0 or -inf as ds_rows_gather writes
 *              it (any entry other than -inf is added to its logit)
 *   invalid    device u32 [rows], as written by ds_rows_gather
 *   scale      finite and > 0 (1/sqrt(512) for the decode core)
 *   workspace  device scratch, workspace_bytes >= ds_rows_attn_workspace_bytes
 *              (contents on entry do not matter; clobbered)
 *   out        device f32 [q_rows, 64, 512], out_elems >= (max q_row+1)*32768
 * Checks: those of [host 0.21] sparse_params / sparse_io_checks on the table,
 * gathered/mask/invalid capacities, scale, sinks and workspace capacity (the
 * KV pointers of the table are not used by this call). */
ds_status ds_rows_sparse_attn(const ds_sparse_rows *rows,
                              const void *q, size_t q_elems,
                              const float *sinks, size_t sinks_elems,
                              const void *gathered, size_t gathered_elems,
                              const void *mask, size_t mask_elems,
                              const uint32_t *invalid, size_t invalid_elems,
                              float scale,
                              void *workspace, size_t workspace_bytes,
                              float *out, size_t out_elems,
                              void *stream);

/* ---- ds_rows_sparse_attn_direct -----------------------------------------
 * ds_rows_gather followed by ds_rows_sparse_attn in one pass: the selected
 * rows are read straight from kv[r] through the indices (slot t of row r uses
 * indices[index_offset[r] + t]), with the gather's rules (-1 sentinel slots
 * are dropped; a bad index or a non-finite KV element zeroes the row's whole
 * output) and the same attention and output. Nothing is written to a
 * gathered operand. Output bit-identical to ds_rows_gather +
 * ds_rows_sparse_attn on the same inputs, except on rows that the fail-closed
 * rule zeroes in both. Source: the index-reading form of the pages' sparse
 * attention, docs.rs "mlx-native 0.21.0 src/ops/deepseek_rows.rs", function
 * dispatch_deepseek_sparse_attention_rows (its score and reduce kernels in
 * "mlx-native 0.18.0 src/shaders/deepseek_rows.metal" read the KV through
 * the indices), with the gather rules of
 * deepseek_sparse_attention_gather_rows_bf16.
 *   indices    device i32, indices_elems >= max(index_offset + width)
 *   workspace  as ds_rows_sparse_attn (same size query)
 * Checks: those of ds_rows_gather on the table and indices, plus those of
 * ds_rows_sparse_attn on q, sinks, scale, workspace and out. */
ds_status ds_rows_sparse_attn_direct(const ds_sparse_rows *rows,
                                     const void *q, size_t q_elems,
                                     const float *sinks, size_t sinks_elems,
                                     const int32_t *indices, size_t indices_elems,
                                     float scale,
                                     void *workspace, size_t workspace_bytes,
                                     float *out, size_t out_elems,
                                     void *stream);

/* ---- ds_rows_indexer_topk_attn ------------------------------------------
 * The decode core in one call: ds_rows_indexer_topk on irows followed by
 * ds_rows_sparse_attn_direct on srows reading the indices it wrote, with the
 * same scores, indices and output bit for bit. Sources: the pages' rows
 * dispatches run back to back ([host 0.21] dispatch_deepseek_indexer_*_rows
 * and dispatch_deepseek_sparse_attention_rows; [shader 0.18]
 * deepseek_indexer_topk_finalize_rows_i32 and
 * deepseek_sparse_attention_score_rows_bf16).
 * When ds_rows_indexer_topk would keep the first selection stage in the
 * indexer (every row has at least 16384 visible keys) and each row has at
 * most 16384 candidates (up to 131072 keys, or 524288 when every row has at
 * least 262144 visible keys), the final selection level runs inside the
 * attention's workgroups: each repeats its row's selection and
 * reads its slots' indices from LDS, which removes a kernel boundary and the
 * attention's index load. When instead every row has at most 16384 visible
 * keys, the score kernel runs alone and the one selection level, over the
 * scores, runs inside the attention's workgroups in the same way. When the
 * indexer keeps the first stage but a row has more candidates, the selection
 * passes of ds_rows_indexer_topk run, and the last runs inside the
 * attention's workgroups if every row reaches it in the same pass. Otherwise
 * the two calls run as they are.
 *   irows, idx_q, weights, scores, idx_workspace, indices
 *              as ds_rows_indexer_topk (idx_workspace sized by
 *              ds_rows_indexer_topk_workspace_bytes(irows))
 *   srows, q, sinks, scale, attn_workspace, out
 *              as ds_rows_sparse_attn_direct (attn_workspace sized by
 *              ds_rows_attn_workspace_bytes(srows)); srows must list the
 *              same rows in the same order, each with width <= 512 and
 *              index_offset equal to irows' output_offset (the attention
 *              reads the first `width` of the 512 selected slots of its
 *              row; all 512 are written to indices)
 * Checks: those of both calls, plus the row correspondence above. */
ds_status ds_rows_indexer_topk_attn(const ds_indexer_rows *irows, const ds_sparse_rows *srows,
                                    const void *idx_q, size_t idx_q_elems,
                                    const float *weights, size_t weights_elems,
                                    float *scores, size_t scores_elems,
                                    void *idx_workspace, size_t idx_workspace_bytes,
                                    int32_t *indices, size_t indices_elems,
                                    const void *q, size_t q_elems,
                                    const float *sinks, size_t sinks_elems,
                                    float scale,
                                    void *attn_workspace, size_t attn_workspace_bytes,
                                    float *out, size_t out_elems,
                                    void *stream);

/* ---- ds_rows_indexer_topk_attn_noalloc ----------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same
 * computation, results and checks as ds_rows_indexer_topk_attn, with both
 * workspaces taken from a device array the library holds on each GPU it runs
 * on (DS_NOALLOC_SCRATCH_BYTES, kept until the process ends) instead of
 * caller buffers. The caller still passes every input and output. Nothing is
 * allocated or freed by the call.
 * The array must hold ds_rows_indexer_topk_workspace_bytes(irows), rounded up
 * to 256, plus ds_rows_attn_workspace_bytes(srows); a larger call fails with
 * DS_ERR_INVALID_ARGUMENT before anything is enqueued (8 rows of 512 slots
 * fit up to 897024 keys each; one row up to 13.59 million keys). The array
 * needs no clearing: no kernel depends on its contents at entry.
 * Calls on one GPU share its array: calls that overlap in time (e.g. on two
 * streams) race and must be serialised by the caller. The first call on a
 * device looks up the array's device address (DS_ERR_HIP if that fails). */
#define DS_NOALLOC_SCRATCH_BYTES (16u << 20)
ds_status ds_rows_indexer_topk_attn_noalloc(const ds_indexer_rows *irows, const ds_sparse_rows *srows,
                                            const void *idx_q, size_t idx_q_elems,
                                            const float *weights, size_t weights_elems,
                                            float *scores, size_t scores_elems,
                                            int32_t *indices, size_t indices_elems,
                                            const void *q, size_t q_elems,
                                            const float *sinks, size_t sinks_elems,
                                            float scale,
                                            float *out, size_t out_elems,
                                            void *stream);

/* ---- ds_rows_compressor -------------------------------------------------
 * One decode token of the learned KV compressor per row, each row with its
 * own recurrent state ([shader 0.18] deepseek_compressor_rows_bf16;
 * [host 0.21] dispatch_deepseek_compressor_rows). The step that produces the
 * compressed KV rows and indexer keys the calls above read.
 * Shapes: (ratio, head_dim) in {(4,128), (4,512), (128,512)}; coff = 2 for
 * ratio 4 (each window reaches one block back) and 1 for ratio 128;
 * P = coff * head_dim; every state is f32 [coff * ratio, P] row-major
 * (ds_rows_compressor_state_elems).
 * For row r with token position pos = start_pos[r], t = pos % ratio:
 *   - state row slot = (ratio if ratio == 4 else 0) + t takes
 *       kv_state  = kv[r, :]                 (0 where not finite)
 *       score_state = score[r, :] + ape[t, :] (f32 sum; NaN where the sum or
 *                                              the value is not finite)
 *   - if (pos + 1) % ratio == 0, output feature f < head_dim pools the window
 *     (ratio 4: state rows 0..3 at feature f and rows 4..7 at feature
 *     head_dim + f; ratio 128: rows 0..127 at feature f):
 *       c[f] = bf16( sum_i e^(s_i - m) v_i / sum_i e^(s_i - m) ),  m = max s_i
 *       out[r, f] = bf16( c[f] * rsqrt(mean_f c^2 + epsilon) * norm[f] )
 *     and the whole output row is zero if a window score is NaN or +inf, a
 *     window value is not finite, a pooled value, norm element, the RMS
 *     scale or an output value is not finite. With ratio 4 the state rows
 *     0..3 then take rows 4..7 (this block becomes the previous one).
 *   - otherwise out[r, :] = 0.
 * Pooling and normalisation accumulate in f32 (exp via the hardware
 * exponential), so outputs agree with an exact evaluation to within two bf16
 * units in the last place; the state update is exact.
 *   rows       table: start_pos[r] in 1..UINT32_MAX-1; kv_state[r] and
 *              score_state[r] device f32 (read and written), capacities in
 *              elements; all 2 * rows state buffers must be disjoint
 *   kv, score  device f32 [rows, P] (row r of the call is entry r)
 *   ape        device f32 [ratio, P] (position-in-block embedding)
 *   norm       device f32 [head_dim] (RMS scale)
 *   epsilon    finite and > 0
 *   output     device bf16 [rows, head_dim]
 * Checks: those of [host 0.21] dispatch_deepseek_compressor_rows (rows,
 * shape, epsilon, positions, state capacities, disjoint states, operand
 * capacities) and non-null pointers. */
typedef struct {
  uint32_t rows;                        /* 1..DS_ROWS_MAX */
  uint32_t start_pos[DS_ROWS_MAX];      /* the token's absolute position, > 0 */
  float *kv_state[DS_ROWS_MAX];         /* device f32 [coff*ratio, P] */
  float *score_state[DS_ROWS_MAX];      /* device f32 [coff*ratio, P] */
  uint64_t kv_state_elems[DS_ROWS_MAX];
  uint64_t score_state_elems[DS_ROWS_MAX];
} ds_compressor_rows;

size_t ds_rows_compressor_state_elems(uint32_t ratio, uint32_t head_dim);  /* 0 if unsupported */

ds_status ds_rows_compressor(const ds_compressor_rows *rows,
                             uint32_t ratio, uint32_t head_dim, float epsilon,
                             const float *kv, size_t kv_elems,
                             const float *score, size_t score_elems,
                             const float *ape, size_t ape_elems,
                             const float *norm, size_t norm_elems,
                             void *output, size_t output_elems,
                             void *stream);

/* Timing of one indexer launch, for measurement tools.
 *
 * Arms the calling thread's next launch of the indexer kernel (plain or with
 * the fused top-k stage, made by any entry point above) to write wall-clock
 * stamps into `stamps`, a device buffer of `stamps_elems` uint64 entries that
 * the caller owns and fills with zeros beforehand: DS_TIMER_STAMPS_PER_WG
 * entries per workgroup of the launch's grid (workgroup g of the grid, in
 * launch order, at g * DS_TIMER_STAMPS_PER_WG), entry 0 its start and
 * entries 1 .. 4 the ends of its four waves, in ticks of the device's
 * constant wall clock (hipDeviceAttributeWallClockRate, kHz). The span from
 * the smallest start to the largest end is the kernel's execution time where
 * it ran; the launch is an ordinary one (a few extra stores per workgroup),
 * so the kernels around it run as they would. The grid has ceil(max kv_len
 * / B) x rows workgroups, B = 1024 keys with the fused top-k stage; the plain
 * kernel takes the largest power of two B from 1024 down to 64 keys giving
 * at least 256 blocks (sum over rows of ceil(kv_len / B)), and one workgroup
 * per block instead when that grid would be more than twice the blocks;
 * ceil(max kv_len / 64) x rows x DS_TIMER_STAMPS_PER_WG entries always
 * suffice. A launch whose grid needs more entries than
 * `stamps_elems` fails with DS_ERR_INVALID_ARGUMENT (nothing enqueued). One arm serves one launch; a call that fails its argument
 * checks before the launch leaves the arm in place. `stamps` must be
 * non-null (DS_ERR_INVALID_ARGUMENT otherwise); this call enqueues nothing. */
#define DS_TIMER_STAMPS_PER_WG 8
ds_status ds_rows_time_next_indexer(uint64_t *stamps, size_t stamps_elems);

/* Frequency of that wall clock on the current device, in kHz (*khz), from
 * hipDeviceAttributeWallClockRate. DS_ERR_DEVICE without a current device. */
ds_status ds_rows_wall_clock_khz(int *khz);

/* Message of the last failed call on this thread ("ds_rows: ..."), or "". */
const char *ds_rows_last_error(void);

/* Library version string. */
const char *ds_rows_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS_ROWS_H */
