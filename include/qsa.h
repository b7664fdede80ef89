/*
 * qsa.h -- C ABI of libqsa.so, the QSA token indexer's hot path on one AMD
 * Instinct MI355X (gfx950): pool -> score -> select/mask.
 *
 * Sources (web pages, cited by title and section):
 *   [SEL]   pegainfer pull request 1178, "select QSA indexer blocks and their tail"
 *   [SCORE] pegainfer pull request 1160, "score QSA token-indexer blocks in native CUDA"
 *   [QSA]   metrale model layers, layers/qsa.rs (source view)
 *
 * Geometry is compiled in: 4 query heads, head dim 128, 4-token blocks, at most
 * 512 kept blocks per row ([SCORE] "Frozen semantics"; [SEL] "Exact semantics").
 * rotary_dim, rope_theta, rms_eps and budget are run-time arguments.
 *
 * Conventions shared by every call:
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are
 *     row-major, in device memory, owned by the caller.
 *   - The library allocates, frees, synchronises and reads back nothing.
 *     All work is enqueued on `stream` (a hipStream_t; NULL = null stream).
 *     Calls are thread-safe and keep no state between calls, with one
 *     exception: qsa_select_mask_noalloc works in a library-owned device
 *     array per GPU, whose address it looks up once under a lock, and calls
 *     of it that overlap on one GPU race (see there).
 *   - Host-side refusals return a negative QSA_ERR_* code before any launch;
 *     nothing is written then.  An empty launch (zero rows / tokens / blocks)
 *     returns QSA_OK and enqueues nothing.
 *   - Device-side refusals never trap: kernels OR bits into the caller-owned,
 *     caller-zeroed int32 *dev_status (QSA_STATUS_*) and write the documented
 *     fallback for the offending row.
 *   - Supported key caches hold at most QSA_MAX_TOKENS tokens.
 */
#ifndef QSA_H
#define QSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 10

#define QSA_HEADS 4
#define QSA_HEAD_DIM 128
#define QSA_RATIO 4
#define QSA_MAX_KEEP_BLOCKS 512
/* 65536 blocks plus a 3-token tail: the longest row whose visible blocks the
 * selector holds on chip. */
#define QSA_MAX_TOKENS 262147

/* Return codes. */
#define QSA_OK 0
#define QSA_ERR_NULL (-1)     /* a required pointer is NULL while its extent is > 0 */
#define QSA_ERR_EXTENT (-2)   /* negative extent, or a block range past tokens/4 */
#define QSA_ERR_BUDGET (-3)   /* budget not a positive multiple of 4, or budget/4 > 512 */
#define QSA_ERR_STRIDE (-4)   /* a row stride narrower than its row */
#define QSA_ERR_CAPACITY (-5) /* an output buffer too short, or tokens > QSA_MAX_TOKENS */
#define QSA_ERR_PARAM (-6)    /* rotary_dim, rope_theta or rms_eps out of range */
#define QSA_ERR_LAUNCH (-7)   /* the HIP runtime refused the launch */

/* Bits OR-ed into *dev_status by the kernels. */
#define QSA_STATUS_BAD_POSITION 1   /* pos[r] outside [0, tokens) */
#define QSA_STATUS_NONFINITE_SCORE 2 /* a NaN or +-Inf among a row's visible block scores */
#define QSA_STATUS_BAD_INDEX 4       /* qsa_gather_kv: a token outside the cache, or a bad count */
#define QSA_STATUS_BAD_GEOMETRY 8    /* *_dev calls: the device token count outside [0, max_tokens] */

/*
 * qsa_pool_keys -- pooled key of every 4-token block in
 * [first_block, first_block + n_blocks).
 *
 * [SCORE] summary: the block's four raw keys are averaged in float32 and cast
 * to bf16, then (1 + w) RMSNorm with k_norm_w and partial RoPE at the block's
 * first token 4b.  [QSA] pool_new_blocks: only newly completed blocks need
 * pooling, hence the block range.
 *
 *   raw_keys    [tokens, key_stride] bf16; the key is the first 128 columns of
 *               each row.  key_stride >= 128 (elements).
 *   k_norm_w    [128] bf16 norm weight (the scale is 1 + w).
 *   rotary_dim  even, 0..128: channels [0, rotary_dim) rotate as pairs
 *               (i, i + rotary_dim/2) at frequency theta^(-2i/rotary_dim);
 *               the rest pass through.
 *   rope_theta  > 0 and finite.   rms_eps  >= 0 and finite.
 *   pooled      [tokens/4, 128] bf16; rows [first_block, first_block+n_blocks)
 *               are written, all others untouched.
 * Refusals: NULL pointers (QSA_ERR_NULL); negative extents or
 * first_block + n_blocks > tokens/4 (QSA_ERR_EXTENT); key_stride < 128
 * (QSA_ERR_STRIDE); bad rotary_dim / theta / eps (QSA_ERR_PARAM).
 */
int qsa_pool_keys(const uint16_t* raw_keys, int64_t key_stride, int64_t tokens,
                  const uint16_t* k_norm_w, int32_t rotary_dim, float rope_theta,
                  float rms_eps, int64_t first_block, int64_t n_blocks,
                  uint16_t* pooled, void* stream);

/*
 * qsa_score_rows -- block scores of query rows against the pooled keys.
 *
 * [SCORE] summary: each of the row's 4 query heads is (1 + w) RMSNorm-ed with
 * q_norm_w and roped at the row's own position p; the score of block b is
 * sum_h relu(q_h . k_b) / sqrt(128), relu per head before the head sum, f32.
 * relu keeps NaN, so a poisoned key scores NaN ([SCORE] review).  Row r sees
 * blocks b < (pos[r] + 1) / 4 ([SEL] "Exact semantics").
 *
 *   q           [rows, q_stride] bf16; heads h at columns [128h, 128h + 128).
 *               q_stride >= 512 (elements).
 *   pos         [rows] int32 row positions, token 0 first visible.
 *   q_norm_w    [128] bf16.
 *   pooled      [tokens/4, 128] bf16 from qsa_pool_keys.
 *   scores      f32, row stride score_cols >= tokens/4, scores_len elements
 *               (spare capacity allowed).  Exactly scores[r*score_cols + b] for
 *               b < (pos[r]+1)/4 is written; every other element is untouched.
 *   dev_status  int32 flag word; a row with pos outside [0, tokens) sets
 *               QSA_STATUS_BAD_POSITION and writes nothing.
 * Refusals: QSA_ERR_NULL, QSA_ERR_EXTENT (negative rows/tokens),
 * QSA_ERR_STRIDE (q_stride < 512, score_cols < tokens/4), QSA_ERR_CAPACITY
 * (scores_len < rows*score_cols, tokens > QSA_MAX_TOKENS), QSA_ERR_PARAM.
 */
int qsa_score_rows(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                   const uint16_t* q_norm_w, int32_t rotary_dim, float rope_theta,
                   float rms_eps, const uint16_t* pooled, int64_t tokens, float* scores,
                   int64_t score_cols, int64_t scores_len, int32_t* dev_status,
                   void* stream);

/*
 * qsa_prep_queries -- the normed, roped query heads of every row, computed
 * once per row, for qsa_score_prepped.
 *
 * [SCORE] summary: each of the row's 4 query heads is (1 + w) RMSNorm-ed with
 * q_norm_w and roped at the row's own position p, with the norm and rotary
 * conventions of qsa_pool_keys.  Splitting this step out lets the scorer
 * read finished query fragments instead of redoing the prep in every
 * workgroup that scores a slice of the row's blocks.
 *
 *   q, pos, q_norm_w, rotary_dim, rope_theta, rms_eps, tokens: as for
 *               qsa_score_rows (tokens bounds the valid positions).
 *   qhat        [rows, 4, 128] bf16, dense (row stride 512 elements), written
 *               for every row; a row with pos outside [0, tokens) is written
 *               as zeros and sets QSA_STATUS_BAD_POSITION.
 * Refusals: QSA_ERR_NULL, QSA_ERR_EXTENT (negative rows/tokens),
 * QSA_ERR_STRIDE (q_stride < 512), QSA_ERR_CAPACITY (rows > INT32_MAX,
 * tokens > QSA_MAX_TOKENS), QSA_ERR_PARAM.
 */
int qsa_prep_queries(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                     const uint16_t* q_norm_w, int32_t rotary_dim, float rope_theta,
                     float rms_eps, int64_t tokens, uint16_t* qhat, int32_t* dev_status,
                     void* stream);

/*
 * qsa_pool_prep -- qsa_pool_keys and qsa_prep_queries in one launch.
 *
 * [SCORE] summary: the scorer's two inputs, the pooled keys and the normed,
 * roped query heads, are computed independently of each other; a decode step
 * that needs both (a batch of query rows against a cache whose newest blocks
 * still need pooling) runs them in one grid instead of two dependent
 * launches.  The outputs are bit for bit those of the two calls.
 *
 *   raw_keys, key_stride, tokens, k_norm_w, first_block, n_blocks, pooled:
 *               as for qsa_pool_keys.
 *   q, q_stride, pos, rows, q_norm_w, qhat, dev_status: as for
 *               qsa_prep_queries (tokens bounds the valid positions).
 *   rotary_dim, rope_theta, rms_eps: shared by the keys and the queries.
 * n_blocks = 0 or rows = 0 runs only the other stage.  Refusals: those of
 * qsa_pool_keys and qsa_prep_queries for their arguments; the pool's
 * pointers are checked only when n_blocks > 0, the prep's when rows > 0.
 */
int qsa_pool_prep(const uint16_t* raw_keys, int64_t key_stride, int64_t tokens,
                  const uint16_t* k_norm_w, int64_t first_block, int64_t n_blocks, uint16_t* pooled,
                  const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                  const uint16_t* q_norm_w, uint16_t* qhat, int32_t rotary_dim, float rope_theta,
                  float rms_eps, int32_t* dev_status, void* stream);

/*
 * qsa_score_prepped -- qsa_score_rows on queries already prepared by
 * qsa_prep_queries.  Same scores, bit for bit, as qsa_score_rows on the raw
 * queries with the same norm and rotary arguments.
 *
 *   qhat        [rows, 4, 128] bf16 from qsa_prep_queries.
 *   pos, pooled, tokens, scores, score_cols, scores_len, dev_status: as for
 *               qsa_score_rows.
 * Refusals: as for qsa_score_rows, without the rotary/norm parameters.
 */
int qsa_score_prepped(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                      const uint16_t* pooled, int64_t tokens, float* scores,
                      int64_t score_cols, int64_t scores_len, int32_t* dev_status,
                      void* stream);

/*
 * qsa_select_mask -- exact per-row top-(budget/4) block select and the u8
 * token visibility mask.
 *
 * [SEL] "Exact semantics": for a row at position p, blocks n = (p+1)/4, tail
 * = (p+1)%4 tokens at 4n..p, keep = min(budget/4, n).  The keep first blocks
 * under the order (score descending, block index ascending; -0.0 ties +0.0)
 * are kept.  mask[r*tokens + t] = 1 for the 4 tokens of every kept block and
 * for the tail, 0 for every other t in [0, tokens).
 *
 *   scores      f32, row stride score_cols >= tokens/4, scores_len elements;
 *               only each row's first (p+1)/4 entries are read.
 *   pos         [rows] int32.
 *   budget      positive multiple of 4, budget/4 <= 512.
 *   mask        [rows, tokens] u8, every byte written.
 *   dev_status  a row with pos outside [0, tokens) sets QSA_STATUS_BAD_POSITION;
 *               a row with a non-finite score among its first (p+1)/4 sets
 *               QSA_STATUS_NONFINITE_SCORE.  Such rows are written all zero.
 * Refusals: QSA_ERR_NULL, QSA_ERR_EXTENT, QSA_ERR_BUDGET, QSA_ERR_STRIDE
 * (score_cols < tokens/4), QSA_ERR_CAPACITY (scores_len < rows*score_cols,
 * tokens > QSA_MAX_TOKENS).
 */
int qsa_select_mask(const float* scores, int64_t score_cols, int64_t scores_len,
                    const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                    uint8_t* mask, int32_t* dev_status, void* stream);

/*
 * qsa_select_indices -- the same selection as qsa_select_mask, written as
 * the list of visible token indices a sparse-attention gather consumes.
 *
 * [QSA] decode select (the host top-k it performs): the kept blocks sorted
 * ascending, each expanded to its 4 tokens 4b .. 4b + 3, then the tail tokens
 * 4n .. p; at most budget + 3 entries ([SCORE] "Next: P3": buffer bound
 * budget + ratio - 1).  Kept set and order as in [SEL] "Exact semantics".
 *
 *   scores, score_cols, scores_len, pos, rows, tokens, budget, dev_status:
 *               as for qsa_select_mask.
 *   idx         [rows, idx_stride] int32, idx_stride >= budget + 3.  Row r's
 *               entries [0, counts[r]) hold the ascending token indices,
 *               entries [counts[r], budget + 3) hold -1; columns at or past
 *               budget + 3 are untouched.  counts[r] = 4 min(budget/4, n) +
 *               (p + 1) % 4, which is p + 1 for a row under the budget.
 *   counts      [rows] int32.
 *   A refused row (position out of range, non-finite score) gets count 0 and
 *   -1 entries, and sets its QSA_STATUS_* bit.
 * Refusals: those of qsa_select_mask, and QSA_ERR_STRIDE (idx_stride <
 * budget + 3), QSA_ERR_EXTENT (idx_stride < 0), QSA_ERR_CAPACITY
 * (rows * idx_stride overflows), QSA_ERR_NULL (idx or counts NULL).
 */
int qsa_select_indices(const float* scores, int64_t score_cols, int64_t scores_len,
                       const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                       int32_t* idx, int64_t idx_stride, int32_t* counts, int32_t* dev_status,
                       void* stream);

/*
 * qsa_select_workspace_bytes -- device workspace qsa_select_mask_ws (and the
 * index-list forms qsa_select_indices_ws / _dev) needs for
 * `rows` rows over a `tokens`-token cache: 0 when it selects one workgroup
 * per row (more than 128 rows, or caches of at most 65536 + 3 tokens), else
 * 4352 bytes per 16384 tokens (rounded up) per row.  Negative QSA_ERR_EXTENT /
 * QSA_ERR_CAPACITY for negative extents or tokens > QSA_MAX_TOKENS.
 */
int64_t qsa_select_workspace_bytes(int64_t rows, int64_t tokens);

/*
 * qsa_select_mask_ws -- qsa_select_mask, same kept sets and mask bytes, for
 * batches of few long rows (decode).  [SEL] "Exact semantics" as for
 * qsa_select_mask.  When qsa_select_workspace_bytes(rows, tokens) > 0 each
 * row is split into chunks of 4096 blocks: one kernel emits every chunk's
 * exact local top-(budget/4) into the workspace (the row's kept blocks are
 * among them), a second finds the row's cut from that union and writes the
 * mask, one 16384-token slice per workgroup.  Otherwise it runs the
 * one-workgroup-per-row kernel of qsa_select_mask and ignores the workspace.
 *
 *   workspace        device memory owned by the caller, 16-byte aligned, at
 *                    least workspace_bytes >= qsa_select_workspace_bytes(rows,
 *                    tokens) long; its contents on entry do not matter and
 *                    on return are unspecified.  Two calls in flight on the
 *                    same workspace race.
 * Refusals: those of qsa_select_mask; QSA_ERR_NULL (workspace NULL when
 * needed), QSA_ERR_CAPACITY (workspace_bytes too small), QSA_ERR_EXTENT
 * (workspace_bytes < 0), QSA_ERR_PARAM (workspace not 16-byte aligned).
 */
int qsa_select_mask_ws(const float* scores, int64_t score_cols, int64_t scores_len,
                       const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                       uint8_t* mask, int32_t* dev_status, void* workspace,
                       int64_t workspace_bytes, void* stream);

/* Bytes of the device scratch array qsa_select_mask_noalloc uses (per GPU). */
#define QSA_NOALLOC_SCRATCH_BYTES (8 << 20)

/*
 * qsa_select_mask_noalloc -- qsa_select_mask_ws without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid allocation): same kept sets, mask
 * bytes and status bits.  When the split select runs (the rows and tokens
 * for which qsa_select_workspace_bytes(rows, tokens) > 0) its workspace is a
 * library-owned device array of QSA_NOALLOC_SCRATCH_BYTES, one per GPU, held
 * until the process ends; otherwise the call is qsa_select_mask.  The call
 * allocates and frees nothing; its first call on a device looks up that
 * device's array (with that device current).  Calls that overlap on one
 * GPU share the array and race: serialise them (one stream, or events).
 * Refusals: those of qsa_select_mask, and QSA_ERR_CAPACITY when the split
 * select would need more than QSA_NOALLOC_SCRATCH_BYTES (about 113 rows at
 * QSA_MAX_TOKENS tokens, 120 rows at 262144); QSA_ERR_LAUNCH if the array's
 * address cannot be obtained.
 */
int qsa_select_mask_noalloc(const float* scores, int64_t score_cols, int64_t scores_len,
                            const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                            uint8_t* mask, int32_t* dev_status, void* stream);

/*
 * qsa_score_select_workspace_bytes -- device workspace qsa_score_select_mask
 * needs for `rows` rows over a `tokens`-token cache at `budget`: a full
 * score matrix for the rows that fall back (rows * tokens bytes), sampled
 * scores (rows * tokens / 16 bytes) and candidate regions (8192 rows of 65536
 * tokens at budget 2048: 0.82 GB in all).  0 for an empty call;
 * QSA_ERR_EXTENT / QSA_ERR_BUDGET / QSA_ERR_CAPACITY as for
 * qsa_score_select_mask.
 */
int64_t qsa_score_select_workspace_bytes(int64_t rows, int64_t tokens, int64_t budget);

/*
 * qsa_score_select_mask -- qsa_score_prepped followed by qsa_select_mask, as
 * one call that does not write the block scores out: the same mask bytes and
 * status bits, bit for bit.
 *
 * [SCORE] "Next" names a fused score -> select pass for long prefill; [SEL]
 * "Exact semantics" fixes the kept set.  Each row's keep-th largest block is
 * found among the blocks scoring at or above a per-row threshold taken from
 * every 16th block's score; a row whose threshold admits fewer than
 * budget/4 blocks, or more than the workspace holds, is scored and selected
 * again in full, inside the same call.  The result never depends on the
 * threshold; the time does.  Meant for prefill batches (many rows sharing
 * one cache); it works for any batch.
 *
 *   qhat        [rows, 4, 128] bf16 from qsa_prep_queries.
 *   pos, rows, pooled, tokens, budget, mask, dev_status: as for
 *               qsa_score_prepped and qsa_select_mask.
 *   workspace   device memory owned by the caller, 256-byte aligned, at least
 *               workspace_bytes >= qsa_score_select_workspace_bytes(rows,
 *               tokens, budget) long; contents on entry do not matter, on
 *               return unspecified.  Two calls in flight on the same
 *               workspace race.
 * Refusals: QSA_ERR_EXTENT (negative rows, tokens or workspace_bytes),
 * QSA_ERR_BUDGET, QSA_ERR_CAPACITY (tokens > QSA_MAX_TOKENS, rows >
 * INT32_MAX, rows * tokens overflows, workspace_bytes too small),
 * QSA_ERR_NULL (qhat, pos, mask, dev_status or workspace NULL; pooled NULL
 * with tokens >= 4), QSA_ERR_PARAM (workspace not 256-byte aligned).
 */
int qsa_score_select_mask(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                          const uint16_t* pooled, int64_t tokens, int64_t budget, uint8_t* mask,
                          int32_t* dev_status, void* workspace, int64_t workspace_bytes,
                          void* stream);

/*
 * qsa_score_select_flags_offset -- where qsa_score_select_mask records which
 * rows it selected in full: the byte offset, within its workspace, of an
 * int32 [rows] array that a call leaves holding 1 for every row whose
 * sampled threshold did not settle it (scored and selected in full inside
 * the call) and 0 for every other row.  The mask does not depend on it; it
 * tells tests and tuning which path each row took.  0 for an empty call;
 * negative QSA_ERR_* as qsa_score_select_workspace_bytes.
 */
int64_t qsa_score_select_flags_offset(int64_t rows, int64_t tokens, int64_t budget);

/*
 * qsa_gather_kv -- each row's selected tokens' K and V vectors, copied from a
 * paged cache into contiguous per-row scratch, with the identity page table
 * that presents the scratch as a paged cache.
 *
 * [QSA] module notes and decode_select: decode selection gathers the kept
 * tokens' K/V into a contiguous NHD scratch that the paged decode attention
 * reads through an identity block table (ceil(n_sel / block_size) pages,
 * sequence length n_sel).  The token lists are qsa_select_indices' output.
 *
 *   k_cache, v_cache  [n_pages, page_size, kv_dim] bf16, dense: page, slot,
 *                     then the kv_heads x head_dim vector (kv_dim elements).
 *   page_table        int32; token t of row r lives at page
 *                     page_table[r * table_stride + t / page_size], slot t %
 *                     page_size, for t / page_size < table_len.
 *                     table_stride 0: one table for every row.
 *   idx, idx_stride, counts   row r's list: idx[r * idx_stride + i], i <
 *                     counts[r] (as qsa_select_indices writes them).
 *   slots             entries per row of the scratch, a multiple of
 *                     page_size (>= the longest list: budget + 3 rounded up).
 *   k_out, v_out      [rows, slots, kv_dim] bf16: entry i < counts[r] is the
 *                     listed token's vector, every other entry zero.
 *   out_table         [rows, slots / page_size] int32: row r's page j is
 *                     page r * (slots / page_size) + j of k_out / v_out
 *                     viewed as [rows * slots / page_size, page_size, kv_dim];
 *                     the row's sequence length is counts[r].
 *   dev_status        a token index that is negative, at or past table_len *
 *                     page_size, or whose page lies outside [0, n_pages), is
 *                     written as zeros; a count outside [0, min(slots,
 *                     idx_stride)] is clamped into it; both set
 *                     QSA_STATUS_BAD_INDEX.
 * Refusals: QSA_ERR_EXTENT (negative n_pages, table_len, table_stride,
 * idx_stride, rows or slots), QSA_ERR_PARAM (page_size or kv_dim < 1, slots
 * not a multiple of page_size), QSA_ERR_STRIDE (0 < table_stride <
 * table_len), QSA_ERR_CAPACITY (a buffer extent overflows, or
 * rows * slots / 4 > INT32_MAX), QSA_ERR_NULL (a pointer the extents make
 * necessary is NULL).  rows == 0 or slots == 0: QSA_OK, nothing enqueued.
 */
int qsa_gather_kv(const uint16_t* k_cache, const uint16_t* v_cache, int64_t n_pages,
                  int32_t page_size, int32_t kv_dim, const int32_t* page_table,
                  int64_t table_stride, int64_t table_len, const int32_t* idx,
                  int64_t idx_stride, const int32_t* counts, int64_t rows, int64_t slots,
                  uint16_t* k_out, uint16_t* v_out, int32_t* out_table, int32_t* dev_status,
                  void* stream);

/*
 * Device-geometry calls, for a decode step captured once as a HIP graph and
 * replayed while the cache grows.  A graph freezes every host argument it was
 * captured with; these calls take the live cache length from a device int32
 * (*dev_tokens, 0 <= T <= max_tokens) read when the kernels run, and size their
 * launches for max_tokens, the ceiling.  Positions (pos) are already device
 * data.  A T outside [0, max_tokens] is clamped into it and sets
 * QSA_STATUS_BAD_GEOMETRY.  Refusals are those of the host-count call with
 * tokens = max_tokens, plus QSA_ERR_NULL for a NULL dev_tokens.
 *
 * qsa_pool_window -- [QSA] pool_new_blocks: a decode step pools only the
 * blocks its new tokens completed.  Pools the last n_blocks complete blocks,
 * [max(0, T/4 - n_blocks), T/4), with qsa_pool_keys' arithmetic; pooling a
 * block again writes the same bytes, so n_blocks only has to cover the
 * blocks completed since the previous call (1 for one-token decode steps).
 * n_blocks <= max_tokens / 4 (QSA_ERR_EXTENT); 0 enqueues nothing.
 */
int qsa_pool_window(const uint16_t* raw_keys, int64_t key_stride, int64_t max_tokens,
                    const uint16_t* k_norm_w, int32_t rotary_dim, float rope_theta, float rms_eps,
                    const int32_t* dev_tokens, int64_t n_blocks, uint16_t* pooled,
                    int32_t* dev_status, void* stream);

/* qsa_prep_queries with the live cache length on the device (validity of pos). */
int qsa_prep_queries_dev(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                         const uint16_t* q_norm_w, int32_t rotary_dim, float rope_theta,
                         float rms_eps, const int32_t* dev_tokens, int64_t max_tokens,
                         uint16_t* qhat, int32_t* dev_status, void* stream);

/* qsa_pool_window and qsa_prep_queries_dev in one launch (see qsa_pool_prep):
 * the last n_blocks complete blocks of the live cache, and the batch's
 * prepared query heads.  Refusals: those of the two calls. */
int qsa_pool_prep_dev(const uint16_t* raw_keys, int64_t key_stride, int64_t max_tokens,
                      const uint16_t* k_norm_w, int64_t n_blocks, uint16_t* pooled, const uint16_t* q,
                      int64_t q_stride, const int32_t* pos, int64_t rows, const uint16_t* q_norm_w,
                      uint16_t* qhat, int32_t rotary_dim, float rope_theta, float rms_eps,
                      const int32_t* dev_tokens, int32_t* dev_status, void* stream);

/* qsa_score_prepped with the live cache length on the device; score_cols >=
 * max_tokens / 4.  Workgroups past a batch's longest visible prefix exit. */
int qsa_score_prepped_dev(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                          const uint16_t* pooled, const int32_t* dev_tokens, int64_t max_tokens,
                          float* scores, int64_t score_cols, int64_t scores_len,
                          int32_t* dev_status, void* stream);

/* qsa_select_indices_ws with the live cache length on the device; the index
 * lists do not depend on the cache length beyond the validity of pos.  The
 * workspace rules use max_tokens: qsa_select_workspace_bytes(rows,
 * max_tokens) bytes. */
int qsa_select_indices_dev(const float* scores, int64_t score_cols, int64_t scores_len,
                           const int32_t* pos, int64_t rows, const int32_t* dev_tokens,
                           int64_t max_tokens, int64_t budget, int32_t* idx, int64_t idx_stride,
                           int32_t* counts, int32_t* dev_status, void* workspace,
                           int64_t workspace_bytes, void* stream);

/*
 * qsa_select_indices_ws -- qsa_select_indices, same lists and counts, with
 * the split form of qsa_select_mask_ws for batches of few long rows: when
 * qsa_select_workspace_bytes(rows, tokens) > 0, the chunks' local top lists
 * go to the workspace and one workgroup per (row, 16384-token slice) writes
 * the slice's kept tokens at the position the earlier slices' kept blocks
 * leave free.  Otherwise it is qsa_select_indices and ignores the workspace.
 * Arguments and refusals: those of qsa_select_indices, and the workspace
 * rules of qsa_select_mask_ws.
 */
int qsa_select_indices_ws(const float* scores, int64_t score_cols, int64_t scores_len,
                          const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                          int32_t* idx, int64_t idx_stride, int32_t* counts, int32_t* dev_status,
                          void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qsa_rope_inv_freq -- host only: the rotary frequencies the kernels use,
 * out[i] = (float)(theta^(-2i/rotary_dim)) evaluated in double, i < rotary_dim/2.
 * Returns QSA_ERR_NULL / QSA_ERR_PARAM on bad arguments.
 */
int qsa_rope_inv_freq(int32_t rotary_dim, float rope_theta, float* out);

/* Static description of a return code.  Never NULL. */
const char* qsa_strerror(int code);

/* QSA_ABI_VERSION of the loaded library. */
int qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
