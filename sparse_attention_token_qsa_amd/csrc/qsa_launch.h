// Internal launch interface between the C ABI layer and the kernels.
// Arguments reach here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

struct RopeParams {
  int rotary_dim;
  float eps;
  float inv_freq[64];
};

// With dev_tokens set: pool the last n_blocks complete blocks of a cache of
// *dev_tokens tokens (ceiling at most), first_block unused.
hipError_t launch_pool(const uint16_t* raw, int64_t key_stride, const uint16_t* w,
                       const RopeParams& rp, int64_t first_block, int64_t n_blocks,
                       uint16_t* pooled, hipStream_t stream, const int32_t* dev_tokens = nullptr,
                       int64_t ceiling = 0, int32_t* status = nullptr);

hipError_t launch_score(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                        const uint16_t* w, const RopeParams& rp, const uint16_t* pooled,
                        int64_t tokens, float* scores, int64_t score_cols, int32_t* status,
                        hipStream_t stream);

// dev_tokens (optional, below): a device int32 holding the live cache length;
// `tokens` is then its ceiling (launch geometry and buffer extents).
hipError_t launch_prep(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                       const uint16_t* w, const RopeParams& rp, int64_t tokens, uint16_t* qhat,
                       int32_t* status, hipStream_t stream, const int32_t* dev_tokens = nullptr);

// The pool of a block range and the prep of a batch of query rows in one
// launch (pool_prep.hip).  With dev_tokens set, the pool takes the last
// n_blocks complete blocks of the live cache (first_block unused) and
// `tokens` is the ceiling, as for launch_pool and launch_prep.
hipError_t launch_pool_prep(const uint16_t* raw, int64_t key_stride, const uint16_t* wk,
                            int64_t first_block, int64_t n_blocks, uint16_t* pooled,
                            const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                            const uint16_t* wq, uint16_t* qhat, const RopeParams& rp, int64_t tokens,
                            int32_t* status, hipStream_t stream, const int32_t* dev_tokens = nullptr);

hipError_t launch_score_prepped(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                                const uint16_t* pooled, int64_t tokens, float* scores,
                                int64_t score_cols, int32_t* status, hipStream_t stream,
                                const int32_t* dev_tokens = nullptr);

hipError_t launch_select(const float* scores, int64_t score_cols, const int32_t* pos,
                         int64_t rows, int64_t tokens, int keep_max, uint8_t* mask,
                         int32_t* status, hipStream_t stream);

// Index-list output of the one-workgroup-per-row selector (select.hip).
hipError_t launch_select_indices(const float* scores, int64_t score_cols, const int32_t* pos,
                                 int64_t rows, int64_t tokens, int keep_max, int32_t* idx,
                                 int64_t idx_stride, int32_t* counts, int32_t* status,
                                 hipStream_t stream, const int32_t* dev_tokens = nullptr);

// Split select for few long rows (select_split.hip): two launches over a
// caller-provided workspace of select_split_workspace_bytes(rows, tokens).
bool select_split_pays(int64_t rows, int64_t tokens);
int64_t select_split_workspace_bytes(int64_t rows, int64_t tokens);
hipError_t launch_select_split(const float* scores, int64_t score_cols, const int32_t* pos,
                               int64_t rows, int64_t tokens, int keep_max, uint8_t* mask,
                               int32_t* status, void* workspace, hipStream_t stream);
// The device address, on the current device, of the library's scratch array
// for qsa_select_mask_noalloc (QSA_NOALLOC_SCRATCH_BYTES); looked up once per
// device, no allocation.
hipError_t noalloc_scratch(void** out);
// The same split, writing index lists (qsa_select_indices' format).
hipError_t launch_select_split_indices(const float* scores, int64_t score_cols, const int32_t* pos,
                                       int64_t rows, int64_t tokens, int keep_max, int32_t* idx,
                                       int64_t idx_stride, int32_t* counts, int32_t* status,
                                       void* workspace, hipStream_t stream,
                                       const int32_t* dev_tokens = nullptr);

// One-workgroup-per-row selector over the rows whose row_flag is nonzero
// only (the others are left untouched): the fused path's fallback.
hipError_t launch_select_flagged(const float* scores, int64_t score_cols, const int32_t* pos,
                                 int64_t rows, int64_t tokens, int keep_max, uint8_t* mask,
                                 int32_t* status, const int32_t* row_flag, hipStream_t stream);

// Ring scorer jobs (score.hip): prepared queries in groups of kRingRows rows,
// pooled keys streamed through LDS.  Column j of a row scores the pooled key
// of block j * bstride; row r has ceil(((pos[r] + 1) / 4) / bstride) columns.
// With cand == NULL the scores go to scores[r * score_cols + j].  Otherwise
// nothing is stored but the blocks whose score has bits >= thr[r] (as
// unsigned integers), as (score bits, block) entries in
// cand[((r * splits + split) * 4 + g) * cap + e], e < cap, where g = (block
// % 32) / 8, with the per-region totals in cnt[(r * splits + split) * 4 + g].
// group_flag, when set, restricts the job to row groups whose flag is nonzero.
constexpr int kRingRows = 128;
struct RingJob {
  const uint16_t* qhat;
  const int32_t* pos;
  int64_t rows;
  const uint16_t* pooled;
  int64_t tokens;
  int bstride;
  float* scores;
  int64_t score_cols;
  int32_t* status;
  const int32_t* group_flag;
  const uint32_t* thr;  // padded to a multiple of kRingRows rows
  uint2* cand;
  int32_t* cnt;
  int cap;
};
// splits per row group of a job over `cols` columns with `target` workgroups
int64_t ring_splits(int64_t rows, int64_t cols, int64_t target);
hipError_t launch_ring(const RingJob& j, int64_t target, hipStream_t stream);

// Decode K/V gather from a paged cache (gather.hip).
hipError_t launch_gather_kv(const uint16_t* k, const uint16_t* v, int64_t n_pages, int page_size,
                            int kv_dim, const int32_t* table, int64_t table_stride, int64_t table_len,
                            const int32_t* idx, int64_t idx_stride, const int32_t* counts, int64_t rows,
                            int64_t slots, uint16_t* ko, uint16_t* vo, int32_t* otable, int32_t* status,
                            hipStream_t stream);

// Fused score -> select for prefill batches (fused.hip).
int64_t score_select_workspace_bytes(int64_t rows, int64_t tokens, int keep_max);
// byte offset of the per-row fallback flags (int32 [rows]) in that workspace
int64_t score_select_flags_offset(int64_t rows, int64_t tokens, int keep_max);
hipError_t launch_score_select(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                               const uint16_t* pooled, int64_t tokens, int keep_max,
                               uint8_t* mask, int32_t* status, void* workspace,
                               hipStream_t stream);

}  // namespace qsa
