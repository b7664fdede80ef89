// C ABI of libqsa.so: argument refusals, rotary table, launches.
// Contract and citations: include/qsa.h.  Every refusal returns before any
// HIP call, so this layer is exercised without a GPU.
#include <math.h>
#include <stdint.h>

#include "../../include/qsa.h"
#include "qsa_launch.h"

namespace {

bool mul_overflows(int64_t a, int64_t b, int64_t* out) {
  return __builtin_mul_overflow(a, b, out);
}

int check_rope(int32_t rotary_dim, float theta, float eps) {
  if (rotary_dim < 0 || rotary_dim > QSA_HEAD_DIM || (rotary_dim & 1)) return QSA_ERR_PARAM;
  if (!(theta > 0.0f) || !isfinite(theta)) return QSA_ERR_PARAM;
  if (!(eps >= 0.0f) || !isfinite(eps)) return QSA_ERR_PARAM;
  return QSA_OK;
}

void fill_inv_freq(int32_t rotary_dim, float theta, float* out) {
  const int half = rotary_dim / 2;
  for (int i = 0; i < half; ++i)
    out[i] = static_cast<float>(pow(static_cast<double>(theta), -(2.0 * i) / static_cast<double>(rotary_dim)));
}

int launch_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH; }

// Refusals of qsa_pool_prep(_dev) past its extents: those of the pool call for
// its key arguments and of the prep call for its query arguments.  The pool's
// pointers are needed only when n_blocks > 0, the prep's when rows > 0.
int check_pool_prep(const uint16_t* raw_keys, int64_t key_stride, int64_t tokens,
                    const uint16_t* k_norm_w, int64_t n_blocks, const uint16_t* pooled,
                    const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                    const uint16_t* q_norm_w, const uint16_t* qhat, int32_t rotary_dim,
                    float rope_theta, float rms_eps, const int32_t* dev_status) {
  if (key_stride < QSA_HEAD_DIM || q_stride < QSA_HEADS * QSA_HEAD_DIM) return QSA_ERR_STRIDE;
  const int rc = check_rope(rotary_dim, rope_theta, rms_eps);
  if (rc != QSA_OK) return rc;
  if (tokens > QSA_MAX_TOKENS || rows > INT32_MAX) return QSA_ERR_CAPACITY;
  int64_t need;
  if (n_blocks > 0) {
    if (raw_keys == nullptr || k_norm_w == nullptr || pooled == nullptr) return QSA_ERR_NULL;
    if (mul_overflows(tokens, key_stride, &need)) return QSA_ERR_CAPACITY;
  }
  if (rows > 0) {
    if (q == nullptr || pos == nullptr || q_norm_w == nullptr || qhat == nullptr || dev_status == nullptr)
      return QSA_ERR_NULL;
    if (mul_overflows(rows, q_stride, &need)) return QSA_ERR_CAPACITY;
  }
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char* qsa_strerror(int code) {
  switch (code) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "qsa: a required pointer is NULL";
    case QSA_ERR_EXTENT: return "qsa: negative extent or block range past tokens/4";
    case QSA_ERR_BUDGET: return "qsa: budget must be a positive multiple of 4 with budget/4 <= 512";
    case QSA_ERR_STRIDE: return "qsa: a row stride is narrower than its row";
    case QSA_ERR_CAPACITY: return "qsa: output buffer too short or tokens above the supported maximum";
    case QSA_ERR_PARAM: return "qsa: rotary_dim, rope_theta or rms_eps out of range";
    case QSA_ERR_LAUNCH: return "qsa: the HIP runtime refused the launch";
    default: return "qsa: unknown error code";
  }
}

int qsa_rope_inv_freq(int32_t rotary_dim, float rope_theta, float* out) {
  const int rc = check_rope(rotary_dim, rope_theta, 0.0f);
  if (rc != QSA_OK) return rc;
  if (rotary_dim > 0 && out == nullptr) return QSA_ERR_NULL;
  fill_inv_freq(rotary_dim, rope_theta, out);
  return QSA_OK;
}

int qsa_pool_keys(const uint16_t* raw_keys, int64_t key_stride, int64_t tokens,
                  const uint16_t* k_norm_w, int32_t rotary_dim, float rope_theta,
                  float rms_eps, int64_t first_block, int64_t n_blocks, uint16_t* pooled,
                  void* stream) {
  if (tokens < 0 || first_block < 0 || n_blocks < 0) return QSA_ERR_EXTENT;
  if (first_block > tokens / QSA_RATIO || n_blocks > tokens / QSA_RATIO - first_block)
    return QSA_ERR_EXTENT;
  if (key_stride < QSA_HEAD_DIM) return QSA_ERR_STRIDE;
  const int rc = check_rope(rotary_dim, rope_theta, rms_eps);
  if (rc != QSA_OK) return rc;
  if (n_blocks == 0) return QSA_OK;
  if (raw_keys == nullptr || k_norm_w == nullptr || pooled == nullptr) return QSA_ERR_NULL;
  int64_t span;
  if (mul_overflows(tokens, key_stride, &span)) return QSA_ERR_CAPACITY;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_pool(raw_keys, key_stride, k_norm_w, rp, first_block,
                                        n_blocks, pooled, static_cast<hipStream_t>(stream)));
}

int qsa_score_rows(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                   const uint16_t* q_norm_w, int32_t rotary_dim, float rope_theta,
                   float rms_eps, const uint16_t* pooled, int64_t tokens, float* scores,
                   int64_t score_cols, int64_t scores_len, int32_t* dev_status, void* stream) {
  if (rows < 0 || tokens < 0 || score_cols < 0 || scores_len < 0) return QSA_ERR_EXTENT;
  if (q_stride < QSA_HEADS * QSA_HEAD_DIM) return QSA_ERR_STRIDE;
  if (score_cols < tokens / QSA_RATIO) return QSA_ERR_STRIDE;
  const int rc = check_rope(rotary_dim, rope_theta, rms_eps);
  if (rc != QSA_OK) return rc;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, score_cols, &need) || scores_len < need) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0) return QSA_OK;
  if (q == nullptr || pos == nullptr || q_norm_w == nullptr || dev_status == nullptr)
    return QSA_ERR_NULL;
  if (tokens >= QSA_RATIO && (pooled == nullptr || scores == nullptr)) return QSA_ERR_NULL;
  if (mul_overflows(rows, q_stride, &need)) return QSA_ERR_CAPACITY;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_score(q, q_stride, pos, rows, q_norm_w, rp, pooled, tokens,
                                         scores, score_cols, dev_status,
                                         static_cast<hipStream_t>(stream)));
}

int qsa_prep_queries(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                     const uint16_t* q_norm_w, int32_t rotary_dim, float rope_theta,
                     float rms_eps, int64_t tokens, uint16_t* qhat, int32_t* dev_status,
                     void* stream) {
  if (rows < 0 || tokens < 0) return QSA_ERR_EXTENT;
  if (q_stride < QSA_HEADS * QSA_HEAD_DIM) return QSA_ERR_STRIDE;
  const int rc = check_rope(rotary_dim, rope_theta, rms_eps);
  if (rc != QSA_OK) return rc;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0) return QSA_OK;
  if (q == nullptr || pos == nullptr || q_norm_w == nullptr || qhat == nullptr ||
      dev_status == nullptr)
    return QSA_ERR_NULL;
  int64_t need;
  if (mul_overflows(rows, q_stride, &need)) return QSA_ERR_CAPACITY;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_prep(q, q_stride, pos, rows, q_norm_w, rp, tokens, qhat,
                                        dev_status, static_cast<hipStream_t>(stream)));
}

int qsa_pool_prep(const uint16_t* raw_keys, int64_t key_stride, int64_t tokens,
                  const uint16_t* k_norm_w, int64_t first_block, int64_t n_blocks, uint16_t* pooled,
                  const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                  const uint16_t* q_norm_w, uint16_t* qhat, int32_t rotary_dim, float rope_theta,
                  float rms_eps, int32_t* dev_status, void* stream) {
  if (tokens < 0 || first_block < 0 || n_blocks < 0 || rows < 0) return QSA_ERR_EXTENT;
  if (first_block > tokens / QSA_RATIO || n_blocks > tokens / QSA_RATIO - first_block)
    return QSA_ERR_EXTENT;
  const int rc = check_pool_prep(raw_keys, key_stride, tokens, k_norm_w, n_blocks, pooled, q, q_stride,
                                 pos, rows, q_norm_w, qhat, rotary_dim, rope_theta, rms_eps, dev_status);
  if (rc != QSA_OK) return rc;
  if (n_blocks == 0 && rows == 0) return QSA_OK;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_pool_prep(raw_keys, key_stride, k_norm_w, first_block, n_blocks, pooled,
                                             q, q_stride, pos, rows, q_norm_w, qhat, rp, tokens,
                                             dev_status, static_cast<hipStream_t>(stream)));
}

int qsa_score_prepped(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                      const uint16_t* pooled, int64_t tokens, float* scores,
                      int64_t score_cols, int64_t scores_len, int32_t* dev_status,
                      void* stream) {
  if (rows < 0 || tokens < 0 || score_cols < 0 || scores_len < 0) return QSA_ERR_EXTENT;
  if (score_cols < tokens / QSA_RATIO) return QSA_ERR_STRIDE;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, score_cols, &need) || scores_len < need) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0) return QSA_OK;
  if (qhat == nullptr || pos == nullptr || dev_status == nullptr) return QSA_ERR_NULL;
  if (tokens >= QSA_RATIO && (pooled == nullptr || scores == nullptr)) return QSA_ERR_NULL;
  return launch_status(qsa::launch_score_prepped(qhat, pos, rows, pooled, tokens, scores,
                                                 score_cols, dev_status,
                                                 static_cast<hipStream_t>(stream)));
}

namespace {
int check_select(const float* scores, int64_t score_cols, int64_t scores_len, const int32_t* pos,
                 int64_t rows, int64_t tokens, int64_t budget, uint8_t* mask, int32_t* dev_status) {
  if (rows < 0 || tokens < 0 || score_cols < 0 || scores_len < 0) return QSA_ERR_EXTENT;
  if (budget <= 0 || budget % QSA_RATIO != 0 || budget / QSA_RATIO > QSA_MAX_KEEP_BLOCKS)
    return QSA_ERR_BUDGET;
  if (score_cols < tokens / QSA_RATIO) return QSA_ERR_STRIDE;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, score_cols, &need) || scores_len < need) return QSA_ERR_CAPACITY;
  if (mul_overflows(rows, tokens, &need)) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;  // one workgroup per row
  if (rows == 0 || tokens == 0) return QSA_OK;
  if (pos == nullptr || mask == nullptr || dev_status == nullptr) return QSA_ERR_NULL;
  if (tokens >= QSA_RATIO && scores == nullptr) return QSA_ERR_NULL;
  return 1;  // valid and not empty
}
}  // namespace

int qsa_select_mask(const float* scores, int64_t score_cols, int64_t scores_len,
                    const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                    uint8_t* mask, int32_t* dev_status, void* stream) {
  const int rc = check_select(scores, score_cols, scores_len, pos, rows, tokens, budget, mask, dev_status);
  if (rc <= 0) return rc;
  return launch_status(qsa::launch_select(scores, score_cols, pos, rows, tokens,
                                          static_cast<int>(budget / QSA_RATIO), mask,
                                          dev_status, static_cast<hipStream_t>(stream)));
}

int qsa_select_indices(const float* scores, int64_t score_cols, int64_t scores_len,
                       const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                       int32_t* idx, int64_t idx_stride, int32_t* counts, int32_t* dev_status,
                       void* stream) {
  if (rows < 0 || tokens < 0 || score_cols < 0 || scores_len < 0 || idx_stride < 0) return QSA_ERR_EXTENT;
  if (budget <= 0 || budget % QSA_RATIO != 0 || budget / QSA_RATIO > QSA_MAX_KEEP_BLOCKS)
    return QSA_ERR_BUDGET;
  if (score_cols < tokens / QSA_RATIO) return QSA_ERR_STRIDE;
  if (idx_stride < budget + QSA_RATIO - 1) return QSA_ERR_STRIDE;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, score_cols, &need) || scores_len < need) return QSA_ERR_CAPACITY;
  if (mul_overflows(rows, idx_stride, &need)) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0) return QSA_OK;
  if (pos == nullptr || idx == nullptr || counts == nullptr || dev_status == nullptr) return QSA_ERR_NULL;
  if (tokens >= QSA_RATIO && scores == nullptr) return QSA_ERR_NULL;
  return launch_status(qsa::launch_select_indices(scores, score_cols, pos, rows, tokens,
                                                  static_cast<int>(budget / QSA_RATIO), idx, idx_stride,
                                                  counts, dev_status, static_cast<hipStream_t>(stream)));
}

int64_t qsa_select_workspace_bytes(int64_t rows, int64_t tokens) {
  if (rows < 0 || tokens < 0) return QSA_ERR_EXTENT;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0 || !qsa::select_split_pays(rows, tokens)) return 0;
  return qsa::select_split_workspace_bytes(rows, tokens);
}

int qsa_select_mask_ws(const float* scores, int64_t score_cols, int64_t scores_len,
                       const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                       uint8_t* mask, int32_t* dev_status, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  const int rc = check_select(scores, score_cols, scores_len, pos, rows, tokens, budget, mask, dev_status);
  if (rc <= 0) return rc;
  if (workspace_bytes < 0) return QSA_ERR_EXTENT;
  const int keep_max = static_cast<int>(budget / QSA_RATIO);
  if (!qsa::select_split_pays(rows, tokens))
    return launch_status(qsa::launch_select(scores, score_cols, pos, rows, tokens, keep_max, mask,
                                            dev_status, static_cast<hipStream_t>(stream)));
  if (workspace == nullptr) return QSA_ERR_NULL;
  if (workspace_bytes < qsa::select_split_workspace_bytes(rows, tokens)) return QSA_ERR_CAPACITY;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return QSA_ERR_PARAM;
  return launch_status(qsa::launch_select_split(scores, score_cols, pos, rows, tokens, keep_max, mask,
                                                dev_status, workspace, static_cast<hipStream_t>(stream)));
}

int qsa_select_mask_noalloc(const float* scores, int64_t score_cols, int64_t scores_len,
                            const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                            uint8_t* mask, int32_t* dev_status, void* stream) {
  const int rc = check_select(scores, score_cols, scores_len, pos, rows, tokens, budget, mask, dev_status);
  if (rc <= 0) return rc;
  const int keep_max = static_cast<int>(budget / QSA_RATIO);
  if (!qsa::select_split_pays(rows, tokens))
    return launch_status(qsa::launch_select(scores, score_cols, pos, rows, tokens, keep_max, mask,
                                            dev_status, static_cast<hipStream_t>(stream)));
  if (qsa::select_split_workspace_bytes(rows, tokens) > QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_CAPACITY;
  void* ws = nullptr;
  if (qsa::noalloc_scratch(&ws) != hipSuccess) return QSA_ERR_LAUNCH;
  return launch_status(qsa::launch_select_split(scores, score_cols, pos, rows, tokens, keep_max, mask,
                                                dev_status, ws, static_cast<hipStream_t>(stream)));
}

int64_t qsa_score_select_workspace_bytes(int64_t rows, int64_t tokens, int64_t budget) {
  if (rows < 0 || tokens < 0) return QSA_ERR_EXTENT;
  if (budget <= 0 || budget % QSA_RATIO != 0 || budget / QSA_RATIO > QSA_MAX_KEEP_BLOCKS)
    return QSA_ERR_BUDGET;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0) return 0;
  return qsa::score_select_workspace_bytes(rows, tokens, static_cast<int>(budget / QSA_RATIO));
}

int64_t qsa_score_select_flags_offset(int64_t rows, int64_t tokens, int64_t budget) {
  const int64_t n = qsa_score_select_workspace_bytes(rows, tokens, budget);
  if (n <= 0) return n;
  return qsa::score_select_flags_offset(rows, tokens, static_cast<int>(budget / QSA_RATIO));
}

int qsa_score_select_mask(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                          const uint16_t* pooled, int64_t tokens, int64_t budget, uint8_t* mask,
                          int32_t* dev_status, void* workspace, int64_t workspace_bytes,
                          void* stream) {
  if (rows < 0 || tokens < 0 || workspace_bytes < 0) return QSA_ERR_EXTENT;
  if (budget <= 0 || budget % QSA_RATIO != 0 || budget / QSA_RATIO > QSA_MAX_KEEP_BLOCKS)
    return QSA_ERR_BUDGET;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, tokens, &need)) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0) return QSA_OK;
  if (qhat == nullptr || pos == nullptr || mask == nullptr || dev_status == nullptr ||
      workspace == nullptr)
    return QSA_ERR_NULL;
  if (tokens >= QSA_RATIO && pooled == nullptr) return QSA_ERR_NULL;
  const int keep_max = static_cast<int>(budget / QSA_RATIO);
  if (workspace_bytes < qsa::score_select_workspace_bytes(rows, tokens, keep_max)) return QSA_ERR_CAPACITY;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return QSA_ERR_PARAM;
  return launch_status(qsa::launch_score_select(qhat, pos, rows, pooled, tokens, keep_max, mask, dev_status,
                                                workspace, static_cast<hipStream_t>(stream)));
}

int qsa_gather_kv(const uint16_t* k_cache, const uint16_t* v_cache, int64_t n_pages,
                  int32_t page_size, int32_t kv_dim, const int32_t* page_table,
                  int64_t table_stride, int64_t table_len, const int32_t* idx,
                  int64_t idx_stride, const int32_t* counts, int64_t rows, int64_t slots,
                  uint16_t* k_out, uint16_t* v_out, int32_t* out_table, int32_t* dev_status,
                  void* stream) {
  if (n_pages < 0 || table_len < 0 || table_stride < 0 || idx_stride < 0 || rows < 0 || slots < 0)
    return QSA_ERR_EXTENT;
  if (page_size < 1 || kv_dim < 1 || slots % page_size != 0) return QSA_ERR_PARAM;
  if (table_stride != 0 && table_stride < table_len) return QSA_ERR_STRIDE;
  int64_t need, span;
  if (mul_overflows(rows, slots, &need) || mul_overflows(need, kv_dim, &span) || need / 4 > INT32_MAX)
    return QSA_ERR_CAPACITY;
  if (mul_overflows(n_pages, page_size, &need) || mul_overflows(need, kv_dim, &span))
    return QSA_ERR_CAPACITY;
  if (mul_overflows(rows, idx_stride, &need) || mul_overflows(rows, table_stride, &need))
    return QSA_ERR_CAPACITY;
  if (rows == 0 || slots == 0) return QSA_OK;
  if (k_out == nullptr || v_out == nullptr || out_table == nullptr || counts == nullptr ||
      dev_status == nullptr)
    return QSA_ERR_NULL;
  if (idx_stride > 0 && idx == nullptr) return QSA_ERR_NULL;
  if (table_len > 0 && page_table == nullptr) return QSA_ERR_NULL;
  if (n_pages > 0 && (k_cache == nullptr || v_cache == nullptr)) return QSA_ERR_NULL;
  return launch_status(qsa::launch_gather_kv(k_cache, v_cache, n_pages, page_size, kv_dim, page_table,
                                             table_stride, table_len, idx, idx_stride, counts, rows, slots,
                                             k_out, v_out, out_table, dev_status,
                                             static_cast<hipStream_t>(stream)));
}

int qsa_pool_window(const uint16_t* raw_keys, int64_t key_stride, int64_t max_tokens,
                    const uint16_t* k_norm_w, int32_t rotary_dim, float rope_theta, float rms_eps,
                    const int32_t* dev_tokens, int64_t n_blocks, uint16_t* pooled,
                    int32_t* dev_status, void* stream) {
  if (max_tokens < 0 || n_blocks < 0) return QSA_ERR_EXTENT;
  if (n_blocks > max_tokens / QSA_RATIO) return QSA_ERR_EXTENT;
  if (key_stride < QSA_HEAD_DIM) return QSA_ERR_STRIDE;
  const int rc = check_rope(rotary_dim, rope_theta, rms_eps);
  if (rc != QSA_OK) return rc;
  if (max_tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  if (n_blocks == 0) return QSA_OK;
  if (raw_keys == nullptr || k_norm_w == nullptr || pooled == nullptr || dev_tokens == nullptr ||
      dev_status == nullptr)
    return QSA_ERR_NULL;
  int64_t span;
  if (mul_overflows(max_tokens, key_stride, &span)) return QSA_ERR_CAPACITY;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_pool(raw_keys, key_stride, k_norm_w, rp, 0, n_blocks, pooled,
                                        static_cast<hipStream_t>(stream), dev_tokens, max_tokens,
                                        dev_status));
}

int qsa_prep_queries_dev(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                         const uint16_t* q_norm_w, int32_t rotary_dim, float rope_theta,
                         float rms_eps, const int32_t* dev_tokens, int64_t max_tokens,
                         uint16_t* qhat, int32_t* dev_status, void* stream) {
  if (rows < 0 || max_tokens < 0) return QSA_ERR_EXTENT;
  if (q_stride < QSA_HEADS * QSA_HEAD_DIM) return QSA_ERR_STRIDE;
  const int rc = check_rope(rotary_dim, rope_theta, rms_eps);
  if (rc != QSA_OK) return rc;
  if (max_tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0) return QSA_OK;
  if (q == nullptr || pos == nullptr || q_norm_w == nullptr || qhat == nullptr ||
      dev_status == nullptr || dev_tokens == nullptr)
    return QSA_ERR_NULL;
  int64_t need;
  if (mul_overflows(rows, q_stride, &need)) return QSA_ERR_CAPACITY;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_prep(q, q_stride, pos, rows, q_norm_w, rp, max_tokens, qhat, dev_status,
                                        static_cast<hipStream_t>(stream), dev_tokens));
}

int qsa_pool_prep_dev(const uint16_t* raw_keys, int64_t key_stride, int64_t max_tokens,
                      const uint16_t* k_norm_w, int64_t n_blocks, uint16_t* pooled, const uint16_t* q,
                      int64_t q_stride, const int32_t* pos, int64_t rows, const uint16_t* q_norm_w,
                      uint16_t* qhat, int32_t rotary_dim, float rope_theta, float rms_eps,
                      const int32_t* dev_tokens, int32_t* dev_status, void* stream) {
  if (max_tokens < 0 || n_blocks < 0 || rows < 0) return QSA_ERR_EXTENT;
  if (n_blocks > max_tokens / QSA_RATIO) return QSA_ERR_EXTENT;
  const int rc = check_pool_prep(raw_keys, key_stride, max_tokens, k_norm_w, n_blocks, pooled, q, q_stride,
                                 pos, rows, q_norm_w, qhat, rotary_dim, rope_theta, rms_eps, dev_status);
  if (rc != QSA_OK) return rc;
  if (n_blocks == 0 && rows == 0) return QSA_OK;
  if (dev_tokens == nullptr || dev_status == nullptr) return QSA_ERR_NULL;
  qsa::RopeParams rp{};
  rp.rotary_dim = rotary_dim;
  rp.eps = rms_eps;
  fill_inv_freq(rotary_dim, rope_theta, rp.inv_freq);
  return launch_status(qsa::launch_pool_prep(raw_keys, key_stride, k_norm_w, 0, n_blocks, pooled, q,
                                             q_stride, pos, rows, q_norm_w, qhat, rp, max_tokens,
                                             dev_status, static_cast<hipStream_t>(stream), dev_tokens));
}

int qsa_score_prepped_dev(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                          const uint16_t* pooled, const int32_t* dev_tokens, int64_t max_tokens,
                          float* scores, int64_t score_cols, int64_t scores_len,
                          int32_t* dev_status, void* stream) {
  if (rows < 0 || max_tokens < 0 || score_cols < 0 || scores_len < 0) return QSA_ERR_EXTENT;
  if (score_cols < max_tokens / QSA_RATIO) return QSA_ERR_STRIDE;
  if (max_tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, score_cols, &need) || scores_len < need) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0 || max_tokens == 0) return QSA_OK;
  if (qhat == nullptr || pos == nullptr || dev_status == nullptr || dev_tokens == nullptr) return QSA_ERR_NULL;
  if (max_tokens >= QSA_RATIO && (pooled == nullptr || scores == nullptr)) return QSA_ERR_NULL;
  return launch_status(qsa::launch_score_prepped(qhat, pos, rows, pooled, max_tokens, scores, score_cols,
                                                 dev_status, static_cast<hipStream_t>(stream), dev_tokens));
}

namespace {
// Refusals of the index-list selectors (host checks only); 1 = valid, not empty.
int check_indices(const float* scores, int64_t score_cols, int64_t scores_len, const int32_t* pos,
                  int64_t rows, int64_t tokens, int64_t budget, int32_t* idx, int64_t idx_stride,
                  int32_t* counts, int32_t* dev_status) {
  if (rows < 0 || tokens < 0 || score_cols < 0 || scores_len < 0 || idx_stride < 0) return QSA_ERR_EXTENT;
  if (budget <= 0 || budget % QSA_RATIO != 0 || budget / QSA_RATIO > QSA_MAX_KEEP_BLOCKS)
    return QSA_ERR_BUDGET;
  if (score_cols < tokens / QSA_RATIO) return QSA_ERR_STRIDE;
  if (idx_stride < budget + QSA_RATIO - 1) return QSA_ERR_STRIDE;
  if (tokens > QSA_MAX_TOKENS) return QSA_ERR_CAPACITY;
  int64_t need;
  if (mul_overflows(rows, score_cols, &need) || scores_len < need) return QSA_ERR_CAPACITY;
  if (mul_overflows(rows, idx_stride, &need)) return QSA_ERR_CAPACITY;
  if (rows > INT32_MAX) return QSA_ERR_CAPACITY;
  if (rows == 0 || tokens == 0) return QSA_OK;
  if (pos == nullptr || idx == nullptr || counts == nullptr || dev_status == nullptr) return QSA_ERR_NULL;
  if (tokens >= QSA_RATIO && scores == nullptr) return QSA_ERR_NULL;
  return 1;
}

// The one-workgroup-per-row or the split index-list selector.
int launch_indices(const float* scores, int64_t score_cols, const int32_t* pos, int64_t rows, int64_t tokens,
                   int64_t budget, int32_t* idx, int64_t idx_stride, int32_t* counts, int32_t* dev_status,
                   void* workspace, int64_t workspace_bytes, void* stream, const int32_t* dev_tokens) {
  if (workspace_bytes < 0) return QSA_ERR_EXTENT;
  const int keep_max = static_cast<int>(budget / QSA_RATIO);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!qsa::select_split_pays(rows, tokens))
    return launch_status(qsa::launch_select_indices(scores, score_cols, pos, rows, tokens, keep_max, idx,
                                                    idx_stride, counts, dev_status, s, dev_tokens));
  if (workspace == nullptr) return QSA_ERR_NULL;
  if (workspace_bytes < qsa::select_split_workspace_bytes(rows, tokens)) return QSA_ERR_CAPACITY;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return QSA_ERR_PARAM;
  return launch_status(qsa::launch_select_split_indices(scores, score_cols, pos, rows, tokens, keep_max, idx,
                                                        idx_stride, counts, dev_status, workspace, s, dev_tokens));
}
}  // namespace

int qsa_select_indices_ws(const float* scores, int64_t score_cols, int64_t scores_len,
                          const int32_t* pos, int64_t rows, int64_t tokens, int64_t budget,
                          int32_t* idx, int64_t idx_stride, int32_t* counts, int32_t* dev_status,
                          void* workspace, int64_t workspace_bytes, void* stream) {
  const int rc = check_indices(scores, score_cols, scores_len, pos, rows, tokens, budget, idx, idx_stride,
                               counts, dev_status);
  if (rc <= 0) return rc;
  return launch_indices(scores, score_cols, pos, rows, tokens, budget, idx, idx_stride, counts, dev_status,
                        workspace, workspace_bytes, stream, nullptr);
}

int qsa_select_indices_dev(const float* scores, int64_t score_cols, int64_t scores_len,
                           const int32_t* pos, int64_t rows, const int32_t* dev_tokens,
                           int64_t max_tokens, int64_t budget, int32_t* idx, int64_t idx_stride,
                           int32_t* counts, int32_t* dev_status, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  const int rc = check_indices(scores, score_cols, scores_len, pos, rows, max_tokens, budget, idx, idx_stride,
                               counts, dev_status);
  if (rc <= 0) return rc;
  if (dev_tokens == nullptr) return QSA_ERR_NULL;
  return launch_indices(scores, score_cols, pos, rows, max_tokens, budget, idx, idx_stride, counts, dev_status,
                        workspace, workspace_bytes, stream, dev_tokens);
}

}  // extern "C"
