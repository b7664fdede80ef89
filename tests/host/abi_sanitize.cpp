// Host-only build of the C-ABI layer (qsa_abi.hip) for AddressSanitizer and
// UndefinedBehaviorSanitizer.  The kernel launchers are replaced by stubs
// that never touch device memory: they check the invariants the launched
// kernels rely on (extents validated, sizes in range) and count launches.
// main() sweeps every entry point over valid, refused and extreme argument
// combinations (deterministic), checks that every return is QSA_OK or a
// documented QSA_ERR_* code, and checks a handful of exact refusals.
// Built and run by tests/test_abi_sanitizers.py with g++ -fsanitize=...
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../sparse_attention_token_qsa_amd/csrc/qsa_abi.hip"

static long g_launches = 0;
static int g_fail = 0;

#define REQUIRE(c)                                                    \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "%s:%d: requirement failed: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                       \
      std::abort();                                                   \
    }                                                                 \
  } while (0)

namespace qsa {

static void check_rope(const RopeParams& rp) {
  REQUIRE(rp.rotary_dim >= 0 && rp.rotary_dim <= 128 && rp.rotary_dim % 2 == 0);
  REQUIRE(rp.eps >= 0.0f && std::isfinite(rp.eps));
  for (int i = 0; i < rp.rotary_dim / 2; ++i) REQUIRE(std::isfinite(rp.inv_freq[i]) && rp.inv_freq[i] >= 0.0f);
}

hipError_t launch_pool(const uint16_t* raw, int64_t key_stride, const uint16_t* w, const RopeParams& rp,
                       int64_t first_block, int64_t n_blocks, uint16_t* pooled, hipStream_t, const int32_t* dev_tokens,
                       int64_t ceiling, int32_t* status) {
  REQUIRE(raw && w && pooled && key_stride >= 128 && n_blocks > 0 && first_block >= 0);
  if (dev_tokens) REQUIRE(status && ceiling >= 0 && ceiling <= QSA_MAX_TOKENS && n_blocks <= ceiling / 4);
  check_rope(rp);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_score(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows, const uint16_t* w,
                        const RopeParams& rp, const uint16_t*, int64_t tokens, float*, int64_t score_cols,
                        int32_t* status, hipStream_t) {
  REQUIRE(q && pos && w && status && q_stride >= 512 && rows > 0 && rows <= INT32_MAX);
  REQUIRE(tokens > 0 && tokens <= QSA_MAX_TOKENS && score_cols >= tokens / 4);
  check_rope(rp);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_prep(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows, const uint16_t* w,
                       const RopeParams& rp, int64_t tokens, uint16_t* qhat, int32_t* status, hipStream_t,
                       const int32_t*) {
  REQUIRE(q && pos && w && qhat && status && q_stride >= 512 && rows > 0 && rows <= INT32_MAX);
  REQUIRE(tokens >= 0 && tokens <= QSA_MAX_TOKENS);
  check_rope(rp);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_pool_prep(const uint16_t* raw, int64_t key_stride, const uint16_t* wk, int64_t first_block,
                            int64_t n_blocks, uint16_t* pooled, const uint16_t* q, int64_t q_stride,
                            const int32_t* pos, int64_t rows, const uint16_t* wq, uint16_t* qhat,
                            const RopeParams& rp, int64_t tokens, int32_t* status, hipStream_t,
                            const int32_t* dev_tokens) {
  REQUIRE(n_blocks >= 0 && rows >= 0 && rows <= INT32_MAX && (n_blocks > 0 || rows > 0));
  REQUIRE(tokens >= 0 && tokens <= QSA_MAX_TOKENS);
  if (n_blocks > 0) {
    REQUIRE(raw && wk && pooled && key_stride >= 128 && first_block >= 0);
    REQUIRE(dev_tokens ? n_blocks <= tokens / 4 : first_block + n_blocks <= tokens / 4);
  }
  if (rows > 0) REQUIRE(q && pos && wq && qhat && status && q_stride >= 512);
  if (dev_tokens) REQUIRE(status);
  check_rope(rp);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_score_prepped(const uint16_t* qhat, const int32_t* pos, int64_t rows, const uint16_t*,
                                int64_t tokens, float*, int64_t score_cols, int32_t* status, hipStream_t,
                                const int32_t*) {
  REQUIRE(qhat && pos && status && rows > 0 && rows <= INT32_MAX);
  REQUIRE(tokens > 0 && tokens <= QSA_MAX_TOKENS && score_cols >= tokens / 4);
  ++g_launches;
  return hipSuccess;
}

static void check_select(const int32_t* pos, int64_t rows, int64_t tokens, int keep_max, int64_t score_cols,
                         int32_t* status) {
  REQUIRE(pos && status && rows > 0 && rows <= INT32_MAX && tokens > 0 && tokens <= QSA_MAX_TOKENS);
  REQUIRE(keep_max >= 1 && keep_max <= QSA_MAX_KEEP_BLOCKS && score_cols >= tokens / 4);
}

hipError_t launch_select(const float*, int64_t score_cols, const int32_t* pos, int64_t rows, int64_t tokens,
                         int keep_max, uint8_t* mask, int32_t* status, hipStream_t) {
  check_select(pos, rows, tokens, keep_max, score_cols, status);
  REQUIRE(mask);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_select_indices(const float*, int64_t score_cols, const int32_t* pos, int64_t rows, int64_t tokens,
                                 int keep_max, int32_t* idx, int64_t idx_stride, int32_t* counts, int32_t* status,
                                 hipStream_t, const int32_t*) {
  check_select(pos, rows, tokens, keep_max, score_cols, status);
  REQUIRE(idx && counts && idx_stride >= 4 * keep_max + 3);
  ++g_launches;
  return hipSuccess;
}

bool select_split_pays(int64_t rows, int64_t tokens) { return tokens / 4 > 16384 && rows <= 128; }
int64_t select_split_workspace_bytes(int64_t rows, int64_t tokens) {
  REQUIRE(rows >= 0 && rows <= 128 && tokens >= 0 && tokens <= QSA_MAX_TOKENS);
  return rows * ((tokens + 16383) / 16384) * (512 * 8 + 256);
}

hipError_t launch_select_split(const float*, int64_t score_cols, const int32_t* pos, int64_t rows, int64_t tokens,
                               int keep_max, uint8_t* mask, int32_t* status, void* workspace, hipStream_t) {
  check_select(pos, rows, tokens, keep_max, score_cols, status);
  REQUIRE(mask && workspace && reinterpret_cast<uintptr_t>(workspace) % 16 == 0);
  ++g_launches;
  return hipSuccess;
}

hipError_t noalloc_scratch(void** out) {
  static unsigned char fake_scratch[256] __attribute__((aligned(256)));
  *out = fake_scratch;  // the stubs never touch it
  return hipSuccess;
}

hipError_t launch_select_split_indices(const float*, int64_t score_cols, const int32_t* pos, int64_t rows,
                                       int64_t tokens, int keep_max, int32_t* idx, int64_t idx_stride,
                                       int32_t* counts, int32_t* status, void* workspace, hipStream_t,
                                       const int32_t*) {
  check_select(pos, rows, tokens, keep_max, score_cols, status);
  REQUIRE(idx && counts && workspace && idx_stride >= 4 * keep_max + 3);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_select_flagged(const float*, int64_t, const int32_t*, int64_t, int64_t, int, uint8_t*, int32_t*,
                                 const int32_t*, hipStream_t) {
  REQUIRE(false);  // reached only from inside the fused launcher
  return hipSuccess;
}

int64_t ring_splits(int64_t, int64_t, int64_t) { return 1; }
hipError_t launch_ring(const RingJob&, int64_t, hipStream_t) {
  REQUIRE(false);  // reached only from inside the fused launcher
  return hipSuccess;
}

hipError_t launch_gather_kv(const uint16_t* k, const uint16_t* v, int64_t n_pages, int page_size, int kv_dim,
                            const int32_t* table, int64_t table_stride, int64_t table_len, const int32_t* idx,
                            int64_t idx_stride, const int32_t* counts, int64_t rows, int64_t slots, uint16_t* ko,
                            uint16_t* vo, int32_t* otable, int32_t* status, hipStream_t) {
  REQUIRE(page_size >= 1 && kv_dim >= 1 && rows > 0 && slots > 0 && slots % page_size == 0);
  REQUIRE(ko && vo && otable && counts && status && n_pages >= 0 && table_len >= 0);
  REQUIRE(table_stride == 0 || table_stride >= table_len);
  if (n_pages > 0) REQUIRE(k && v);
  if (table_len > 0) REQUIRE(table);
  if (idx_stride > 0) REQUIRE(idx);
  ++g_launches;
  return hipSuccess;
}

int64_t score_select_workspace_bytes(int64_t rows, int64_t tokens, int keep_max) {
  REQUIRE(rows > 0 && rows <= INT32_MAX && tokens > 0 && tokens <= QSA_MAX_TOKENS && keep_max >= 1 &&
          keep_max <= 512);
  return 4096 + rows * (tokens / 4 + 64) * 4;
}
int64_t score_select_flags_offset(int64_t rows, int64_t tokens, int keep_max) {
  REQUIRE(score_select_workspace_bytes(rows, tokens, keep_max) > 4 * rows);
  return 256;
}

hipError_t launch_score_select(const uint16_t* qhat, const int32_t* pos, int64_t rows, const uint16_t*,
                               int64_t tokens, int keep_max, uint8_t* mask, int32_t* status, void* workspace,
                               hipStream_t) {
  REQUIRE(qhat && pos && mask && status && workspace && rows > 0 && rows <= INT32_MAX);
  REQUIRE(tokens > 0 && tokens <= QSA_MAX_TOKENS && keep_max >= 1 && keep_max <= 512);
  REQUIRE(reinterpret_cast<uintptr_t>(workspace) % 256 == 0);
  ++g_launches;
  return hipSuccess;
}

}  // namespace qsa

// ---- the sweep ----------------------------------------------------------

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static const int64_t kInts[] = {-1, 0, 1, 2, 3, 4, 5, 7, 16, 64, 127, 128, 129, 511, 512, 513, 640, 2047, 2048,
                                2051, 2052, 4096, 16384, 65536, 65540, 262144, 262147, 262148, 1 << 20,
                                INT32_MAX, (int64_t)INT32_MAX + 1, INT64_MAX / 4, INT64_MAX - 1, INT64_MAX,
                                INT64_MIN, -4096};
// an extreme value, or (half the time) the argument's valid value `good`
static int64_t any_int(int64_t good) {
  if (next_u64() % 2) return good;
  return kInts[next_u64() % (sizeof(kInts) / sizeof(kInts[0]))];
}
static int32_t any_i32(int32_t good) {
  const int64_t v = any_int(good);
  return v > INT32_MAX ? INT32_MAX : (v < INT32_MIN ? INT32_MIN : static_cast<int32_t>(v));
}
static float any_float(float good) {
  switch (next_u64() % 6) {
    case 0: return 0.0f;
    case 1: return -1.0f;
    case 2: return NAN;
    case 3: return INFINITY;
    default: return good;
  }
}
// fake device addresses: never dereferenced by the stubs
static void* any_ptr() {
  switch (next_u64() % 12) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<void*>(0x1008);  // 8-byte aligned only
    default: return reinterpret_cast<void*>(0x100000);
  }
}

static bool documented(int64_t rc) { return rc == QSA_OK || (rc <= -1 && rc >= -7); }

template <typename T>
static T* P() { return static_cast<T*>(any_ptr()); }

int main() {
  // host-side rotary table: exact-size heap buffers (ASan sees an overrun)
  for (int rd = 0; rd <= 130; ++rd) {
    std::vector<float> buf(static_cast<size_t>(rd / 2 > 0 ? rd / 2 : 1));
    const int rc = qsa_rope_inv_freq(rd, 1e4f, buf.data());
    REQUIRE(rc == ((rd % 2 == 0 && rd <= 128) ? QSA_OK : QSA_ERR_PARAM));
  }
  REQUIRE(qsa_rope_inv_freq(64, NAN, nullptr) == QSA_ERR_PARAM);
  for (int c = -8; c <= 1; ++c) REQUIRE(qsa_strerror(c) != nullptr);
  REQUIRE(qsa_abi_version() == QSA_ABI_VERSION);

  // exact refusals and launches
  void* F = reinterpret_cast<void*>(0x100000);
  const uint16_t* u = static_cast<const uint16_t*>(F);
  const long l0 = g_launches;
  REQUIRE(qsa_pool_keys(u, 128, 64, u, 64, 1e4f, 1e-6f, 0, 16, (uint16_t*)F, nullptr) == QSA_OK);
  REQUIRE(g_launches == l0 + 1);
  // the combined pool + prep: either stage alone, neither, and each stage's refusals
  {
    int32_t* i32 = static_cast<int32_t*>(F);
    uint16_t* w16 = static_cast<uint16_t*>(F);
    const long l1 = g_launches;
    REQUIRE(qsa_pool_prep(u, 128, 64, u, 0, 16, w16, u, 512, i32, 4, u, w16, 64, 1e4f, 1e-6f, i32, nullptr) == QSA_OK);
    REQUIRE(qsa_pool_prep(nullptr, 128, 64, nullptr, 0, 0, nullptr, u, 512, i32, 4, u, w16, 64, 1e4f, 1e-6f, i32,
                          nullptr) == QSA_OK);
    REQUIRE(qsa_pool_prep(u, 128, 64, u, 0, 16, w16, nullptr, 512, nullptr, 0, nullptr, nullptr, 64, 1e4f, 1e-6f,
                          nullptr, nullptr) == QSA_OK);
    REQUIRE(qsa_pool_prep(u, 128, 64, u, 0, 0, w16, u, 512, i32, 0, u, w16, 64, 1e4f, 1e-6f, i32, nullptr) == QSA_OK);
    REQUIRE(g_launches == l1 + 3);
    REQUIRE(qsa_pool_prep(u, 128, 64, u, 0, 16, w16, u, 511, i32, 4, u, w16, 64, 1e4f, 1e-6f, i32, nullptr) ==
            QSA_ERR_STRIDE);
    REQUIRE(qsa_pool_prep(u, 128, 64, u, 1, 16, w16, u, 512, i32, 4, u, w16, 64, 1e4f, 1e-6f, i32, nullptr) ==
            QSA_ERR_EXTENT);
    REQUIRE(qsa_pool_prep(u, 128, 64, u, 0, 16, w16, u, 512, i32, 4, u, w16, 64, 1e4f, 1e-6f, nullptr, nullptr) ==
            QSA_ERR_NULL);
    REQUIRE(qsa_pool_prep_dev(u, 128, 64, u, 1, w16, u, 512, i32, 4, u, w16, 64, 1e4f, 1e-6f, nullptr, i32,
                              nullptr) == QSA_ERR_NULL);
    REQUIRE(qsa_pool_prep_dev(u, 128, 64, u, 17, w16, u, 512, i32, 4, u, w16, 64, 1e4f, 1e-6f, i32, i32,
                              nullptr) == QSA_ERR_EXTENT);
    REQUIRE(g_launches == l1 + 3);
  }
  // the no-allocation select: its scratch limit, then an accepted split call
  REQUIRE(qsa_select_mask_noalloc((float*)F, 65536, 128 * 65536, (int32_t*)F, 128, 262144, 2048, (uint8_t*)F,
                                  (int32_t*)F, nullptr) == QSA_ERR_CAPACITY);
  REQUIRE(qsa_select_mask_noalloc((float*)F, 65536, 16 * 65536, (int32_t*)F, 16, 262144, 2048, (uint8_t*)F,
                                  (int32_t*)F, nullptr) == QSA_OK);
  REQUIRE(g_launches == l0 + 5);
  REQUIRE(qsa_pool_keys(u, 128, INT64_MAX, u, 64, 1e4f, 1e-6f, 0, 16, (uint16_t*)F, nullptr) == QSA_ERR_CAPACITY);
  REQUIRE(qsa_select_mask((float*)F, INT64_MAX, INT64_MAX, (int32_t*)F, INT64_MAX, 64, 64, (uint8_t*)F,
                          (int32_t*)F, nullptr) == QSA_ERR_CAPACITY);
  REQUIRE(qsa_select_indices((float*)F, 16, 1 << 20, (int32_t*)F, 8, 64, INT64_MAX, (int32_t*)F, 100,
                             (int32_t*)F, (int32_t*)F, nullptr) == QSA_ERR_BUDGET);
  REQUIRE(qsa_select_workspace_bytes(INT64_MAX, 262144) == 0);
  REQUIRE(qsa_score_select_workspace_bytes(INT64_MAX, 64, 4) == QSA_ERR_CAPACITY);
  REQUIRE(g_launches == l0 + 5);

  // the sweep: every entry point, random combinations of extreme extents,
  // bad and good parameters and NULL / fake pointers
  const int kIters = 200000;
  long counted = 0;
  for (int it = 0; it < kIters; ++it) {
    int64_t rc = 0;
    switch (it % 20) {
      case 0:
        rc = qsa_pool_keys(P<uint16_t>(), any_int(128), any_int(4096), P<uint16_t>(), any_i32(64), any_float(1e4f),
                           any_float(1e-6f), any_int(0), any_int(1024), P<uint16_t>(), nullptr);
        break;
      case 1:
        rc = qsa_score_rows(P<uint16_t>(), any_int(512), P<int32_t>(), any_int(64), P<uint16_t>(), any_i32(64),
                            any_float(1e4f), any_float(1e-6f), P<uint16_t>(), any_int(65536), P<float>(),
                            any_int(16384), any_int(64 * 16384), P<int32_t>(), nullptr);
        break;
      case 2:
        rc = qsa_prep_queries(P<uint16_t>(), any_int(512), P<int32_t>(), any_int(64), P<uint16_t>(), any_i32(64),
                              any_float(1e4f), any_float(1e-6f), any_int(65536), P<uint16_t>(), P<int32_t>(),
                              nullptr);
        break;
      case 3:
        rc = qsa_score_prepped(P<uint16_t>(), P<int32_t>(), any_int(8192), P<uint16_t>(), any_int(65536), P<float>(),
                               any_int(16384), any_int(8192 * 16384), P<int32_t>(), nullptr);
        break;
      case 4:
        rc = qsa_select_mask(P<float>(), any_int(16384), any_int(64 * 16384), P<int32_t>(), any_int(64),
                             any_int(65536), any_int(2048), P<uint8_t>(), P<int32_t>(), nullptr);
        break;
      case 5:
        rc = qsa_select_indices(P<float>(), any_int(16384), any_int(64 * 16384), P<int32_t>(), any_int(64),
                                any_int(65536), any_int(2048), P<int32_t>(), any_int(2051), P<int32_t>(),
                                P<int32_t>(), nullptr);
        break;
      case 6:
        rc = qsa_select_workspace_bytes(any_int(16), any_int(262144));
        break;
      case 7:
        rc = qsa_select_mask_ws(P<float>(), any_int(65536), any_int(16 * 65536), P<int32_t>(), any_int(16),
                                any_int(262144), any_int(2048), P<uint8_t>(), P<int32_t>(), any_ptr(),
                                any_int(16 * 16 * 4352), nullptr);
        break;
      case 8:
        rc = qsa_score_select_workspace_bytes(any_int(8192), any_int(65536), any_int(2048));
        break;
      case 9:
        rc = qsa_score_select_mask(P<uint16_t>(), P<int32_t>(), any_int(1024), P<uint16_t>(), any_int(65536),
                                   any_int(2048), P<uint8_t>(), P<int32_t>(), any_ptr(), any_int(INT64_MAX / 4),
                                   nullptr);
        break;
      case 10:
        rc = qsa_gather_kv(P<uint16_t>(), P<uint16_t>(), any_int(4096), any_i32(16), any_i32(512), P<int32_t>(),
                           any_int(0), any_int(4096), P<int32_t>(), any_int(2051), P<int32_t>(), any_int(16),
                           any_int(2064), P<uint16_t>(), P<uint16_t>(), P<int32_t>(), P<int32_t>(), nullptr);
        break;
      case 11:
        rc = qsa_pool_window(P<uint16_t>(), any_int(128), any_int(65792), P<uint16_t>(), any_i32(64),
                             any_float(1e4f), any_float(1e-6f), P<int32_t>(), any_int(4), P<uint16_t>(),
                             P<int32_t>(), nullptr);
        break;
      case 12:
        rc = qsa_prep_queries_dev(P<uint16_t>(), any_int(512), P<int32_t>(), any_int(4), P<uint16_t>(),
                                  any_i32(64), any_float(1e4f), any_float(1e-6f), P<int32_t>(), any_int(65792),
                                  P<uint16_t>(), P<int32_t>(), nullptr);
        break;
      case 13:
        rc = qsa_score_prepped_dev(P<uint16_t>(), P<int32_t>(), any_int(4), P<uint16_t>(), P<int32_t>(),
                                   any_int(65792), P<float>(), any_int(16448), any_int(4 * 16448), P<int32_t>(),
                                   nullptr);
        break;
      case 14:
        rc = qsa_select_indices_dev(P<float>(), any_int(16448), any_int(4 * 16448), P<int32_t>(), any_int(4),
                                    P<int32_t>(), any_int(65792), any_int(2048), P<int32_t>(), any_int(2051),
                                    P<int32_t>(), P<int32_t>(), any_ptr(), any_int(1 << 20), nullptr);
        break;
      case 15:
        rc = qsa_select_indices_ws(P<float>(), any_int(65536), any_int(16 * 65536), P<int32_t>(), any_int(16),
                                   any_int(262144), any_int(2048), P<int32_t>(), any_int(2051), P<int32_t>(),
                                   P<int32_t>(), any_ptr(), any_int(1 << 20), nullptr);
        break;
      case 16:
        rc = qsa_score_select_flags_offset(any_int(8192), any_int(65536), any_int(2048));
        break;
      case 17:
        rc = qsa_select_mask_noalloc(P<float>(), any_int(65536), any_int(16 * 65536), P<int32_t>(), any_int(16),
                                     any_int(262144), any_int(2048), P<uint8_t>(), P<int32_t>(), nullptr);
        break;
      case 18:
        rc = qsa_pool_prep(P<uint16_t>(), any_int(128), any_int(65536), P<uint16_t>(), any_int(0), any_int(16384),
                           P<uint16_t>(), P<uint16_t>(), any_int(512), P<int32_t>(), any_int(64), P<uint16_t>(),
                           P<uint16_t>(), any_i32(64), any_float(1e4f), any_float(1e-6f), P<int32_t>(), nullptr);
        break;
      case 19:
        rc = qsa_pool_prep_dev(P<uint16_t>(), any_int(128), any_int(65792), P<uint16_t>(), any_int(4), P<uint16_t>(),
                               P<uint16_t>(), any_int(512), P<int32_t>(), any_int(4), P<uint16_t>(), P<uint16_t>(),
                               any_i32(64), any_float(1e4f), any_float(1e-6f), P<int32_t>(), P<int32_t>(), nullptr);
        break;
    }
    const int k = it % 20;
    const bool size_query = k == 6 || k == 8 || k == 16;
    REQUIRE(size_query ? rc >= -7 : documented(rc));
    ++counted;
  }
  std::printf("abi sanitizer sweep: %ld calls, %ld launches reached the stubs, %d failures\n", counted, g_launches,
              g_fail);
  return g_fail == 0 ? 0 : 1;
}
