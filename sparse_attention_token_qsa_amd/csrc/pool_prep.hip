// A decode step's two norm + rope stages in one launch.
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: the scorer reads the pooled keys and the normed, roped
// query heads, and neither of those stages reads the other's output.  One
// grid therefore runs both: workgroups [0, prep groups) prepare four query
// rows each (prep_body.h), the rest pool sixteen key blocks each
// (pool_body.h), with the same arithmetic and outputs as the two separate
// launches.  The prep workgroups come first, so they are dispatched with the
// pool's first workgroups and their chain of dependent loads overlaps the
// pool's streaming instead of adding a launch and its drain to the step.
#include "pool_body.h"
#include "prep_body.h"

namespace qsa {
namespace {

static_assert(kPoolThreads == kPrepThreads, "one workgroup size for both stages");

template <bool kVec, int kHalf>
__global__ __launch_bounds__(kPoolThreads) void pool_prep_kernel(const PoolArgs pa, const PrepArgs qa,
                                                                 const int64_t prep_groups) {
  if (static_cast<int64_t>(blockIdx.x) < prep_groups)  // uniform across the workgroup
    prep_group<kHalf>(qa, blockIdx.x);
  else
    pool_group<kVec, kHalf>(pa, static_cast<int64_t>(blockIdx.x) - prep_groups);
}

}  // namespace

hipError_t launch_pool_prep(const uint16_t* raw, int64_t key_stride, const uint16_t* wk,
                            int64_t first_block, int64_t n_blocks, uint16_t* pooled,
                            const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                            const uint16_t* wq, uint16_t* qhat, const RopeParams& rp, int64_t tokens,
                            int32_t* status, hipStream_t stream, const int32_t* dev_tokens) {
  PoolArgs pa{raw, key_stride, wk, pooled, first_block, n_blocks, rp, dev_tokens, tokens, status};
  PrepArgs qa{};
  qa.q = q;
  qa.q_stride = q_stride;
  qa.pos = pos;
  qa.rows = rows;
  qa.w = wq;
  qa.tokens = tokens;
  qa.dev_tokens = dev_tokens;
  qa.qhat = qhat;
  qa.status = status;
  qa.q_vec = (q_stride % 8 == 0) && (reinterpret_cast<uintptr_t>(q) % 16 == 0);
  qa.rp = rp;
  const int64_t prep_groups = (rows + kPrepRows - 1) / kPrepRows;
  const int64_t pool_groups = (n_blocks + kPoolBlocksPerGroup - 1) / kPoolBlocksPerGroup;
  const int64_t grid = prep_groups + pool_groups;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  const bool vec = (key_stride % 8 == 0) && (reinterpret_cast<uintptr_t>(raw) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(pooled) % 16 == 0);
  const dim3 g(static_cast<unsigned>(grid)), block(kPoolThreads);
  if (rp.rotary_dim == 64) {  // the pages' geometry, its pair count fixed at compile time
    if (vec)
      pool_prep_kernel<true, 32><<<g, block, 0, stream>>>(pa, qa, prep_groups);
    else
      pool_prep_kernel<false, 32><<<g, block, 0, stream>>>(pa, qa, prep_groups);
  } else if (vec) {
    pool_prep_kernel<true, 0><<<g, block, 0, stream>>>(pa, qa, prep_groups);
  } else {
    pool_prep_kernel<false, 0><<<g, block, 0, stream>>>(pa, qa, prep_groups);
  }
  return hipGetLastError();
}

}  // namespace qsa
