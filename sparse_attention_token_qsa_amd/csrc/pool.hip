// Block pooling launch: one workgroup per 16 consecutive blocks (pool_body.h).
#include "pool_body.h"

namespace qsa {
namespace {

template <bool kVec, int kHalf>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const PoolArgs a) {
  pool_group<kVec, kHalf>(a, blockIdx.x);
}

}  // namespace

hipError_t launch_pool(const uint16_t* raw, int64_t key_stride, const uint16_t* w,
                       const RopeParams& rp, int64_t first_block, int64_t n_blocks,
                       uint16_t* pooled, hipStream_t stream, const int32_t* dev_tokens,
                       int64_t ceiling, int32_t* status) {
  PoolArgs a{raw, key_stride, w, pooled, first_block, n_blocks, rp, dev_tokens, ceiling, status};
  const int64_t groups = (n_blocks + kPoolBlocksPerGroup - 1) / kPoolBlocksPerGroup;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool vec = (key_stride % 8 == 0) && (reinterpret_cast<uintptr_t>(raw) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(pooled) % 16 == 0);
  const dim3 grid(static_cast<unsigned>(groups)), block(kPoolThreads);
  if (rp.rotary_dim == 64) {  // the pages' geometry, its pair count fixed at compile time
    if (vec)
      pool_kernel<true, 32><<<grid, block, 0, stream>>>(a);
    else
      pool_kernel<false, 32><<<grid, block, 0, stream>>>(a);
  } else if (vec) {
    pool_kernel<true, 0><<<grid, block, 0, stream>>>(a);
  } else {
    pool_kernel<false, 0><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace qsa
