// Query prep launch: one workgroup per 4 rows (prep_body.h).
#include "prep_body.h"

namespace qsa {
namespace {

template <int kHalf>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const PrepArgs a) {
  prep_group<kHalf>(a, blockIdx.x);
}

}  // namespace

hipError_t launch_prep(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                       const uint16_t* w, const RopeParams& rp, int64_t tokens, uint16_t* qhat,
                       int32_t* status, hipStream_t stream, const int32_t* dev_tokens) {
  PrepArgs a{};
  a.dev_tokens = dev_tokens;
  a.q = q;
  a.q_stride = q_stride;
  a.pos = pos;
  a.rows = rows;
  a.w = w;
  a.tokens = tokens;
  a.qhat = qhat;
  a.status = status;
  a.q_vec = (q_stride % 8 == 0) && (reinterpret_cast<uintptr_t>(q) % 16 == 0);
  a.rp = rp;
  const int64_t grid = (rows + kPrepRows - 1) / kPrepRows;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>(grid)), b(kPrepThreads);
  if (rp.rotary_dim == 64)  // the pages' geometry, its pair count fixed at compile time
    prep_kernel<32><<<g, b, 0, stream>>>(a);
  else
    prep_kernel<0><<<g, b, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
