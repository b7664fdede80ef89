// Query prep launch: one workgroup per 4 rows (prep_body.h).
#include "prep_body.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const PrepArgs a) { prep_group(a, blockIdx.x); }

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
  prep_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(kPrepThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
