// Block pooling: every complete 4-token block's raw keys -> one pooled key.
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: the block's raw keys are averaged in float32 and cast back
// to bf16, then (1 + w) RMSNorm and partial RoPE at the block's first token.
//
// Layout: a workgroup of 256 threads pools 16 consecutive blocks; each block
// is owned by 16 lanes holding 8 channels each, so one block's four 256-byte
// token rows are read as four 16-byte loads per lane and the pooled 256-byte
// row leaves as one 16-byte store per lane.  The loads are issued first; the
// cos/sin of the 16 anchors (one (block, frequency) pair per thread and
// pass) overlap them.  The RMSNorm statistic is a 16-lane DPP reduction in
// double; the RoPE partner is read back from the normed row in LDS, so any
// even rotary_dim works.  Roundings to bf16 use the hardware's
// round-to-nearest-even conversion; a NaN result is written as 0x7FC0.  The
// stage is HBM-bound: 1 KiB read and 256 B written per block.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolBlocksPerGroup = kPoolThreads / 16;

struct PoolArgs {
  const uint16_t* raw;
  int64_t key_stride;
  const uint16_t* w;
  uint16_t* pooled;
  int64_t first_block;
  int64_t n_blocks;
  RopeParams rp;
  // window mode (dev_tokens set): the last n_blocks complete blocks of a
  // cache of *dev_tokens tokens (at most `ceiling`), first_block unused
  const int32_t* dev_tokens;
  int64_t ceiling;
  int32_t* status;
};

__device__ __forceinline__ void unpack8(const uint4 u, float (&v)[8]) {
  const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(wd[i] << 16);
    v[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

template <bool kVec>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const PoolArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t csq[kPoolBlocksPerGroup][kMaxHalfRotary];
  __shared__ __attribute__((aligned(16))) uint4 ys[kPoolBlocksPerGroup][16];

  const int tid = threadIdx.x;
  const int slot = tid >> 4;  // block slot within the group
  const int g = tid & 15;     // channel group: channels 8g .. 8g+7
  const int64_t group_first = static_cast<int64_t>(blockIdx.x) * kPoolBlocksPerGroup;
  const int64_t blk = group_first + slot;
  int64_t first = a.first_block, count = a.n_blocks;
  if (a.dev_tokens != nullptr) {
    const int64_t complete = live_tokens(a.ceiling, a.dev_tokens, a.status) / kRatio;
    first = complete > a.n_blocks ? complete - a.n_blocks : 0;
    count = complete - first;
  }
  const bool live = blk < count;
  const int64_t b = first + blk;

  // raw keys first: four 16-byte token rows per lane
  uint4 v[4];
  if (live) {
    const uint16_t* base = a.raw + kRatio * b * a.key_stride + 8 * g;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint16_t* src = base + t * a.key_stride;
      if constexpr (kVec) {
        v[t] = *reinterpret_cast<const uint4*>(src);
      } else {
        v[t].x = src[0] | (static_cast<uint32_t>(src[1]) << 16);
        v[t].y = src[2] | (static_cast<uint32_t>(src[3]) << 16);
        v[t].z = src[4] | (static_cast<uint32_t>(src[5]) << 16);
        v[t].w = src[6] | (static_cast<uint32_t>(src[7]) << 16);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = make_uint4(0u, 0u, 0u, 0u);
  }
  double wp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wp[e] = 1.0 + static_cast<double>(bf16_to_f32(a.w[8 * g + e]));

  // cos/sin at every slot's anchor 4b: thread (slot, j) takes frequencies
  // j, j + 16, ... below rotary_dim / 2.
  const int rd = a.rp.rotary_dim;
  const int half = rd >> 1;
  const int64_t anchor = kRatio * b;
  for (int i = g; i < half; i += 16) {
    csq[slot][i] = rope_cos_sin_bf16x2(anchor, a.rp.inv_freq[i]);
  }

  // f32 mean of the 4 tokens in token order, cast to bf16.
  float k0[8], k1[8], k2[8], k3[8], m[8];
  unpack8(v[0], k0);
  unpack8(v[1], k1);
  unpack8(v[2], k2);
  unpack8(v[3], k3);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
    float s = k0[e] + k1[e];
    s = s + k2[e];
    s = s + k3[e];
    m[e] = rb_hw(s * 0.25f);
  }

  // (1 + w) RMSNorm in double, rounded to f32 and then to bf16.
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += static_cast<double>(m[e]) * static_cast<double>(m[e]);
  const double r = inv_rms(row16_sum(ss), a.rp.eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
    y[e] = rb_hw(static_cast<float>((static_cast<double>(m[e]) * r) * wp[e]));
  }
  ys[slot][g] = make_uint4(pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]),
                           pack2(y[6], y[7]));
  __syncthreads();

  // Partial RoPE at the block's first token.
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = y[e];
  const int c0 = 8 * g;
  if ((half & 7) == 0) {  // chunks of 8 channels never straddle the halves
    if (c0 < rd) {
      const bool first = c0 < half;
      float yp[8];
      unpack8(ys[slot][first ? g + (half >> 3) : g - (half >> 3)], yp);
      const int f0 = first ? c0 : c0 - half;
      const uint4 cs0 = *reinterpret_cast<const uint4*>(&csq[slot][f0]);
      const uint4 cs1 = *reinterpret_cast<const uint4*>(&csq[slot][f0 + 4]);
      const uint32_t cs[8] = {cs0.x, cs0.y, cs0.z, cs0.w, cs1.x, cs1.y, cs1.z, cs1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
        const float p0 = rb_hw(y[e] * __uint_as_float(cs[e] << 16));
        const float p1 = rb_hw(yp[e] * __uint_as_float(cs[e] & 0xFFFF0000u));
        o[e] = first ? p0 - p1 : p0 + p1;
      }
    }
  } else {
    const uint16_t* yrow = reinterpret_cast<const uint16_t*>(&ys[slot][0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
      const int c = c0 + e;
      if (c < rd) {
        const bool first = c < half;
        const float yp = bf16_to_f32(yrow[first ? c + half : c - half]);
        const uint32_t cs = csq[slot][first ? c : c - half];
        const float p0 = rb_hw(y[e] * __uint_as_float(cs << 16));
        const float p1 = rb_hw(yp * __uint_as_float(cs & 0xFFFF0000u));
        o[e] = first ? p0 - p1 : p0 + p1;
      }
    }
  }
  if (live) {
    uint4 out = make_uint4(pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]),
                           pack2(o[6], o[7]));
    bool nan = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) nan |= o[e] != o[e];
    if (nan) {  // rare: only a non-finite key, weight or norm gets here
      out = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7]));
    }
    uint16_t* dst = a.pooled + b * kHeadDim + c0;
    if constexpr (kVec) {
      *reinterpret_cast<uint4*>(dst) = out;
    } else {
      const uint32_t wd[4] = {out.x, out.y, out.z, out.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[2 * i] = static_cast<uint16_t>(wd[i] & 0xFFFFu);
        dst[2 * i + 1] = static_cast<uint16_t>(wd[i] >> 16);
      }
    }
  }
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
  if (vec)
    pool_kernel<true><<<dim3(static_cast<unsigned>(groups)), dim3(kPoolThreads), 0, stream>>>(a);
  else
    pool_kernel<false><<<dim3(static_cast<unsigned>(groups)), dim3(kPoolThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
