// Block pooling: every complete 4-token block's raw keys -> one pooled key.
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: the block's raw keys are averaged in float32 and cast back
// to bf16, then (1 + w) RMSNorm and partial RoPE at the block's first token.
//
// Layout: a workgroup of 256 threads pools 16 consecutive blocks; each block
// is owned by 16 lanes holding 8 channels each, so one block's four 256-byte
// token rows are read as four 16-byte loads per lane and the pooled 256-byte
// row leaves as one 16-byte store per lane.  The RMSNorm statistic is a
// 16-lane butterfly in double; the RoPE partner channel is exchanged through
// LDS so any even rotary_dim works.  The stage is HBM-bound: 1 KiB read and
// 256 B written per block.
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
};

__device__ __forceinline__ void unpack8(const uint4 v, float out[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

template <bool kVec>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const PoolArgs a) {
  __shared__ float ybuf[kPoolBlocksPerGroup][kHeadDim];
  __shared__ float2 csbuf[kPoolBlocksPerGroup][kMaxHalfRotary];

  const int tid = threadIdx.x;
  const int slot = tid >> 4;  // block slot within the group
  const int g = tid & 15;     // channel group: channels 8g .. 8g+7
  const int64_t group_first = static_cast<int64_t>(blockIdx.x) * kPoolBlocksPerGroup;
  const int64_t blk = group_first + slot;
  const bool live = blk < a.n_blocks;
  const int64_t b = a.first_block + blk;
  const int rd = a.rp.rotary_dim;
  const int half = rd >> 1;

  // cos/sin at every slot's anchor 4b for every rotary frequency.
  for (int idx = tid; idx < kPoolBlocksPerGroup * half; idx += kPoolThreads) {
    const int sl = idx / half;
    const int i = idx - sl * half;
    float c, s;
    rope_cos_sin(kRatio * (a.first_block + group_first + sl), a.rp.inv_freq[i], c, s);
    csbuf[sl][i] = make_float2(c, s);
  }

  // f32 mean of the 4 tokens in token order, cast to bf16.
  float m[8];
  if (live) {
    const uint16_t* base = a.raw + kRatio * b * a.key_stride + 8 * g;
    float k[4][8];
    if constexpr (kVec) {
      uint4 v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = *reinterpret_cast<const uint4*>(base + t * a.key_stride);
#pragma unroll
      for (int t = 0; t < 4; ++t) unpack8(v[t], k[t]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) k[t][e] = bf16_to_f32(base[t * a.key_stride + e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = k[0][e] + k[1][e];
      s = s + k[2][e];
      s = s + k[3][e];
      m[e] = round_bf16(s * 0.25f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = 0.0f;
  }

  // (1 + w) RMSNorm: sum of squares over the block's 16 lanes, in double.
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += static_cast<double>(m[e]) * static_cast<double>(m[e]);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const double r = inv_rms(ss, a.rp.eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y[e] = norm_channel(m[e], r, bf16_to_f32(a.w[8 * g + e]));
    ybuf[slot][8 * g + e] = y[e];
  }
  __syncthreads();

  // Partial RoPE at the block's first token.
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * g + e;
    if (c < rd) {
      const bool first = c < half;
      const int i = first ? c : c - half;
      const float xp = ybuf[slot][first ? c + half : c - half];
      const float2 cs = csbuf[slot][i];
      o[e] = rope_channel(y[e], xp, cs.x, cs.y, first);
    } else {
      o[e] = y[e];
    }
  }
  if (live) {
    uint16_t* dst = a.pooled + b * kHeadDim + 8 * g;
    if constexpr (kVec) {
      uint4 v;
      v.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
      v.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
      v.z = f32_to_bf16(o[4]) | (f32_to_bf16(o[5]) << 16);
      v.w = f32_to_bf16(o[6]) | (f32_to_bf16(o[7]) << 16);
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = static_cast<uint16_t>(f32_to_bf16(o[e]));
    }
  }
}

}  // namespace

hipError_t launch_pool(const uint16_t* raw, int64_t key_stride, const uint16_t* w,
                       const RopeParams& rp, int64_t first_block, int64_t n_blocks,
                       uint16_t* pooled, hipStream_t stream) {
  PoolArgs a{raw, key_stride, w, pooled, first_block, n_blocks, rp};
  const int64_t groups = (n_blocks + kPoolBlocksPerGroup - 1) / kPoolBlocksPerGroup;
  const bool vec = (key_stride % 8 == 0) && (reinterpret_cast<uintptr_t>(raw) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(pooled) % 16 == 0);
  if (vec)
    pool_kernel<true><<<dim3(static_cast<unsigned>(groups)), dim3(kPoolThreads), 0, stream>>>(a);
  else
    pool_kernel<false><<<dim3(static_cast<unsigned>(groups)), dim3(kPoolThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
