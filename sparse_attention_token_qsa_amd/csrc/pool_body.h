// Block pooling: every complete 4-token block's raw keys -> one pooled key.
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: the block's raw keys are averaged in float32 and cast back
// to bf16, then (1 + w) RMSNorm and partial RoPE at the block's first token.
//
// Layout: a workgroup of 256 threads pools 16 consecutive blocks; each block
// is owned by 16 lanes (of one wave) holding 8 channels each, so one block's
// four 256-byte token rows are read as four 16-byte loads per lane and the
// pooled 256-byte row leaves as one 16-byte store per lane.  The loads are
// issued first; each lane's cos/sin (for the rotary pairs it rotates: 2g and
// 2g + 1 at rotary_dim 64, else g, g + 16, ... below rotary_dim / 2) overlap
// them.  The RMSNorm statistic is a 16-lane DPP reduction in double.  The
// RoPE goes pair by pair through the block's row in LDS, so every lane
// rotates and any even rotary_dim works; a block's lanes share a wave, so
// wave-level ordering of the LDS traffic suffices.  Roundings to bf16 use the
// hardware's round-to-nearest-even conversion; a NaN result is written as
// 0x7FC0.  The stage moves 1 KiB read and 256 B written per block; on long
// caches its instruction issue, more than HBM, sets its time.
#pragma once

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

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

__device__ __forceinline__ uint32_t pool_pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 NaN test of both halves of a packed word: a half is NaN exactly when
// its magnitude bits exceed 0x7F80, i.e. reach 0x8000 after adding 0x7F
// (no carry crosses into the other half).
__device__ __forceinline__ uint32_t pool_nan_halves(uint32_t d) {
  return ((d & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
}

// The pooled keys of workgroup-sized group `group` (16 consecutive blocks).
// kHalf: rotary_dim / 2 when fixed at compile time (the launch picks 32 for
// rotary_dim 64), else 0 and taken from the arguments.
template <bool kVec, int kHalf = 0>
__device__ __forceinline__ void pool_group(const PoolArgs& a, int64_t group) {
  // one 128-channel bf16 row per block slot: the normed key, then (in place)
  // the rotated channels
  __shared__ __attribute__((aligned(16))) uint16_t ys[kPoolBlocksPerGroup][kHeadDim];
  // (1 + w) in double for the 128 channels.  Every wave converts all of them,
  // two per lane, and writes the same values, so a wave reads back only its
  // own writes: a quarter of the conversions of eight per lane.
  __shared__ __attribute__((aligned(16))) double wpt[kHeadDim];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int slot = tid >> 4;  // block slot within the group (16 lanes of one wave)
  const int g = tid & 15;     // channel group: channels 8g .. 8g+7
  const int64_t group_first = group * kPoolBlocksPerGroup;
  const int64_t blk = group_first + slot;
  int64_t first = a.first_block, count = a.n_blocks;
  if (a.dev_tokens != nullptr) {
    const int64_t complete = live_tokens(a.ceiling, a.dev_tokens, a.status) / kRatio;
    first = complete > a.n_blocks ? complete - a.n_blocks : 0;
    count = complete - first;
  }
  if (count <= 0) return;  // uniform: an empty window
  const bool live = blk < count;
  const int64_t b = first + blk;

  // raw keys first: four 16-byte token rows per lane.  A lane past the range
  // reads the range's last block instead (in bounds; its results are not
  // stored), so every lane loads without a branch.
  uint4 v[4];
  {
    const int64_t bl = live ? b : first + count - 1;
    const uint16_t* base = a.raw + kRatio * bl * a.key_stride + 8 * g;
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
  }
  {
    wpt[2 * lane] = 1.0 + static_cast<double>(bf16_to_f32(a.w[2 * lane]));
    wpt[2 * lane + 1] = 1.0 + static_cast<double>(bf16_to_f32(a.w[2 * lane + 1]));
  }

  // cos/sin at the anchor 4b for the rotary pairs this lane rotates: pairs
  // i = g, g + 16, g + 32, g + 48 below rotary_dim / 2 (computed while the
  // loads are in flight)
  const int half = kHalf > 0 ? kHalf : (a.rp.rotary_dim >> 1);
  constexpr int kPairs = kHalf > 0 ? (kHalf + 15) / 16 : 4;  // pairs per lane, at most
  // (with kHalf 32 the two pairs are the adjacent 2g and 2g + 1 instead)
  const int64_t anchor = kRatio * b;
  auto pair_of = [&](int k) { return kHalf == 32 ? 2 * g + k : g + 16 * k; };
  float fr[kPairs];  // every frequency requested before the first evaluation
#pragma unroll
  for (int k = 0; k < kPairs; ++k) fr[k] = a.rp.inv_freq[pair_of(k)];  // below 64
  uint32_t cs[kPairs];
#pragma unroll
  for (int k = 0; k < kPairs; ++k)
    cs[k] = pair_of(k) < half ? rope_cos_sin_bf16x2(static_cast<int32_t>(anchor), fr[k]) : 0u;  // anchor < 2^31

  // f32 mean of the 4 tokens in token order, cast to bf16.
  float k0[8], k1[8], k2[8], k3[8], m[8];
  unpack_bf16x8(v[0], k0);
  unpack_bf16x8(v[1], k1);
  unpack_bf16x8(v[2], k2);
  unpack_bf16x8(v[3], k3);
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
#pragma clang fp contract(off)
    float s0 = k0[e] + k1[e], s1 = k0[e + 1] + k1[e + 1];
    s0 = s0 + k2[e];
    s1 = s1 + k2[e + 1];
    s0 = s0 + k3[e];
    s1 = s1 + k3[e + 1];
    const uint32_t pk = cvt_pk_bf16(s0 * 0.25f, s1 * 0.25f);
    m[e] = __uint_as_float(pk << 16);
    m[e + 1] = __uint_as_float(pk & 0xFFFF0000u);
  }

  // (1 + w) RMSNorm in double, rounded to f32 and then to bf16.
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += static_cast<double>(m[e]) * static_cast<double>(m[e]);
  const double r = inv_rms(row16_sum(ss), a.rp.eps);
  wave_lds_sync();  // the weight table: this wave's own writes
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
    y[e] = rb_hw(static_cast<float>((static_cast<double>(m[e]) * r) * wpt[8 * g + e]));
  }
  uint16_t* row = &ys[slot][0];
  *reinterpret_cast<uint4*>(row + 8 * g) =
      make_uint4(pool_pack2(y[0], y[1]), pool_pack2(y[2], y[3]), pool_pack2(y[4], y[5]), pool_pack2(y[6], y[7]));
  wave_lds_sync();  // a block's 16 lanes live in one wave

  // Partial RoPE at the block's first token, pair by pair: every product and
  // sum rounds to bf16, o_i = rb(rb(y_i c) - rb(y_{i+h} s)),
  // o_{i+h} = rb(rb(y_{i+h} c) + rb(y_i s)).  All of the row is read before
  // any rotated channel is written back in its place.
  if constexpr (kHalf == 32) {
    // lane g rotates pairs 2g and 2g + 1: one 4-byte word of each half, and
    // every conversion to bf16 takes two values
    const uint32_t xa = *reinterpret_cast<const uint32_t*>(row + 2 * g);       // y_2g, y_2g+1
    const uint32_t xb = *reinterpret_cast<const uint32_t*>(row + 2 * g + 32);  // y_2g+32, y_2g+33
    wave_lds_sync();
    {
#pragma clang fp contract(off)
    const float a0 = __uint_as_float(xa << 16), a1 = __uint_as_float(xa & 0xFFFF0000u);
    const float b0 = __uint_as_float(xb << 16), b1 = __uint_as_float(xb & 0xFFFF0000u);
    const float c0 = __uint_as_float(cs[0] << 16), s0 = __uint_as_float(cs[0] & 0xFFFF0000u);
    const float c1 = __uint_as_float(cs[1] << 16), s1 = __uint_as_float(cs[1] & 0xFFFF0000u);
    const uint32_t pac = cvt_pk_bf16(a0 * c0, a1 * c1);  // rb(y_i c)
    const uint32_t pbs = cvt_pk_bf16(b0 * s0, b1 * s1);  // rb(y_{i+h} s)
    const uint32_t pbc = cvt_pk_bf16(b0 * c0, b1 * c1);  // rb(y_{i+h} c)
    const uint32_t pas = cvt_pk_bf16(a0 * s0, a1 * s1);  // rb(y_i s)
    const uint32_t oa = cvt_pk_bf16(__uint_as_float(pac << 16) - __uint_as_float(pbs << 16),
                                    __uint_as_float(pac & 0xFFFF0000u) - __uint_as_float(pbs & 0xFFFF0000u));
    const uint32_t ob = cvt_pk_bf16(__uint_as_float(pbc << 16) + __uint_as_float(pas << 16),
                                    __uint_as_float(pbc & 0xFFFF0000u) + __uint_as_float(pas & 0xFFFF0000u));
    *reinterpret_cast<uint32_t*>(row + 2 * g) = oa;
    *reinterpret_cast<uint32_t*>(row + 2 * g + 32) = ob;
    }
  } else {
    float x0[kPairs], x1[kPairs];
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int i = g + 16 * k;
      x0[k] = i < half ? bf16_to_f32(row[i]) : 0.0f;
      x1[k] = i < half ? bf16_to_f32(row[i + half]) : 0.0f;
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
#pragma clang fp contract(off)
      const int i = g + 16 * k;
      if (i < half) {
        const float c = __uint_as_float(cs[k] << 16);
        const float sn = __uint_as_float(cs[k] & 0xFFFF0000u);
        const uint32_t pc = cvt_pk_bf16(x0[k] * c, x1[k] * c);    // rb(y_i c), rb(y_{i+h} c)
        const uint32_t ps = cvt_pk_bf16(x1[k] * sn, x0[k] * sn);  // rb(y_{i+h} s), rb(y_i s)
        const uint32_t o = cvt_pk_bf16(__uint_as_float(pc << 16) - __uint_as_float(ps << 16),
                                       __uint_as_float(pc & 0xFFFF0000u) + __uint_as_float(ps & 0xFFFF0000u));
        row[i] = static_cast<uint16_t>(o & 0xFFFFu);
        row[i + half] = static_cast<uint16_t>(o >> 16);
      }
    }
  }
  wave_lds_sync();
  if (live) {
    uint4 out = *reinterpret_cast<const uint4*>(row + 8 * g);
    if (pool_nan_halves(out.x) | pool_nan_halves(out.y) | pool_nan_halves(out.z) | pool_nan_halves(out.w)) {
      // rare: a non-finite key, weight or norm; NaN is written as 0x7FC0
      uint32_t wd[4] = {out.x, out.y, out.z, out.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (pool_nan_halves(wd[i]) & 0x8000u) wd[i] = (wd[i] & 0xFFFF0000u) | 0x7FC0u;
        if (pool_nan_halves(wd[i]) & 0x80000000u) wd[i] = (wd[i] & 0x0000FFFFu) | 0x7FC00000u;
      }
      out = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    uint16_t* dst = a.pooled + b * kHeadDim + 8 * g;
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

}  // namespace qsa
