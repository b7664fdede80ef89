// Query prep: every query head (1 + w) RMSNorm-ed with q_norm_w and roped at
// the row's own position, written once per row as bf16.
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: the query heads are normed and roped at the row position
// before the dot products; the norm and rotary conventions are those of the
// pooled keys (pool_body.h), with bf16 rounding after the norm and after every
// rotary product and sum.
//
// Workgroup: 256 threads = 4 rows = 16 head vectors; 16 lanes per head
// vector, 8 channels per lane.  The cos/sin of the 4 rows are computed once
// per workgroup (one (row, frequency) pair per thread) and shared in LDS.
// The norm runs in double like the pooled keys; roundings to bf16 use the
// hardware's round-to-nearest-even conversion, NaN written as 0x7FC0.
#pragma once

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr int kPrepThreads = 256;
constexpr int kPrepRows = 4;

struct PrepArgs {
  const uint16_t* q;
  int64_t q_stride;
  const int32_t* pos;
  int64_t rows;
  const uint16_t* w;
  int64_t tokens;             // the ceiling when dev_tokens is set
  const int32_t* dev_tokens;  // optional live cache length on the device
  uint16_t* qhat;
  int32_t* status;
  int q_vec;
  RopeParams rp;
};

__device__ __forceinline__ uint4 prep_pack8(const float (&v)[8]) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

// bf16 NaN test of both halves of a packed word (as in the pool): a half is
// NaN exactly when its magnitude bits exceed 0x7F80.
__device__ __forceinline__ uint32_t prep_nan_halves(uint32_t d) {
  return ((d & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
}

// The prepared heads of the kPrepRows rows of group `group`.  kHalf:
// rotary_dim / 2 when fixed at compile time (the launches pick 32 for
// rotary_dim 64), else 0 and taken from the arguments.
template <int kHalf = 0>
__device__ __forceinline__ void prep_group(const PrepArgs& a, int64_t group) {
  __shared__ __attribute__((aligned(16))) uint32_t csq[kPrepRows][kMaxHalfRotary];
  __shared__ __attribute__((aligned(16))) uint4 ys[4 * kPrepRows][16];
  __shared__ int ppos[kPrepRows];
  __shared__ int pvalid[kPrepRows];
  // (1 + w) in double for the 128 channels (kHalf path): every wave converts
  // all of them, two per lane, writing the same values, so a wave reads back
  // only its own writes.
  __shared__ __attribute__((aligned(16))) double wpt[kHalf > 0 ? kHeadDim : 1];

  const int tid = threadIdx.x;
  const int hv = tid >> 4;  // 4 * local row + head
  const int g = tid & 15;   // channels 8g .. 8g+7
  const int lr = hv >> 2;
  const int head = hv & 3;
  const int64_t row0 = group * kPrepRows;
  const int64_t r = row0 + lr;

  uint4 xq = make_uint4(0u, 0u, 0u, 0u);
  if (r < a.rows) {
    const uint16_t* src = a.q + r * a.q_stride + kHeadDim * head + 8 * g;
    if (a.q_vec) {
      xq = *reinterpret_cast<const uint4*>(src);
    } else {
      xq.x = src[0] | (static_cast<uint32_t>(src[1]) << 16);
      xq.y = src[2] | (static_cast<uint32_t>(src[3]) << 16);
      xq.z = src[4] | (static_cast<uint32_t>(src[5]) << 16);
      xq.w = src[6] | (static_cast<uint32_t>(src[7]) << 16);
    }
  }
  double wp[kHalf > 0 ? 1 : 8];
  if constexpr (kHalf > 0) {
    const int lane = tid & 63;
    wpt[2 * lane] = 1.0 + static_cast<double>(bf16_to_f32(a.w[2 * lane]));
    wpt[2 * lane + 1] = 1.0 + static_cast<double>(bf16_to_f32(a.w[2 * lane + 1]));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) wp[e] = 1.0 + static_cast<double>(bf16_to_f32(a.w[8 * g + e]));
  }

  if (tid < kPrepRows) {
    const int64_t rr = row0 + tid;
    int p = 0, ok = 0;
    if (rr < a.rows) {
      p = a.pos[rr];
      ok = p >= 0 && p < live_tokens(a.tokens, a.dev_tokens, a.status);
      if (!ok) atomicOr(a.status, 1);
    }
    ppos[tid] = p;
    pvalid[tid] = ok;
  }
  __syncthreads();

  const int rd = kHalf > 0 ? 2 * kHalf : a.rp.rotary_dim;
  const int half = rd >> 1;
  if (tid < kPrepRows * half) {
    const int rr = tid / half;
    const int i = tid - rr * half;
    csq[rr][i] = rope_cos_sin_bf16x2(ppos[rr], a.rp.inv_freq[i]);
  }

  // (1 + w) RMSNorm in double, rounded to f32 and then to bf16.
  const bool valid = pvalid[lr] != 0;
  float x[8];
  unpack_bf16x8(xq, x);
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += static_cast<double>(x[e]) * static_cast<double>(x[e]);
  const double rinv = inv_rms(row16_sum(ss), a.rp.eps);

  if constexpr (kHalf == 32) {
    // The normed head in LDS as bf16 (a NaN as produced: the output check
    // below writes it as 0x7FC0); lane g then rotates pairs 2g and 2g + 1
    // (one 4-byte word of each half; every conversion takes two values) and
    // the rotated row is read back in 16-byte chunks.
    wave_lds_sync();  // the weight table: this wave's own writes
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
      y[e] = static_cast<float>((static_cast<double>(x[e]) * rinv) * wpt[8 * g + e]);
    }
    uint16_t* row = reinterpret_cast<uint16_t*>(&ys[hv][0]);
    *reinterpret_cast<uint4*>(row + 8 * g) =
        make_uint4(cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3]), cvt_pk_bf16(y[4], y[5]), cvt_pk_bf16(y[6], y[7]));
    __syncthreads();  // the cos/sin table (other waves) and the rows
    const uint32_t xa = *reinterpret_cast<const uint32_t*>(row + 2 * g);       // y_2g, y_2g+1
    const uint32_t xb = *reinterpret_cast<const uint32_t*>(row + 2 * g + 32);  // y_2g+32, y_2g+33
    const uint2 csp = *reinterpret_cast<const uint2*>(&csq[lr][2 * g]);
    wave_lds_sync();  // a head vector's 16 lanes live in one wave
    {
#pragma clang fp contract(off)
      const float a0 = __uint_as_float(xa << 16), a1 = __uint_as_float(xa & 0xFFFF0000u);
      const float b0 = __uint_as_float(xb << 16), b1 = __uint_as_float(xb & 0xFFFF0000u);
      const float c0 = __uint_as_float(csp.x << 16), s0 = __uint_as_float(csp.x & 0xFFFF0000u);
      const float c1 = __uint_as_float(csp.y << 16), s1 = __uint_as_float(csp.y & 0xFFFF0000u);
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
    wave_lds_sync();
    if (r < a.rows) {
      uint4 out = *reinterpret_cast<const uint4*>(row + 8 * g);
      if (prep_nan_halves(out.x) | prep_nan_halves(out.y) | prep_nan_halves(out.z) | prep_nan_halves(out.w)) {
        // rare: a non-finite query, weight or norm; NaN is written as 0x7FC0
        uint32_t wd[4] = {out.x, out.y, out.z, out.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (prep_nan_halves(wd[i]) & 0x8000u) wd[i] = (wd[i] & 0xFFFF0000u) | 0x7FC0u;
          if (prep_nan_halves(wd[i]) & 0x80000000u) wd[i] = (wd[i] & 0x0000FFFFu) | 0x7FC00000u;
        }
        out = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
      if (!valid) out = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(a.qhat + r * (kHeads * kHeadDim) + kHeadDim * head + 8 * g) = out;
    }
    return;
  } else {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
      y[e] = rb_hw(static_cast<float>((static_cast<double>(x[e]) * rinv) * wp[e]));
    }
    ys[hv][g] = prep_pack8(y);
    __syncthreads();

    // RoPE: o_i = rb(rb(y_i c) - rb(y_{i+h} s)), o_{i+h} = rb(rb(y_{i+h} c) + rb(y_i s)).
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = y[e];
    const int c0 = 8 * g;
    if ((half & 7) == 0) {  // chunks of 8 channels never straddle the halves
      if (c0 < rd) {
        const bool first = c0 < half;
        float yp[8];
        unpack_bf16x8(ys[hv][first ? g + (half >> 3) : g - (half >> 3)], yp);
        const int f0 = first ? c0 : c0 - half;
        const uint4 cs0 = *reinterpret_cast<const uint4*>(&csq[lr][f0]);
        const uint4 cs1 = *reinterpret_cast<const uint4*>(&csq[lr][f0 + 4]);
        const uint32_t cs[8] = {cs0.x, cs0.y, cs0.z, cs0.w, cs1.x, cs1.y, cs1.z, cs1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
          const float c = __uint_as_float(cs[e] << 16);
          const float s = __uint_as_float(cs[e] & 0xFFFF0000u);
          const float p0 = rb_hw(y[e] * c);
          const float p1 = rb_hw(yp[e] * s);
          o[e] = rb_hw(first ? p0 - p1 : p0 + p1);
        }
      }
    } else {
      const uint16_t* yrow = reinterpret_cast<const uint16_t*>(&ys[hv][0]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
        const int c = c0 + e;
        if (c < rd) {
          const bool first = c < half;
          const float yp = bf16_to_f32(yrow[first ? c + half : c - half]);
          const uint32_t cs = csq[lr][first ? c : c - half];
          const float p0 = rb_hw(y[e] * __uint_as_float(cs << 16));
          const float p1 = rb_hw(yp * __uint_as_float(cs & 0xFFFF0000u));
          o[e] = rb_hw(first ? p0 - p1 : p0 + p1);
        }
      }
    }
    if (r < a.rows) {
      uint4 out = prep_pack8(o);
      if (!valid) out = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(a.qhat + r * (kHeads * kHeadDim) + kHeadDim * head + c0) = out;
    }
  }
}

}  // namespace qsa
