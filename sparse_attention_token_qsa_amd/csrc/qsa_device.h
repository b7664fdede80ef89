// Device-side helpers shared by the pool, score and select kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_rope_math.h"

namespace qsa {

constexpr int kHeads = 4;
constexpr int kHeadDim = 128;
constexpr int kRatio = 4;
constexpr int kMaxKeep = 512;
constexpr int kMaxHalfRotary = 64;
// The live cache length of a launch: the device word when one is given (read
// by every thread; a value outside [0, ceiling] is clamped and sets status bit
// 8 once per launch), else the host count.  Device words let one captured
// graph serve a cache that grows between replays.
__device__ __forceinline__ int64_t live_tokens(int64_t ceiling, const int32_t* dev, int32_t* status) {
  if (dev == nullptr) return ceiling;
  const int64_t t = *dev;
  if (t >= 0 && t <= ceiling) return t;
  if (status != nullptr && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, 8);
  return t < 0 ? 0 : ceiling;
}

// Row group of entry k of XCD x's share when G row groups (G % 8 == 0) are
// dealt to the 8 XCDs, each share walked in ascending k.  On a causal batch a
// row group's length grows linearly with its index, and the launch lasts as
// long as the XCD with the most work: with G % 16 == 0 each pair of entries
// takes group x and its mirror 15 - x of one 16-group band, so every share
// (and every half of a share walked in turn) sums to the same length; else
// the XCD takes every eighth group.  A bijection of [0, G).
__device__ __forceinline__ int xcd_share_group(int x, int k, int G) {
  if ((G & 15) == 0) return 16 * (k >> 1) + ((k & 1) ? 15 - x : x);
  return x + 8 * k;
}

// score scale 1/sqrt(head dim), rounded once to f32
constexpr float kScale = static_cast<float>(0.088388347648318440550);

// Score of one (row, block) pair from its four head dot products: relu per
// head as a comparison (d < 0 ? 0 : d, so NaN stays NaN and -Inf gives 0),
// heads summed in order in f32, then the 1/sqrt(128) scale.
__device__ __forceinline__ float score_exact(float h0, float h1, float h2, float h3) {
#pragma clang fp contract(off)
  const float r0 = h0 < 0.0f ? 0.0f : h0;
  const float r1 = h1 < 0.0f ? 0.0f : h1;
  const float r2 = h2 < 0.0f ? 0.0f : h2;
  const float r3 = h3 < 0.0f ? 0.0f : h3;
  float s = r0 + r1;
  s = s + r2;
  s = s + r3;
  return s * kScale;
}

// The same score in fewer instructions: relu(d) = (d + |d|) / 2, so the head
// sum of the doubled terms, times scale / 2, is the score: doubling commutes
// with every f32 rounding of the sum.  Equal to score_exact whenever the
// result is finite; it differs only where a doubled term or sum overflows or
// a head is -Inf (then -Inf + Inf = NaN), and then the result is +Inf or NaN.
// Callers recompute a non-finite result with score_exact.  A -0.0 head term
// becomes +0.0, which only changes the sign of an all-zero score.  The
// result is >= +0 or NaN, so its bits as an unsigned integer reach
// 0x7F800000 exactly when it is not finite.
__device__ __forceinline__ float score_fast(float h0, float h1, float h2, float h3) {
#pragma clang fp contract(off)
  float s = (h0 + fabsf(h0)) + (h1 + fabsf(h1));
  s = s + (h2 + fabsf(h2));
  s = s + (h3 + fabsf(h3));
  return s * (0.5f * kScale);
}

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Eight packed bf16 (element 2i in the low half of word i) -> floats (exact).
__device__ __forceinline__ void unpack_bf16x8(const uint4 u, float (&v)[8]) {
  const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(wd[i] << 16);
    v[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
  }
}

// float -> bf16 bit pattern, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Round a float to the nearest bf16 value, returned as float.
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// f32 rounded to the nearest bf16 value by the hardware conversion
// (v_cvt_pk_bf16_f32: round to nearest even, like f32_to_bf16 on every
// non-NaN input; a NaN stays a NaN but keeps its sign and payload).
__device__ __forceinline__ float rb_hw(float f) { return static_cast<float>(static_cast<__bf16>(f)); }

// Two floats to packed bf16 (lo in bits 0..15) by the hardware conversion
// (round to nearest even; a NaN keeps its sign and payload), as one
// instruction: left to itself the compiler may split a packed conversion
// whose halves are used apart into two.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// Two floats to packed bf16 (lo in bits 0..15) by the hardware conversion,
// with every NaN written as the canonical 0x7FC0.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (lo != lo) u = (u & 0xFFFF0000u) | 0x7FC0u;
  if (hi != hi) u = (u & 0x0000FFFFu) | 0x7FC00000u;
  return u;
}

// Order-preserving map of a finite float to u32: a larger score gives a
// larger key; -0.0 is folded onto +0.0 so the two zeros tie.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool is_finite_bits(float s) {
  return (__float_as_uint(s) & 0x7F800000u) != 0x7F800000u;
}

// cos and sin, in double, of an angle given as a float with |angle| < 2^18.
// Cody-Waite reduction (Cody and Waite, "Software Manual for the Elementary
// Functions", 1980): k = nearest integer to angle * 2/pi, r = angle - k pi/2
// with pi/2 split in three parts, the first two of 35 significant bits so
// that k * part is exact for |k| < 2^18.  sin r and cos r are their Taylor
// series to r^17 and r^18 (|r| <= pi/4 + a rounding: the first omitted term
// is below 1e-19 relative).  The quadrant k mod 4 then swaps and negates.
__device__ __forceinline__ void cos_sin_small_angle(float angle, double& c, double& s) {
#pragma clang fp contract(off)
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
  constexpr double kPio2a = 0x1.921fb54440000p+0;   // 35 bits
  constexpr double kPio2b = 0x1.68c234c4c0000p-39;  // 35 bits
  constexpr double kPio2c = 0x1.98a2e03707345p-77;
  const double x = static_cast<double>(angle);
  const double k = rint(x * kTwoOverPi);
  double r = __builtin_fma(-k, kPio2a, x);
  r = __builtin_fma(-k, kPio2b, r);
  r = __builtin_fma(-k, kPio2c, r);
  const double r2 = r * r;
  // 1/n! for n = 2 .. 18
  double ps = 0x1.952c77030ad4ap-49;               // 1/17!
  ps = __builtin_fma(ps, r2, -0x1.ae7f3e733b81fp-41);  // -1/15!
  ps = __builtin_fma(ps, r2, 0x1.6124613a86d09p-33);   // 1/13!
  ps = __builtin_fma(ps, r2, -0x1.ae64567f544e4p-26);  // -1/11!
  ps = __builtin_fma(ps, r2, 0x1.71de3a556c734p-19);   // 1/9!
  ps = __builtin_fma(ps, r2, -0x1.a01a01a01a01ap-13);  // -1/7!
  ps = __builtin_fma(ps, r2, 0x1.1111111111111p-7);    // 1/5!
  ps = __builtin_fma(ps, r2, -0x1.5555555555555p-3);   // -1/3!
  const double sr = __builtin_fma(r * r2, ps, r);
  double pc = 0x1.6827863b97d97p-53;               // 1/18!
  pc = __builtin_fma(pc, r2, -0x1.ae7f3e733b81fp-45);  // -1/16!
  pc = __builtin_fma(pc, r2, 0x1.93974a8c07c9dp-37);   // 1/14!
  pc = __builtin_fma(pc, r2, -0x1.1eed8eff8d898p-29);  // -1/12!
  pc = __builtin_fma(pc, r2, 0x1.27e4fb7789f5cp-22);   // 1/10!
  pc = __builtin_fma(pc, r2, -0x1.a01a01a01a01ap-16);  // -1/8!
  pc = __builtin_fma(pc, r2, 0x1.6c16c16c16c17p-10);   // 1/6!
  pc = __builtin_fma(pc, r2, -0x1.5555555555555p-5);   // -1/4!
  pc = __builtin_fma(pc, r2, 0x1.0000000000000p-1);    // 1/2!
  const double cr = __builtin_fma(-r2, pc, 1.0);
  const int q = static_cast<int>(static_cast<int64_t>(k)) & 3;
  const double c0 = (q & 1) ? sr : cr;
  const double s0 = (q & 1) ? cr : sr;
  c = (q == 1 || q == 2) ? -c0 : c0;
  s = (q & 2) ? -s0 : s0;
}

// Rotary angle of position `p` at frequency `f`: one f32 product, then cos
// and sin of that f32 angle rounded to f32 and then to bf16, as if evaluated
// exactly.  Returned packed: cos in bits 0..15, sin in bits 16..31.  The f32
// evaluation (cos_sin_f32) decides the bf16 values whenever both lie
// farther from a bf16 rounding midpoint than its error allowance (about 99.8%
// of the pairs); the rest are evaluated in double (Cody-Waite below 2^18,
// the library cos/sin beyond: positions below 2^18 with frequencies at most
// 1 keep |angle| < 2^18).  Both values are finite (|.| <= 1), so the
// hardware round-to-nearest-even conversion is the bf16 rounding.
__device__ __forceinline__ uint32_t rope_cos_sin_bf16x2(int32_t p, float f) {
#pragma clang fp contract(off)
  const float angle = static_cast<float>(p) * f;  // int32 -> f32 rounds as int64 -> f32 would
  float c = 0.0f, s = 0.0f;
  bool settled = false;
  if (fabsf(angle) < 262144.0f) {
    cos_sin_f32(angle, c, s);
    settled = bf16_rounding_settled(c, kTrigSettle) && bf16_rounding_settled(s, kTrigSettle);
  }
  if (!settled) {
    double sd, cd;
    if (fabsf(angle) < 262144.0f)
      cos_sin_small_angle(angle, cd, sd);
    else
      sincos(static_cast<double>(angle), &sd, &cd);
    c = static_cast<float>(cd);  // the f32 rounding first
    s = static_cast<float>(sd);
  }
  return cvt_pk_bf16(c, s);
}

// Sum over the 16 lanes of a DPP row, returned in all 16 (rotations 8, 4, 2,
// 1; every lane's source lies in its own row, so no old value is needed).  Used on the sums of squares of bf16 values behind the RMSNorm: each
// square has at most 16 significant bits, so a double sum of 128 of them is
// exact, and the same in any order, while the vector's channel magnitudes
// span less than about 2^18 (the smallest square's lowest bit then stays
// above the sum's last place).  A wider span rounds the sum in an order
// that may differ from another implementation's by one double ulp, which
// reaches a bf16 output only through a value within about 2^-52 of an f32
// rounding boundary.
__device__ __forceinline__ double row16_sum(double v) {
#define QSA_ROR_STEP(CTRL)                                                                  \
  {                                                                                         \
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);      \
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);      \
    v += __hiloint2double(hi, lo);                                                          \
  }
  QSA_ROR_STEP(0x128)  // row_ror 8
  QSA_ROR_STEP(0x124)  // row_ror 4
  QSA_ROR_STEP(0x122)  // row_ror 2
  QSA_ROR_STEP(0x121)  // row_ror 1
#undef QSA_ROR_STEP
  return v;
}

// Inverse RMS of a 128-channel vector from its sum of squares (double):
// 1 / sqrt(ss / 128 + eps).
__device__ __forceinline__ double inv_rms(double ss, float eps) {
#pragma clang fp contract(off)
  const double ms = ss / 128.0;
  return 1.0 / sqrt(ms + static_cast<double>(eps));
}

// (1 + w) RMSNorm output of one bf16 channel value x, rounded to bf16.
__device__ __forceinline__ float norm_channel(float x, double r, float w) {
#pragma clang fp contract(off)
  const double y = (static_cast<double>(x) * r) * (1.0 + static_cast<double>(w));
  return round_bf16(static_cast<float>(y));
}

// Rotated value of channel x against its partner xp with bf16 rounding after
// every op: first half  o = rb(rb(x c) - rb(xp s)),
//           second half o = rb(rb(x c) + rb(xp s)).
__device__ __forceinline__ float rope_channel(float x, float xp, float c, float s, bool first_half) {
#pragma clang fp contract(off)
  const float a = round_bf16(x * c);
  const float b = round_bf16(xp * s);
  return round_bf16(first_half ? (a - b) : (a + b));
}

}  // namespace qsa

namespace qsa {

// ---- wavefront primitives (64 lanes) built on DPP row operations --------
//
// update_dpp(old, v, ctrl, rows, banks, bound_ctrl=false) returns v from the
// lane `ctrl` selects, or `old` where that lane is outside the row or the row
// is masked off.  0x111/0x112/0x114/0x118 = row_shr 1/2/4/8 (within 16-lane
// rows), 0x142 = row_bcast 15 (last lane of each row to the next row),
// 0x143 = row_bcast 31 (lane 31 to rows 2 and 3).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += dpp_u32<0x111>(0u, v);
  v += dpp_u32<0x112>(0u, v);
  v += dpp_u32<0x114>(0u, v);
  v += dpp_u32<0x118>(0u, v);
  v += dpp_u32<0x142, 0xA>(0u, v);
  v += dpp_u32<0x143, 0xC>(0u, v);
  return v;
}

// Maximum / minimum over the wave, returned in every lane (uniform).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111>(v, v));
  v = max(v, dpp_u32<0x112>(v, v));
  v = max(v, dpp_u32<0x114>(v, v));
  v = max(v, dpp_u32<0x118>(v, v));
  v = max(v, dpp_u32<0x142, 0xA>(v, v));
  v = max(v, dpp_u32<0x143, 0xC>(v, v));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0x111>(v, v));
  v = min(v, dpp_u32<0x112>(v, v));
  v = min(v, dpp_u32<0x114>(v, v));
  v = min(v, dpp_u32<0x118>(v, v));
  v = min(v, dpp_u32<0x142, 0xA>(v, v));
  v = min(v, dpp_u32<0x143, 0xC>(v, v));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// 64-bit maximum / minimum over the wave (uniform result).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32(static_cast<uint32_t>(v >> 32));
  const uint32_t lo = wave_max_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  const uint32_t hi = wave_min_u32(static_cast<uint32_t>(v >> 32));
  const uint32_t lo = wave_min_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0xFFFFFFFFu);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Order LDS traffic of one wave against itself (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace qsa
