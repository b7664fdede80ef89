// Device helpers shared by the select kernels: the composite order key, the
// wave-level r-th largest search, mask words and the radix threshold search.
// Every function here works on one workgroup's data; see select.hip.
#pragma once

#include "qsa_device.h"

namespace qsa {
namespace sel {

// A register copy the compiler cannot see through: values derived from it
// are computed where they are used instead of being hoisted and kept live
// (64 keys per thread leave no room for 64 precomputed 64-bit composites).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int b) {
  return (static_cast<uint64_t>(key) << 32) |
         static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(b));
}

// The r-th largest (1 <= r <= 64) of the wave's 64 values, in every lane:
// the largest x with at least r lanes holding a value >= x, built bit by bit
// from bit 31 down to bit LOW.  With LOW > 0 it is that value with its bits
// below LOW cleared: still a value that at least r lanes reach, which is all
// the prefilters need of it.
template <int LOW = 0>
__device__ __forceinline__ uint32_t wave_rth_largest(uint32_t v, int r) {
  uint32_t x = 0u;
#pragma unroll
  for (int bit = 31; bit >= LOW; --bit) {
    const uint32_t c = x | (1u << bit);
    if (__popcll(__ballot(v >= c)) >= r) x = c;
  }
  return x;
}

// Streaming (non-temporal) 16-byte score loads and mask stores.  Every score
// and mask byte is touched once, so keeping them out of the caches' normal
// replacement measured faster: a read-64-KiB, write-64-KiB-per-row pattern
// over 8192 rows ran at 6.1 TB/s with both streaming against 4.8 TB/s with
// neither (5.7 with streaming loads alone, 4.0 with streaming stores alone).
typedef float f32x4_nt_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4_nt_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt_t*>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ void store_stream(uint4* p, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
  __builtin_nontemporal_store(u32x4_nt_t{x, y, z, w}, reinterpret_cast<u32x4_nt_t*>(p));
}

// Mask word of the token group [4w, 4w+4) outside the selected blocks: 1 for
// every token t <= last.
__device__ __forceinline__ uint32_t prefix_word(int64_t w, int64_t last) {
  const int64_t t0 = 4 * w;
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) v |= (t0 + i <= last ? 1u : 0u) << (8 * i);
  return v;
}

// Bytes [0, tokens) of a mask row: 1 for t <= last, else 0.
template <int NT, bool VEC>
__device__ __forceinline__ void write_prefix_row(uint8_t* mrow, int64_t tokens, int64_t last) {
  if constexpr (VEC) {
    const int64_t chunks = tokens >> 4;
    for (int64_t c = threadIdx.x; c < chunks; c += NT) {
      store_stream(reinterpret_cast<uint4*>(mrow) + c, prefix_word(4 * c + 0, last), prefix_word(4 * c + 1, last),
                   prefix_word(4 * c + 2, last), prefix_word(4 * c + 3, last));
    }
  } else {
    for (int64_t t = threadIdx.x; t < tokens; t += NT) mrow[t] = t <= last ? 1 : 0;
  }
}

// Radix search for the keep-th largest composite among a candidate set whose
// composites all lie in [lo, hi].  `each(f)` calls f(composite) for every
// candidate this thread owns.  hist holds three 256-bin buffers; the first
// must be zero on entry (with a barrier since).  Returns C* (or the floor of
// a bin whose candidates are all taken: the same kept set among the
// candidates); every thread returns the same value.
//
// The digits are those of the offset c - lo, 8 bits per pass from the top
// bit of hi - lo down.  Offsets spread the candidates by their distance from
// the lowest one: the top bits of a composite are its score's sign and
// exponent, so scores spanning a few binades would otherwise share a handful
// of bins, and LDS atomics on one address serialise.
template <int NT, typename Each>
__device__ uint64_t radix_threshold(Each each, uint32_t k, uint64_t lo, uint64_t hi, uint32_t* hist) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (lo == hi) return hi;
  int top = 63 - __clzll(hi - lo);  // highest bit any offset may have
  uint64_t prefix = 0;              // digits chosen so far (offset bits above `top`)
  for (int pass = 0;; ++pass) {
    uint32_t* h = hist + 256 * (pass % 3);
    uint32_t* next = hist + 256 * ((pass + 1) % 3);
    const int shift = top >= 7 ? top - 7 : 0;
    const int width = top - shift + 1;
    const uint64_t himask = ~((2ull << top) - 1ull);  // offset bits above the digit
    each([&](uint64_t c) {
      const uint64_t d = c - lo;
      if ((d & himask) == prefix) atomicAdd(&h[(d >> shift) & ((1u << width) - 1u)], 1u);
    });
    for (int i = tid; i < 256; i += NT) next[i] = 0u;
    __syncthreads();
    // every wave: lane l holds bins 4l..4l+3; "above" counts larger digits
    const uint4 hv = reinterpret_cast<const uint4*>(h)[lane];
    const uint32_t tot = hv.x + hv.y + hv.z + hv.w;
    const uint32_t incl = wave_incl_sum(tot);
    const uint32_t total = read_lane(incl, 63);
    const uint32_t a3 = total - incl;
    const uint32_t a2 = a3 + hv.w, a1 = a2 + hv.z, a0 = a1 + hv.y;
    uint32_t digit = 0, above = 0, count = 0;
    bool found = false;
    if (a3 < k && k <= a3 + hv.w) { digit = 4 * lane + 3; above = a3; count = hv.w; found = true; }
    if (a2 < k && k <= a2 + hv.z) { digit = 4 * lane + 2; above = a2; count = hv.z; found = true; }
    if (a1 < k && k <= a1 + hv.y) { digit = 4 * lane + 1; above = a1; count = hv.y; found = true; }
    if (a0 < k && k <= a0 + hv.x) { digit = 4 * lane + 0; above = a0; count = hv.x; found = true; }
    const int src = __ffsll(static_cast<unsigned long long>(__ballot(found))) - 1;
    digit = read_lane(digit, src);
    above = read_lane(above, src);
    count = read_lane(count, src);
    prefix |= static_cast<uint64_t>(digit) << shift;
    k -= above;
    if (count == k || shift == 0) return lo + prefix;  // every candidate of bin `digit` is taken
    top = shift - 1;
  }
}

}  // namespace sel
}  // namespace qsa
