// Exact top-(budget/4) block select per row and the u8 token visibility mask.
//
// pegainfer pull request 1178 ("select QSA indexer blocks and their tail"),
// "Exact semantics": n = (p+1)/4 complete blocks, tail = (p+1)%4 tokens at
// 4n..p, keep = min(budget/4, n); the keep first blocks under (score
// descending, block index ascending, -0.0 == +0.0) are kept; the mask is 1 on
// their 4 tokens and on the tail.  A row under the budget keeps its whole
// visible prefix.  A non-finite score in the row's prefix is refused.
//
// Order as one integer.  Each visible block gets the 64-bit composite
//   C(b) = key(score_b) << 32 | (0xFFFFFFFF - b),
// with key() the order-preserving u32 map of a finite float (-0.0 folded onto
// +0.0).  The canonical order is C descending and all C are distinct, so the
// kept set is exactly {b : C(b) >= C*} where C* is the keep-th largest
// composite: selection is one threshold, ties included.
//
// One workgroup per row; the row's keys live in registers (KPT per thread).
//  1. Long rows: every thread takes the TOPM-th largest of its own keys; in
//     each wave the r-th largest of those 64 values, r = ceil(keep / (waves
//     * TOPM)), is found by a bitwise search over ballots, and the minimum L
//     over the waves leaves at least keep keys >= L.  So C* >= L << 32 and
//     only keys >= L can be kept.  They are compacted into LDS (typically
//     ~1k of 16k-64k).
//  2. Radix select of C* over the candidates (the compacted list, or all
//     keys when the list would overflow or the row is short), 8 bits per
//     pass starting just below the bits every candidate shares.  A pass is
//     one barrier: the histograms rotate through three LDS buffers (fill
//     one, clear the next), and every wave scans the filled one with DPP and
//     picks the digit itself.  A pass ends the search early once every
//     candidate of the chosen bin is taken; the returned bin floor then
//     separates the candidates, and `lowkey` excludes the non-candidates.
//  3. Each thread writes its blocks' mask bytes (16 bytes per 4 blocks), the
//     tail and the zero run from the same loop.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

struct SelectArgs {
  const float* scores;
  int64_t score_cols;
  const int32_t* pos;
  int64_t tokens;
  int keep_max;
  uint8_t* mask;
  int32_t* status;
};

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
// the largest x with at least r lanes holding a value >= x, built bit by bit.
__device__ __forceinline__ uint32_t wave_rth_largest(uint32_t v, int r) {
  uint32_t x = 0u;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = x | (1u << bit);
    if (__popcll(__ballot(v >= c)) >= r) x = c;
  }
  return x;
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
      uint4 v;
      v.x = prefix_word(4 * c + 0, last);
      v.y = prefix_word(4 * c + 1, last);
      v.z = prefix_word(4 * c + 2, last);
      v.w = prefix_word(4 * c + 3, last);
      reinterpret_cast<uint4*>(mrow)[c] = v;
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
template <int NT, typename Each>
__device__ uint64_t radix_threshold(Each each, uint32_t k, uint64_t lo, uint64_t hi, uint32_t* hist) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (lo == hi) return hi;
  int top = 63 - __clzll(lo ^ hi);                 // highest bit not shared by every candidate
  uint64_t prefix = hi & ~((2ull << top) - 1ull);  // the shared bits above `top`
  for (int pass = 0;; ++pass) {
    uint32_t* h = hist + 256 * (pass % 3);
    uint32_t* next = hist + 256 * ((pass + 1) % 3);
    const int shift = top >= 7 ? top - 7 : 0;
    const int width = top - shift + 1;
    const uint64_t himask = ~((2ull << top) - 1ull);  // bits above the digit
    each([&](uint64_t c) {
      if ((c & himask) == prefix) atomicAdd(&h[(c >> shift) & ((1u << width) - 1u)], 1u);
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
    if (count == k || shift == 0) return prefix;  // every candidate of bin `digit` is taken
    top = shift - 1;
  }
}

template <int NT, int KPT, int TOPM, bool VEC>
__global__ __launch_bounds__(NT) void select_kernel(const SelectArgs a) {
  constexpr int NW = NT / 64;
  // The prefilter's per-wave rank r = ceil(512 / (NW * TOPM)) must stay <= 32.
  constexpr bool kPrefilter = NW * TOPM >= 16;
  constexpr int kCandCap = NT >= 1024 ? 4096 : 2048;
  __shared__ __attribute__((aligned(16))) uint32_t hist[3 * 256];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint64_t cand[kPrefilter ? kCandCap : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t T = a.tokens;
  uint8_t* mrow = a.mask + row * T;
  const int64_t p = a.pos[row];

  if (p < 0 || p >= T) {
    write_prefix_row<NT, VEC>(mrow, T, -1);
    if (tid == 0) atomicOr(a.status, 1);
    return;
  }
  const int n = static_cast<int>((p + 1) / kRatio);
  const int keep = n < a.keep_max ? n : a.keep_max;

  // Block of register slot j: 4 consecutive blocks per 16-byte group when
  // vectorised, else one block per slot.
  auto blk = [&](int j) { return VEC ? 4 * (tid + (j >> 2) * NT) + (j & 3) : tid + j * NT; };

  // ---- load the visible prefix as order-keys (0 = absent; a finite score's
  // key is at least 0x00800000).
  const float* srow = a.scores + row * a.score_cols;
  uint32_t key[KPT];
  int bad = 0;
  if (n > 0) {
    if constexpr (VEC) {
      const float4* s4 = reinterpret_cast<const float4*>(srow);
      const int qlast = (n - 1) >> 2;
      float4 v[KPT / 4];
#pragma unroll
      for (int g = 0; g < KPT / 4; ++g) {
        const int q = tid + g * NT;
        v[g] = s4[q < qlast ? q : qlast];
      }
#pragma unroll
      for (int g = 0; g < KPT / 4; ++g) {
        const float e[4] = {v[g].x, v[g].y, v[g].z, v[g].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool live = blk(4 * g + i) < n;
          bad |= live && !is_finite_bits(e[i]);
          key[4 * g + i] = live ? score_key(e[i]) : 0u;
        }
      }
    } else {
      float sv[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int b = blk(j);
        sv[j] = srow[b < n ? b : n - 1];
      }
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool live = blk(j) < n;
        bad |= live && !is_finite_bits(sv[j]);
        key[j] = live ? score_key(sv[j]) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = 0u;
  }
  if (tid < 256) hist[tid] = 0u;  // first radix buffer; the next barrier publishes it
  if (__syncthreads_or(bad)) {
    write_prefix_row<NT, VEC>(mrow, T, -1);
    if (tid == 0) atomicOr(a.status, 2);
    return;
  }
  if (n <= keep) {  // every block kept: the visible prefix [0, p]
    write_prefix_row<NT, VEC>(mrow, T, p);
    return;
  }

  // ---- threshold composite C*.  The search may return the floor of the bin
  // holding C*; it separates the candidates exactly, and `lowkey` (the
  // prefilter bound, or 1 to exclude absent slots) excludes the rest.
  uint64_t cstar = 0;
  uint32_t lowkey = 1u;
  bool done = false;
  if constexpr (kPrefilter) {
    if (n >= 4 * NT) {  // every thread owns at least four visible blocks
      uint32_t t1 = 0u, t2 = 0u;  // this thread's largest and TOPM-th largest key
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if constexpr (TOPM == 2) t2 = max(t2, min(t1, key[j]));
        t1 = max(t1, key[j]);
      }
      const int r = (keep + NW * TOPM - 1) / (NW * TOPM);
      const uint32_t lw = wave_rth_largest(TOPM == 2 ? t2 : t1, r);
      const uint32_t wmax = wave_max_u32(t1);
      if (lane == 0) {
        red[wave] = lw;
        red[NW + wave] = wmax;
      }
      __syncthreads();
      uint32_t L = red[0], kmax = red[NW];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        L = red[w] < L ? red[w] : L;
        kmax = red[NW + w] > kmax ? red[NW + w] : kmax;
      }
      // count and compact the candidates key >= L
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) mine += key[j] >= L ? 1u : 0u;
      const uint32_t incl = wave_incl_sum(mine);
      __syncthreads();  // every wave has read red[]
      if (lane == 63) red[wave] = incl;
      __syncthreads();
      uint32_t base = 0, total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        base += w < wave ? red[w] : 0u;
        total += red[w];
      }
      if (total <= static_cast<uint32_t>(kCandCap)) {
        uint32_t at = base + incl - mine;
        const int t = static_cast<int>(opaque(static_cast<uint32_t>(tid)));
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const int b = VEC ? 4 * (t + (j >> 2) * NT) + (j & 3) : t + j * NT;
          const uint32_t kk = opaque(key[j]);
          if (kk >= L) cand[at++] = composite(kk, b);
        }
        __syncthreads();
        const int c = static_cast<int>(total);
        cstar = radix_threshold<NT>(
            [&](auto f) {
              for (int i = tid; i < c; i += NT) f(cand[i]);
            },
            static_cast<uint32_t>(keep), static_cast<uint64_t>(L) << 32,
            (static_cast<uint64_t>(kmax) << 32) | 0xFFFFFFFFull, hist);
        lowkey = L;
        done = true;
      }
    }
  }
  if (!done) {
    // exact smallest and largest present key bound the composites
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      kmin = key[j] != 0u && key[j] < kmin ? key[j] : kmin;
      kmax = key[j] > kmax ? key[j] : kmax;
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    __syncthreads();  // red[] may still be read by the prefilter
    if (lane == 0) {
      red[wave] = kmin;
      red[NW + wave] = kmax;
    }
    __syncthreads();
    kmin = red[0];
    kmax = red[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      kmin = red[w] < kmin ? red[w] : kmin;
      kmax = red[NW + w] > kmax ? red[NW + w] : kmax;
    }
    cstar = radix_threshold<NT>(
        [&](auto f) {
          // An opaque copy of the thread index: the composites are rebuilt in
          // every pass instead of being hoisted into 2*KPT live registers.
          int t = tid;
          asm volatile("" : "+v"(t));
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const int b = VEC ? 4 * (t + (j >> 2) * NT) + (j & 3) : t + j * NT;
            const uint32_t kk = opaque(key[j]);
            if (kk != 0u) f(composite(kk, b));
          }
        },
        static_cast<uint32_t>(keep), static_cast<uint64_t>(kmin) << 32,
        (static_cast<uint64_t>(kmax) << 32) | 0xFFFFFFFFull, hist);
  }

  // ---- mask: kept blocks, the tail [4n, p] and zeros; every 16-byte chunk
  // of the row belongs to exactly one register group.  C(b) >= C* splits
  // into 32-bit tests: key > K*, or key == K* and b <= B*.
  const uint32_t khi = static_cast<uint32_t>(cstar >> 32);
  const int64_t blim = 0xFFFFFFFFll - static_cast<int64_t>(static_cast<uint32_t>(cstar));
  auto kept = [&](uint32_t kk, int b) {
    return kk >= lowkey && (kk > khi || (kk == khi && static_cast<int64_t>(b) <= blim));
  };
  if constexpr (VEC) {
#pragma unroll
    for (int g = 0; g < KPT / 4; ++g) {
      const int q = tid + g * NT;
      if (static_cast<int64_t>(q) * 16 < T) {
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 4 * q + i;
          const uint32_t kk = opaque(key[4 * g + i]);
          wv[i] = b < n ? (kept(kk, b) ? 0x01010101u : 0u) : prefix_word(b, p);
        }
        reinterpret_cast<uint4*>(mrow)[q] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int b = blk(j);
      if (b < n) {
        const uint8_t v = kept(opaque(key[j]), b) ? 1 : 0;
        mrow[4 * b] = v;
        mrow[4 * b + 1] = v;
        mrow[4 * b + 2] = v;
        mrow[4 * b + 3] = v;
      }
    }
    for (int64_t t = 4 * static_cast<int64_t>(n) + tid; t < T; t += NT) mrow[t] = t <= p ? 1 : 0;
  }
}

template <int NT, int KPT, int TOPM>
hipError_t launch_select_t(const SelectArgs& a, int64_t rows, bool vec, hipStream_t stream) {
  if (vec)
    select_kernel<NT, KPT, TOPM, true><<<dim3(static_cast<unsigned>(rows)), dim3(NT), 0, stream>>>(a);
  else
    select_kernel<NT, KPT, TOPM, false><<<dim3(static_cast<unsigned>(rows)), dim3(NT), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const float* scores, int64_t score_cols, const int32_t* pos,
                         int64_t rows, int64_t tokens, int keep_max, uint8_t* mask,
                         int32_t* status, hipStream_t stream) {
  SelectArgs a{};
  a.scores = scores;
  a.score_cols = score_cols;
  a.pos = pos;
  a.tokens = tokens;
  a.keep_max = keep_max;
  a.mask = mask;
  a.status = status;
  // 16-byte loads of 4 scores and 16-byte mask stores of 4 blocks
  const bool vec = (score_cols % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0) &&
                   (tokens % 16 == 0) && (reinterpret_cast<uintptr_t>(mask) % 16 == 0);
  const int64_t nmax = tokens / kRatio;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (nmax <= 1024) return launch_select_t<256, 4, 1>(a, rows, vec, stream);
  if (nmax <= 2048) return launch_select_t<256, 8, 1>(a, rows, vec, stream);
  if (nmax <= 4096) return launch_select_t<256, 16, 1>(a, rows, vec, stream);
  if (nmax <= 8192) return launch_select_t<512, 16, 2>(a, rows, vec, stream);
  if (nmax <= 16384) return launch_select_t<512, 32, 2>(a, rows, vec, stream);
  if (nmax <= 32768) return launch_select_t<1024, 32, 1>(a, rows, vec, stream);
  if (nmax <= 65536) return launch_select_t<1024, 64, 1>(a, rows, vec, stream);
  return hipErrorInvalidValue;
}

}  // namespace qsa
