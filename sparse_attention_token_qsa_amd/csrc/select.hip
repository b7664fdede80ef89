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
// Scores are loaded and mask bytes stored as streaming (non-temporal) 16-byte
// accesses: each is touched exactly once.
#include "qsa_device.h"
#include "qsa_launch.h"
#include "select_common.h"

namespace qsa {
namespace {

using namespace sel;

struct SelectArgs {
  const float* scores;
  int64_t score_cols;
  const int32_t* pos;
  int64_t tokens;             // mask row length; the ceiling when dev_tokens is set
  const int32_t* dev_tokens;  // optional live cache length on the device
  int keep_max;
  uint8_t* mask;
  int32_t* status;
  int32_t* idx;        // index mode: [rows, idx_stride] kept token indices
  int64_t idx_stride;
  int32_t* counts;     // index mode: [rows] entries written
  int64_t xcd_groups;       // nonzero: rows are visited in group order (row_of)
};

// Row of workgroup b.  Any order gives the same output; the order decides
// which scores are still in the memory-side cache when they are read.  The
// ring scorer (score.hip) deals the 128-row groups of a batch of 1024 g rows
// to the 8 XCDs, g groups per share (xcd_share_group), and each XCD walks its
// share in ascending entry order, so its last workgroups write the last
// entries of every share.  The select visits entry g - 1 of all shares first,
// then g - 2, and so on: workgroup b takes visit k = b / 128, the group of
// entry g - 1 - k / 8 of share k % 8, and row b % 128 of it, a bijection on
// the batch's rows.  Measured on the 8192-row prefill chunk over 64k: 173
// against 178 us in index order.
__device__ __forceinline__ int64_t row_of(const SelectArgs& a, int64_t b) {
  if (a.xcd_groups == 0) return b;
  const int k = static_cast<int>(b >> 7);
  const int g = static_cast<int>(a.xcd_groups);
  return (static_cast<int64_t>(xcd_share_group(k & 7, g - 1 - (k >> 3), 8 * g)) << 7) + (b & 127);
}

// IDX: instead of the mask, row r's kept token indices in ascending order
// (each kept block b as 4b .. 4b + 3, then the tail 4n .. p) go to
// idx[r * idx_stride + i], i < counts[r] = 4 keep + tail, and -1 fills the
// rest of the row's 4 keep_max + 3 entries; a refused row gets count 0.
// The workgroup's LDS for one row, declared by each kernel that selects rows.
template <int NT, int KPT, int TOPM, bool IDX>
struct SelectLds {
  static constexpr int NW = NT / 64;
  static constexpr int kWords = IDX ? (KPT * NT + 31) / 32 : 1;  // bitmap of the row's blocks
  // The prefilter's per-wave rank r = ceil(512 / (NW * TOPM)) must stay <= 32.
  static constexpr bool kPrefilter = NW * TOPM >= 16;
  static constexpr int kCandCap = NT >= 1024 ? 4096 : 2048;
  __attribute__((aligned(16))) uint32_t hist[3 * 256];
  uint32_t red[2 * NW];
  uint64_t cand[kPrefilter ? kCandCap : 1];
  uint32_t ccount;  // candidates compacted (one LDS atomic per wave)
  uint32_t kbits[kWords];
};

// The selection of row row_of(a, b) by the calling workgroup (every thread).
template <int NT, int KPT, int TOPM, bool VEC, bool IDX>
__device__ __forceinline__ void select_row(const SelectArgs& a, uint32_t b, SelectLds<NT, KPT, TOPM, IDX>& L) {
  using LD = SelectLds<NT, KPT, TOPM, IDX>;
  constexpr int NW = LD::NW;
  constexpr int kWords = LD::kWords;
  constexpr bool kPrefilter = LD::kPrefilter;
  constexpr int kCandCap = LD::kCandCap;
  // Few-row geometries (1024 threads per row: decode batches and single
  // rows, latency-bound) take the leaner compaction and mask code below.  The
  // prefill batch keeps the longer forms: its rows stream HBM at the memory
  // system's limit, and the leaner code, with fewer instructions between the
  // stores, measured slower there (compaction 172 -> 178-183 us, mask -> 201).
  constexpr bool kLean = NT >= 1024;
  uint32_t* hist = L.hist;
  uint32_t* red = L.red;
  uint64_t* cand = L.cand;
  uint32_t& ccount = L.ccount;
  uint32_t* kbits = L.kbits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = row_of(a, b);
  const int64_t T = a.tokens;
  uint8_t* mrow = a.mask + row * T;
  const int64_t p = a.pos[row];
  const int64_t live = live_tokens(T, a.dev_tokens, a.status);

  const int cap = 4 * a.keep_max + 3;  // index mode: entries per row
  int32_t* irow = IDX ? a.idx + row * a.idx_stride : nullptr;
  // index mode, rows without a selection: entries i <= last are i, the rest -1
  auto write_prefix_idx = [&](int64_t last) {
    for (int i = tid; i < cap; i += NT) irow[i] = i <= last ? i : -1;
    if (tid == 0) a.counts[row] = static_cast<int32_t>(last + 1);
  };
  if (p < 0 || p >= live) {
    if constexpr (IDX)
      write_prefix_idx(-1);
    else
      write_prefix_row<NT, VEC>(mrow, T, -1);
    if (tid == 0) atomicOr(a.status, 1);
    return;
  }
  const int n = static_cast<int>((p + 1) / kRatio);
  const int keep = n < a.keep_max ? n : a.keep_max;

  // Block of register slot j: 4 consecutive blocks per 16-byte group when
  // vectorised, else one block per slot.
  auto blk = [&](int j) { return VEC ? 4 * (tid + (j >> 2) * NT) + (j & 3) : tid + j * NT; };

  // ---- the visible prefix as order-keys (0 = absent; a finite score's key
  // is at least 0x00800000).  The loads wait for the position: clamped to
  // the row's own prefix they stay within the lines the scorer wrote (a
  // causal prefill row's prefix is shorter than the buffer's width).
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
        v[g] = load_stream(s4 + (q < qlast ? q : qlast));
      }
#pragma unroll
      for (int g = 0; g < KPT / 4; ++g) {
        const float e[4] = {v[g].x, v[g].y, v[g].z, v[g].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = blk(4 * g + i) < n;
          bad |= vis && !is_finite_bits(e[i]);
          key[4 * g + i] = vis ? score_key(e[i]) : 0u;
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
        const bool vis = blk(j) < n;
        bad |= vis && !is_finite_bits(sv[j]);
        key[j] = vis ? score_key(sv[j]) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = 0u;
  }
  if (tid < 256) hist[tid] = 0u;  // first radix buffer; the next barrier publishes it
  if (tid == 0) ccount = 0u;
  if constexpr (IDX)
    for (int i = tid; i < kWords; i += NT) kbits[i] = 0u;
  if (__syncthreads_or(bad)) {
    if constexpr (IDX)
      write_prefix_idx(-1);
    else
      write_prefix_row<NT, VEC>(mrow, T, -1);
    if (tid == 0) atomicOr(a.status, 2);
    return;
  }
  if (n <= keep) {  // every block kept: the visible prefix [0, p]
    if constexpr (IDX)
      write_prefix_idx(p);
    else
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
      // few-row geometries (1024 threads): the bound from the top 16 bits
      // only (a latency-bound row takes 16 fewer ballot steps: 64 rows over
      // 64k 11.3 -> 10.7 us); the prefill batch keeps all 32 (fewer
      // candidates: 175 against 180 us with 16)
      const uint32_t lw = wave_rth_largest<NT >= 1024 ? 16 : 0>(TOPM == 2 ? t2 : t1, r);
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
      // count and compact the candidates key >= L: each wave takes its slot
      // range with one LDS atomic (candidate order does not matter to the
      // search); writes past the capacity are dropped, and such a total
      // sends the row to the exact search over all keys below
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) mine += key[j] >= L ? 1u : 0u;
      const uint32_t incl = wave_incl_sum(mine);
      uint32_t wbase = 0;
      if (lane == 63) wbase = atomicAdd(&ccount, incl);
      if constexpr (kLean) {
        wbase = read_lane(wbase, 63);
        uint32_t at = wbase + incl - mine;
        if (wbase + read_lane(incl, 63) <= static_cast<uint32_t>(kCandCap)) {  // uniform: the wave's slots fit
          // composite low word ~b = ~b0 - (b - b0) from one base per thread;
          // the slot's LDS address advances by 8 bytes per candidate
          const uint32_t nb0 = opaque(~static_cast<uint32_t>(VEC ? 4 * tid : tid));
          uint64_t* slot = cand + at;
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const uint32_t off = VEC ? 4 * (j >> 2) * NT + (j & 3) : j * NT;
            const uint32_t kk = opaque(key[j]);
            if (kk >= L) {
              *slot = (static_cast<uint64_t>(kk) << 32) | (nb0 - off);
              ++slot;
            }
          }
        } else {
          const int t = static_cast<int>(opaque(static_cast<uint32_t>(tid)));
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const int b = VEC ? 4 * (t + (j >> 2) * NT) + (j & 3) : t + j * NT;
            const uint32_t kk = opaque(key[j]);
            if (kk >= L) {
              if (at < static_cast<uint32_t>(kCandCap)) cand[at] = composite(kk, b);
              ++at;
            }
          }
        }
      } else {
        uint32_t at = read_lane(wbase, 63) + incl - mine;
        {
          const int t = static_cast<int>(opaque(static_cast<uint32_t>(tid)));
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const int b = VEC ? 4 * (t + (j >> 2) * NT) + (j & 3) : t + j * NT;
            const uint32_t kk = opaque(key[j]);
            if (kk >= L) {
              if (at < static_cast<uint32_t>(kCandCap)) cand[at] = composite(kk, b);
              ++at;
            }
          }
        }
      }
      __syncthreads();  // every wave has read red[], counted and written
      const uint32_t total = ccount;
      if (total <= static_cast<uint32_t>(kCandCap)) {
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
  if constexpr (IDX) {
    // kept blocks into the bitmap, then each thread takes a run of words:
    // an exclusive scan of the runs' popcounts is the rank of the run's
    // first kept block, and its blocks follow in ascending order.
    const int t = static_cast<int>(opaque(static_cast<uint32_t>(tid)));
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int b = VEC ? 4 * (t + (j >> 2) * NT) + (j & 3) : t + j * NT;
      if (b < n && kept(opaque(key[j]), b)) atomicOr(&kbits[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    const int words = (n + 31) >> 5;
    constexpr int WPT = (kWords + NT - 1) / NT;
    uint32_t wv[WPT];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int w = tid * WPT + i;
      wv[i] = w < words ? kbits[w] : 0u;
      mine += static_cast<uint32_t>(__popc(wv[i]));
    }
    const uint32_t incl = wave_incl_sum(mine);
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    uint32_t rank = incl - mine;
#pragma unroll
    for (int w = 0; w < NW; ++w) rank += w < wave ? red[w] : 0u;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      uint32_t bits = wv[i];
      while (bits) {
        const int b = 32 * (tid * WPT + i) + __ffs(bits) - 1;
        bits &= bits - 1u;
        int32_t* dst = irow + 4 * rank;
        dst[0] = 4 * b;
        dst[1] = 4 * b + 1;
        dst[2] = 4 * b + 2;
        dst[3] = 4 * b + 3;
        ++rank;
      }
    }
    // tail tokens 4n .. p after the 4 keep block tokens, then -1
    const int tail = static_cast<int>(p + 1) - 4 * n;
    for (int i = 4 * keep + tid; i < cap; i += NT) irow[i] = i < 4 * keep + tail ? 4 * n + (i - 4 * keep) : -1;
    if (tid == 0) a.counts[row] = 4 * keep + tail;
    return;
  }
  if constexpr (VEC && kLean) {
    // One test per block: C(b) >= max(C*, lowkey << 32) is kept() (when the
    // search returned a bin floor below lowkey << 32, every candidate is
    // kept, and the candidates are exactly the keys >= lowkey), and it is
    // false for every slot past the prefix (key 0, while lowkey >= 1).  Past
    // the prefix only block n is nonzero: the tail tokens.
    const uint64_t cthr = cstar > (static_cast<uint64_t>(lowkey) << 32) ? cstar : static_cast<uint64_t>(lowkey) << 32;
    const int tail = static_cast<int>(p + 1 - 4 * static_cast<int64_t>(n));  // 0..3
    const uint32_t tailw = tail > 0 ? 0x01010101u >> (32 - 8 * tail) : 0u;
    const int64_t qlim64 = (T + 15) >> 4;  // 16-byte mask chunks in the row
    const int qlim = qlim64 < 0x7FFFFFFF ? static_cast<int>(qlim64) : 0x7FFFFFFF;
    // The test in 32-bit words: key > K, or key == K and b <= ~(low word),
    // K the high word (a 64-bit compare would pair every key register with a
    // scratch register)
    const uint32_t kthr = static_cast<uint32_t>(cthr >> 32);
    const uint32_t bmax = ~static_cast<uint32_t>(cthr);
#pragma unroll
    for (int g = 0; g < KPT / 4; ++g) {
      const int q = tid + g * NT;
      if (q < qlim) {
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t kk = opaque(key[4 * g + i]);
          const uint32_t b = static_cast<uint32_t>(4 * q + i);
          wv[i] = (kk > kthr || (kk == kthr && b <= bmax)) ? 0x01010101u : 0u;
        }
        if (q == (n >> 2)) {  // the chunk holding block n: one lane of the row
          asm volatile("");   // a branch, not selects in every chunk
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[i] = i == (n & 3) ? tailw : wv[i];
        }
        store_stream(reinterpret_cast<uint4*>(mrow) + q, wv[0], wv[1], wv[2], wv[3]);
      }
    }
  } else if constexpr (VEC) {
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
        store_stream(reinterpret_cast<uint4*>(mrow) + q, wv[0], wv[1], wv[2], wv[3]);
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

template <int NT, int KPT, int TOPM, bool VEC, bool IDX>
__global__ __launch_bounds__(NT) void select_kernel(const SelectArgs a) {
  __shared__ SelectLds<NT, KPT, TOPM, IDX> L;
  select_row<NT, KPT, TOPM, VEC, IDX>(a, blockIdx.x, L);
}

// Rows whose flag is nonzero only (the others left untouched), for a caller
// that expects few of them: workgroup w owns rows [w per, w per + per), per
// <= NT, reads their flags with one load per thread, lists the flagged ones
// and selects them one after another.  With nothing flagged the launch costs
// a flag load per row instead of a workgroup per row.
template <int NT, int KPT, int TOPM, bool VEC>
__global__ __launch_bounds__(NT) void select_flagged_kernel(const SelectArgs a, const int32_t* flag, int64_t rows,
                                                             int per) {
  __shared__ SelectLds<NT, KPT, TOPM, false> L;
  __shared__ int32_t list[NT];
  __shared__ uint32_t nlist;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t r = r0 + tid;
  const bool mine = tid < per && r < rows && flag[r] != 0;
  if (tid == 0) nlist = 0u;
  __syncthreads();
  const uint64_t bal = __ballot(mine);
  uint32_t wbase = 0;
  if (lane == 0 && bal != 0ull) wbase = atomicAdd(&nlist, static_cast<uint32_t>(__popcll(bal)));
  wbase = read_lane(wbase, 0);
  if (mine) list[wbase + __popcll(bal & ((1ull << lane) - 1ull))] = static_cast<int32_t>(tid);
  __syncthreads();
  const int n = static_cast<int>(nlist);
  for (int k = 0; k < n; ++k) {
    select_row<NT, KPT, TOPM, VEC, false>(a, static_cast<uint32_t>(r0 + list[k]), L);  // rows in index order
    __syncthreads();  // this row's LDS read everywhere before the next row's
  }
}

// LDS per CU on gfx950.  The prefill-batch select (512 threads, 32 keys per
// thread) runs 3 workgroups per CU faster than 4 (172 against 206 us on the
// 8192-row chunk over 64k; 2 per CU: 217 us), so its launch reserves enough
// unused LDS that a fourth does not fit.
constexpr size_t kLdsPerCu = 160 * 1024;
template <int NT, int KPT, int TOPM, bool IDX>
constexpr size_t select_lds_pad() {
  if (!(NT == 512 && KPT == 32)) return 0;
  constexpr size_t need = kLdsPerCu / 4 + 1024;  // per workgroup, so that 4 exceed the CU and 3 fit
  constexpr size_t have = sizeof(SelectLds<NT, KPT, TOPM, IDX>);
  return need > have ? need - have : 0;
}

template <int NT, int KPT, int TOPM, bool IDX>
hipError_t launch_select_t(const SelectArgs& a, int64_t rows, bool vec, hipStream_t stream) {
  constexpr size_t pad = select_lds_pad<NT, KPT, TOPM, IDX>();
  static_assert(3 * (sizeof(SelectLds<NT, KPT, TOPM, IDX>) + pad) <= kLdsPerCu, "three workgroups fit a CU");
  if (vec)
    select_kernel<NT, KPT, TOPM, true, IDX><<<dim3(static_cast<unsigned>(rows)), dim3(NT), pad, stream>>>(a);
  else
    select_kernel<NT, KPT, TOPM, false, IDX><<<dim3(static_cast<unsigned>(rows)), dim3(NT), pad, stream>>>(a);
  return hipGetLastError();
}

template <bool IDX>
hipError_t launch_select_rows(const SelectArgs& args, int64_t rows, bool vec, hipStream_t stream) {
  const int64_t nmax = args.tokens / kRatio;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  SelectArgs a = args;
  a.xcd_groups = rows % 1024 == 0 ? rows / 1024 : 0;
  if (nmax <= 1024) return launch_select_t<256, 4, 1, IDX>(a, rows, vec, stream);
  if (nmax <= 2048) return launch_select_t<256, 8, 1, IDX>(a, rows, vec, stream);
  if (nmax <= 4096) return launch_select_t<256, 16, 1, IDX>(a, rows, vec, stream);
  if (nmax <= 8192) return launch_select_t<512, 16, 2, IDX>(a, rows, vec, stream);
  // Few rows (decode batches) leave most CUs idle: twice the threads per row
  // shorten each row's load, search and mask phases (64 rows over 64k: 12.3
  // -> 11.1 us); with many rows the 512-thread form keeps more rows in flight.
  if (nmax <= 16384)
    return rows <= 256 ? launch_select_t<1024, 16, 1, IDX>(a, rows, vec, stream)
                       : launch_select_t<512, 32, 2, IDX>(a, rows, vec, stream);
  if (nmax <= 32768) return launch_select_t<1024, 32, 1, IDX>(a, rows, vec, stream);
  if (nmax <= 65536) return launch_select_t<1024, 64, 1, IDX>(a, rows, vec, stream);
  return hipErrorInvalidValue;
}

// The geometries of launch_select_rows; at most 256 workgroups of `per`
// rows each.
template <int NT, int KPT, int TOPM>
hipError_t launch_flagged_t(const SelectArgs& a, const int32_t* flag, int64_t rows, bool vec, hipStream_t stream) {
  int64_t grid = rows < 256 ? rows : 256;
  if (grid < 1) return hipSuccess;
  int64_t per = (rows + grid - 1) / grid;
  if (per > NT) {
    per = NT;
    grid = (rows + per - 1) / per;
  }
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    select_flagged_kernel<NT, KPT, TOPM, true><<<dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream>>>(
        a, flag, rows, static_cast<int>(per));
  else
    select_flagged_kernel<NT, KPT, TOPM, false><<<dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream>>>(
        a, flag, rows, static_cast<int>(per));
  return hipGetLastError();
}

hipError_t launch_select_flagged_rows(const SelectArgs& a, const int32_t* flag, int64_t rows, bool vec,
                                      hipStream_t stream) {
  const int64_t nmax = a.tokens / kRatio;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (nmax <= 1024) return launch_flagged_t<256, 4, 1>(a, flag, rows, vec, stream);
  if (nmax <= 2048) return launch_flagged_t<256, 8, 1>(a, flag, rows, vec, stream);
  if (nmax <= 4096) return launch_flagged_t<256, 16, 1>(a, flag, rows, vec, stream);
  if (nmax <= 8192) return launch_flagged_t<512, 16, 2>(a, flag, rows, vec, stream);
  if (nmax <= 16384) return launch_flagged_t<512, 32, 2>(a, flag, rows, vec, stream);
  if (nmax <= 32768) return launch_flagged_t<1024, 32, 1>(a, flag, rows, vec, stream);
  if (nmax <= 65536) return launch_flagged_t<1024, 64, 1>(a, flag, rows, vec, stream);
  return hipErrorInvalidValue;
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
  return launch_select_rows<false>(a, rows, vec, stream);
}

hipError_t launch_select_flagged(const float* scores, int64_t score_cols, const int32_t* pos,
                                 int64_t rows, int64_t tokens, int keep_max, uint8_t* mask,
                                 int32_t* status, const int32_t* row_flag, hipStream_t stream) {
  SelectArgs a{};
  a.scores = scores;
  a.score_cols = score_cols;
  a.pos = pos;
  a.tokens = tokens;
  a.keep_max = keep_max;
  a.mask = mask;
  a.status = status;
  a.xcd_groups = 0;  // the flagged kernel passes rows, not workgroup indices
  const bool vec = (score_cols % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0) &&
                   (tokens % 16 == 0) && (reinterpret_cast<uintptr_t>(mask) % 16 == 0);
  return launch_select_flagged_rows(a, row_flag, rows, vec, stream);
}

hipError_t launch_select_indices(const float* scores, int64_t score_cols, const int32_t* pos,
                                 int64_t rows, int64_t tokens, int keep_max, int32_t* idx,
                                 int64_t idx_stride, int32_t* counts, int32_t* status,
                                 hipStream_t stream, const int32_t* dev_tokens) {
  SelectArgs a{};
  a.dev_tokens = dev_tokens;
  a.scores = scores;
  a.score_cols = score_cols;
  a.pos = pos;
  a.tokens = tokens;
  a.keep_max = keep_max;
  a.status = status;
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.counts = counts;
  // 16-byte loads of 4 scores
  const bool vec = (score_cols % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  return launch_select_rows<true>(a, rows, vec, stream);
}

}  // namespace qsa
