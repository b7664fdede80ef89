// Exact top-(budget/4) block select for few long rows, split over many
// workgroups per row.
//
// pegainfer pull request 1178 ("select QSA indexer blocks and their tail"),
// "Exact semantics": the same kept set and mask as select.hip; only the work
// division differs.  With one workgroup per row, a decode batch of 16-64
// rows of 16k-64k blocks leaves most of the chip idle and streams each row
// through one CU.  Here a row's visible blocks are cut into chunks of
// kSplitChunk blocks:
//
//  1. select_chunk_kernel, one workgroup per (row, chunk): the chunk's
//     exact local top-min(keep, chunk blocks) under the composite order of
//     select.hip, emitted as composites (key << 32 | ~index, global block
//     index) to the caller's workspace.  Every block the row keeps is among
//     its chunk's local top-keep, so the union of the emitted lists holds
//     the row's kept set.  A refused row (bad position, non-finite score)
//     emits a count of -1.
//  2. select_merge_kernel, one workgroup per (row, 16384-token slice): the
//     row's threshold composite C* from the union (at most 16 x 512
//     composites: a prefilter on the keys, then the radix search of
//     select_common.h), and the slice's mask bytes: kept blocks, the tail
//     and the zeros past the row's position.  Every workgroup of a row finds
//     the same C*, so the slices need no exchange.
#include <mutex>

#include "../../include/qsa.h"
#include "qsa_device.h"
#include "qsa_launch.h"
#include "select_common.h"

namespace qsa {
namespace {

using namespace sel;

constexpr int kSplitChunk = 4096;                  // blocks per chunk
constexpr int kSliceTokens = kRatio * kSplitChunk;  // mask bytes per merge workgroup

struct SplitArgs {
  const float* scores;
  int64_t score_cols;
  const int32_t* pos;
  int64_t tokens;             // mask row length; the ceiling when dev_tokens is set
  const int32_t* dev_tokens;  // optional live cache length on the device
  int keep_max;
  uint8_t* mask;
  int32_t* idx;        // index mode: [rows, idx_stride] kept token indices
  int64_t idx_stride;
  int32_t* counts;     // index mode: [rows] entries written
  int32_t* status;
  uint64_t* cand;  // [rows][chunks][kMaxKeep] composites
  int32_t* cnt;    // [rows][chunks] composites emitted, -1 for a refused row
  int chunks;      // chunks (and mask slices) per row
};

// ---- 1. local top-keep of one chunk (512 threads, 8 blocks each) ----------
template <bool VEC>
__global__ __launch_bounds__(512) void select_chunk_kernel(const SplitArgs a) {
  constexpr int NT = 512, KPT = 8, NW = NT / 64, TOPM = 2;
  constexpr int kCandCap = 2048;
  __shared__ __attribute__((aligned(16))) uint32_t hist[3 * 256];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint64_t lcand[kCandCap];
  __shared__ uint32_t ccount;  // candidates compacted (one LDS atomic per wave)
  __shared__ uint32_t wsum[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x / a.chunks;
  const int chunk = static_cast<int>(blockIdx.x - row * a.chunks);
  const int64_t slot = row * a.chunks + chunk;
  const int64_t p = a.pos[row];
  const int64_t live = live_tokens(a.tokens, a.dev_tokens, a.status);
  const int b0 = chunk * kSplitChunk;
  // The chunk's scores are requested before the row's position arrives,
  // clamped to the buffer's first tokens / 4 columns; the keys below keep
  // only the visible ones.
  const float* srow = a.scores + row * a.score_cols + b0;
  const int ncap = static_cast<int>(min(max(a.tokens / kRatio - b0, static_cast<int64_t>(0)),
                                        static_cast<int64_t>(kSplitChunk)));
  float4 v[VEC ? KPT / 4 : 1];
  float sv[VEC ? 1 : KPT];
  if (ncap > 0) {  // uniform
    if constexpr (VEC) {
      const float4* s4 = reinterpret_cast<const float4*>(srow);
      const int qcap = (ncap - 1) >> 2;
#pragma unroll
      for (int g = 0; g < KPT / 4; ++g) {
        const int q = tid + g * NT;
        v[g] = s4[q < qcap ? q : qcap];
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int b = tid + j * NT;
        sv[j] = srow[b < ncap ? b : ncap - 1];
      }
    }
  }
  if (p < 0 || p >= live) {
    if (tid == 0) {
      if (chunk == 0) atomicOr(a.status, QSA_STATUS_BAD_POSITION);
      a.cnt[slot] = -1;
    }
    return;
  }
  const int n_row = static_cast<int>((p + 1) / kRatio);
  const int n = min(max(n_row - b0, 0), kSplitChunk);  // this chunk's visible blocks
  if (n == 0) {
    if (tid == 0) a.cnt[slot] = 0;
    return;
  }
  const int keep = min(n, a.keep_max);
  uint64_t* out = a.cand + slot * kMaxKeep;

  auto blk = [&](int j) { return VEC ? 4 * (tid + (j >> 2) * NT) + (j & 3) : tid + j * NT; };

  uint32_t key[KPT];
  int bad = 0;
  if constexpr (VEC) {
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
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool vis = blk(j) < n;
      bad |= vis && !is_finite_bits(sv[j]);
      key[j] = vis ? score_key(sv[j]) : 0u;
    }
  }
  if (tid < 256) hist[tid] = 0u;
  if (tid == 0) ccount = 0u;
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      atomicOr(a.status, QSA_STATUS_NONFINITE_SCORE);
      a.cnt[slot] = -1;
    }
    return;
  }

  // threshold C* of the chunk (the keep-th largest composite, or the floor of
  // its radix bin; `lowkey` excludes what the prefilter dropped)
  uint64_t cstar = 0;
  uint32_t lowkey = 1u;
  if (n > keep) {
    bool done = false;
    if (n >= 4 * NT) {
      uint32_t t1 = 0u, t2 = 0u;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        t2 = max(t2, min(t1, key[j]));
        t1 = max(t1, key[j]);
      }
      const int r = (keep + NW * TOPM - 1) / (NW * TOPM);
      // the bound from the top 16 bits only: 16 fewer ballot steps in a
      // latency-bound chain (16 rows over 256k: 18.7 -> 17.4 us)
      const uint32_t lw = wave_rth_largest<16>(t2, r);
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
      // compaction: one LDS atomic per wave for its slot range (order does
      // not matter to the search); writes past the capacity are dropped and
      // such a total takes the exact search over all keys below
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) mine += key[j] >= L ? 1u : 0u;
      const uint32_t incl = wave_incl_sum(mine);
      uint32_t wbase = 0;
      if (lane == 63) wbase = atomicAdd(&ccount, incl);
      uint32_t at = read_lane(wbase, 63) + incl - mine;
      {
        const int t = static_cast<int>(opaque(static_cast<uint32_t>(tid)));
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const int b = VEC ? 4 * (t + (j >> 2) * NT) + (j & 3) : t + j * NT;
          const uint32_t kk = opaque(key[j]);
          if (kk >= L) {
            if (at < static_cast<uint32_t>(kCandCap)) lcand[at] = composite(kk, b);
            ++at;
          }
        }
      }
      __syncthreads();  // every wave has read red[], counted and written
      const uint32_t total = ccount;
      if (total <= static_cast<uint32_t>(kCandCap)) {
        const int c = static_cast<int>(total);
        cstar = radix_threshold<NT>(
            [&](auto f) {
              for (int i = tid; i < c; i += NT) f(lcand[i]);
            },
            static_cast<uint32_t>(keep), static_cast<uint64_t>(L) << 32,
            (static_cast<uint64_t>(kmax) << 32) | 0xFFFFFFFFull, hist);
        lowkey = L;
        done = true;
      }
    }
    if (!done) {
      uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        kmin = key[j] != 0u && key[j] < kmin ? key[j] : kmin;
        kmax = key[j] > kmax ? key[j] : kmax;
      }
      kmin = wave_min_u32(kmin);
      kmax = wave_max_u32(kmax);
      __syncthreads();
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
  }

  // ---- emit the chunk's kept composites with their row-global block index
  // (keep of them: the chunk's whole prefix when n <= keep)
  const uint32_t khi = static_cast<uint32_t>(cstar >> 32);
  const int64_t blim = 0xFFFFFFFFll - static_cast<int64_t>(static_cast<uint32_t>(cstar));
  // slots from a block prefix sum of the kept counts
  uint32_t keptbits = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int b = blk(j);
    const uint32_t kk = key[j];
    const bool kept = b < n && (n <= keep || (kk >= lowkey && (kk > khi || (kk == khi && b <= blim))));
    keptbits |= (kept ? 1u : 0u) << j;
  }
  const uint32_t mine = static_cast<uint32_t>(__popc(keptbits));
  const uint32_t incl = wave_incl_sum(mine);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t at = incl - mine;
#pragma unroll
  for (int w = 0; w < NW; ++w) at += w < wave ? wsum[w] : 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((keptbits >> j) & 1u) out[at++] = composite(key[j], b0 + blk(j));
  if (tid == 0) a.cnt[slot] = keep;
}

// ---- 2. the row's threshold from the union, and one slice of its mask ----
// IDX: instead of the mask slice, the slice's part of the row's index list
// (see select.hip's index mode): its kept blocks' tokens at the position the
// kept blocks of the earlier chunks leave free; slice 0 also writes the
// tail, the -1 fill and the count.
template <bool VEC, bool IDX>
__global__ __launch_bounds__(1024) void select_merge_kernel(const SplitArgs a) {
  constexpr int NT = 1024, NW = NT / 64;
  constexpr int KPT = 8;  // composites per thread: 16 chunks x 512 / 1024
  constexpr int kCandCap = 4096;
  __shared__ __attribute__((aligned(16))) uint32_t hist[3 * 256];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint64_t lcand[kCandCap];
  __shared__ uint32_t ccount;  // candidates compacted (one LDS atomic per wave)
  __shared__ int cnts[64];
  __shared__ int offs[65];
  __shared__ int kcount[64];  // index mode: kept blocks per chunk
  __shared__ __attribute__((aligned(16))) uint32_t keptbits[kSplitChunk / 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x / a.chunks;
  const int slice = static_cast<int>(blockIdx.x - row * a.chunks);
  const int64_t T = a.tokens;
  uint8_t* mrow = a.mask + row * T;
  const int64_t t_begin = static_cast<int64_t>(slice) * kSliceTokens;
  const int64_t t_end = min(t_begin + kSliceTokens, T);
  const int64_t p = a.pos[row];
  const int64_t live = live_tokens(T, a.dev_tokens, nullptr);

  // this slice's bytes: block bytes from keptbits (kept = 1), the rest 1 for
  // t <= last, 0 otherwise
  const int cap = 4 * a.keep_max + 3;  // index mode: entries per row
  int32_t* irow = IDX ? a.idx + row * a.idx_stride : nullptr;
  // index mode, rows without a selection: entries i <= last are i (this
  // slice's tokens), and slice 0 writes the -1 fill and the count
  auto write_prefix_idx = [&](int64_t last) {
    for (int64_t t = t_begin + tid; t < t_end && t <= last; t += NT) irow[t] = static_cast<int32_t>(t);
    if (slice == 0) {
      for (int i = static_cast<int>(last + 1) + tid; i < cap; i += NT) irow[i] = -1;
      if (tid == 0) a.counts[row] = static_cast<int32_t>(last + 1);
    }
  };
  auto write_slice = [&](int n, int64_t last, bool use_bits) {
    if constexpr (IDX) {
      write_prefix_idx(use_bits ? -1 : last);  // never called with use_bits in index mode
      return;
    }
    const int blk0 = slice * kSplitChunk;
    if constexpr (VEC) {
      for (int64_t c = t_begin / 16 + tid; c < t_end / 16; c += NT) {
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = static_cast<int>(4 * c + i);
          if (b < n && use_bits) {
            const int lb = b - blk0;
            wv[i] = (keptbits[lb >> 5] >> (lb & 31)) & 1u ? 0x01010101u : 0u;
          } else {
            wv[i] = prefix_word(b, last);
          }
        }
        reinterpret_cast<uint4*>(mrow)[c] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    } else {
      for (int64_t t = t_begin + tid; t < t_end; t += NT) {
        const int b = static_cast<int>(t / kRatio);
        uint8_t v;
        if (b < n && use_bits) {
          const int lb = b - blk0;
          v = (keptbits[lb >> 5] >> (lb & 31)) & 1u;
        } else {
          v = t <= last ? 1 : 0;
        }
        mrow[t] = v;
      }
    }
  };

  // The union's slots, loaded before the position and the counts arrive:
  // every chunk before the row's last visible one is full (4096 >= keep
  // blocks) and emitted exactly keep composites, so slot i is entry i % keep
  // of chunk i / keep; slots past the emitted total are cleared once the
  // counts are known.
  const int keep = a.keep_max;
  const uint64_t* base = a.cand + row * a.chunks * kMaxKeep;
  uint64_t cv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * NT;
    const int c = i / keep;
    cv[j] = c < a.chunks ? base[static_cast<int64_t>(c) * kMaxKeep + (i - c * keep)] : 0ull;
  }
  const int mycnt = tid < a.chunks ? a.cnt[row * a.chunks + tid] : 0;
  if (p < 0 || p >= live) {
    write_slice(0, -1, false);
    return;
  }
  const int n = static_cast<int>((p + 1) / kRatio);
  if (tid < a.chunks) cnts[tid] = mycnt;
  if (tid < 64) kcount[tid] = 0;
  if (tid < kSplitChunk / 32) keptbits[tid] = 0u;
  if (tid < 256) hist[tid] = 0u;
  if (tid == 0) ccount = 0u;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    bool refused = false;
    for (int c = 0; c < a.chunks; ++c) {
      offs[c] = acc;
      refused |= cnts[c] < 0;
      acc += cnts[c] > 0 ? cnts[c] : 0;
    }
    offs[a.chunks] = refused ? -1 : acc;
  }
  __syncthreads();
  const int total = offs[a.chunks];
  if (total < 0) {  // refused row: all zero
    write_slice(0, -1, false);
    return;
  }
  if (n <= a.keep_max) {  // every visible block kept: the prefix [0, p]
    write_slice(0, p, false);
    return;
  }

  // the union, KPT composites per thread (0 = absent)
#pragma unroll
  for (int j = 0; j < KPT; ++j) cv[j] = tid + j * NT < total ? cv[j] : 0ull;
  // prefilter: the wave's r-th largest thread maximum, minimum over waves
  uint32_t t1 = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) t1 = max(t1, static_cast<uint32_t>(cv[j] >> 32));
  const int r = (keep + NW - 1) / NW;
  const uint32_t lw = wave_rth_largest<16>(t1, r);  // top 16 bits, as in the chunk kernel
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
  L = L > 1u ? L : 1u;  // absent slots (0) never count
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) mine += static_cast<uint32_t>(cv[j] >> 32) >= L ? 1u : 0u;
  const uint32_t incl = wave_incl_sum(mine);
  uint32_t wbase = 0;
  if (lane == 63) wbase = atomicAdd(&ccount, incl);
  uint32_t at = read_lane(wbase, 63) + incl - mine;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (static_cast<uint32_t>(cv[j] >> 32) >= L) {
      if (at < static_cast<uint32_t>(kCandCap)) lcand[at] = cv[j];
      ++at;
    }
  __syncthreads();  // every wave has read red[], counted and written
  const uint32_t ctotal = ccount;
  uint64_t cstar;
  uint32_t lowkey;
  if (ctotal <= static_cast<uint32_t>(kCandCap)) {
    const int c = static_cast<int>(ctotal);
    cstar = radix_threshold<NT>(
        [&](auto f) {
          for (int i = tid; i < c; i += NT) f(lcand[i]);
        },
        static_cast<uint32_t>(keep), static_cast<uint64_t>(L) << 32,
        (static_cast<uint64_t>(kmax) << 32) | 0xFFFFFFFFull, hist);
    lowkey = L;
  } else {
    uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      lo = cv[j] != 0ull && cv[j] < lo ? cv[j] : lo;
      hi = cv[j] > hi ? cv[j] : hi;
    }
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    __syncthreads();
    uint64_t* red64 = reinterpret_cast<uint64_t*>(lcand);
    if (lane == 0) {
      red64[wave] = lo;
      red64[NW + wave] = hi;
    }
    __syncthreads();
    lo = red64[0];
    hi = red64[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      lo = red64[w] < lo ? red64[w] : lo;
      hi = red64[NW + w] > hi ? red64[NW + w] : hi;
    }
    __syncthreads();  // red64 aliases lcand, unused below
    cstar = radix_threshold<NT>(
        [&](auto f) {
#pragma unroll
          for (int j = 0; j < KPT; ++j)
            if (cv[j] != 0ull) f(cv[j]);
        },
        static_cast<uint32_t>(keep), lo, hi, hist);
    lowkey = 1u;
  }
  // kept blocks of this slice into the bitmap
  const uint32_t khi = static_cast<uint32_t>(cstar >> 32);
  const uint32_t klo = static_cast<uint32_t>(cstar);
  const int blk0 = slice * kSplitChunk;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t kk = static_cast<uint32_t>(cv[j] >> 32);
    const uint32_t lo32 = static_cast<uint32_t>(cv[j]);
    const bool kept = cv[j] != 0ull && kk >= lowkey && (kk > khi || (kk == khi && lo32 >= klo));
    const int b = static_cast<int>(0xFFFFFFFFu - lo32);
    if (kept && b >= blk0 && b < blk0 + kSplitChunk) {
      const int lb = b - blk0;
      atomicOr(&keptbits[lb >> 5], 1u << (lb & 31));
    }
    if constexpr (IDX)
      if (kept) atomicAdd(&kcount[b / kSplitChunk], 1);
  }
  __syncthreads();
  if constexpr (!IDX) {
    write_slice(n, p, true);
  } else {
    // this slice's kept blocks follow those of the earlier chunks, ascending
    int before = 0;
    for (int c = 0; c < slice; ++c) before += kcount[c];
    constexpr int kWords = kSplitChunk / 32;
    const uint32_t word = tid < kWords ? keptbits[tid] : 0u;
    const uint32_t pc = static_cast<uint32_t>(__popc(word));
    const uint32_t incl = wave_incl_sum(pc);  // waves 0 and 1 hold the 128 words
    if (lane == 63 && wave < 2) red[wave] = incl;
    __syncthreads();
    uint32_t rank = incl - pc + (wave == 1 ? red[0] : 0u);
    uint32_t wb = word;
    while (wb != 0u) {
      const int bit = __ffs(wb) - 1;
      wb &= wb - 1u;
      const int b = blk0 + 32 * tid + bit;
      const int at = 4 * (before + static_cast<int>(rank));
#pragma unroll
      for (int k = 0; k < kRatio; ++k) irow[at + k] = kRatio * b + k;
      ++rank;
    }
    if (slice == 0) {
      const int tail = static_cast<int>(p + 1) - kRatio * n;
      for (int i = tid; i < cap - 4 * keep; i += NT)
        irow[4 * keep + i] = i < tail ? kRatio * n + i : -1;
      if (tid == 0) a.counts[row] = 4 * keep + tail;
    }
  }
}

}  // namespace

int64_t select_split_chunks(int64_t tokens) {
  return (tokens + kSliceTokens - 1) / kSliceTokens;
}

int64_t select_split_workspace_bytes(int64_t rows, int64_t tokens) {
  const int64_t chunks = select_split_chunks(tokens);
  return rows * chunks * (kMaxKeep * static_cast<int64_t>(sizeof(uint64_t)) + 256);
}

bool select_split_pays(int64_t rows, int64_t tokens) {
  // rows past 16384 blocks (64k tokens), and too few of them to fill the
  // chip one workgroup per row; shorter rows finish sooner on one workgroup
  // than through the two launches
  return tokens / kRatio > 4 * kSplitChunk && rows <= 128;
}

namespace {

hipError_t launch_split(SplitArgs a, int64_t rows, bool idx_mode, void* workspace, hipStream_t stream) {
  const int64_t chunks = select_split_chunks(a.tokens);
  if (chunks > 64 || rows * chunks > 0x7FFFFFFF) return hipErrorInvalidValue;
  a.chunks = static_cast<int>(chunks);
  // candidates first (16-byte aligned), then the per-chunk counts
  a.cand = static_cast<uint64_t*>(workspace);
  a.cnt = reinterpret_cast<int32_t*>(a.cand + rows * chunks * kMaxKeep);
  const dim3 grid(static_cast<unsigned>(rows * chunks));
  const bool svec = (a.score_cols % 4 == 0) && (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0);
  if (svec)
    select_chunk_kernel<true><<<grid, dim3(512), 0, stream>>>(a);
  else
    select_chunk_kernel<false><<<grid, dim3(512), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (idx_mode) {
    select_merge_kernel<false, true><<<grid, dim3(1024), 0, stream>>>(a);
  } else {
    const bool mvec = (a.tokens % 16 == 0) && (reinterpret_cast<uintptr_t>(a.mask) % 16 == 0);
    if (mvec)
      select_merge_kernel<true, false><<<grid, dim3(1024), 0, stream>>>(a);
    else
      select_merge_kernel<false, false><<<grid, dim3(1024), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_split(const float* scores, int64_t score_cols, const int32_t* pos,
                               int64_t rows, int64_t tokens, int keep_max, uint8_t* mask,
                               int32_t* status, void* workspace, hipStream_t stream) {
  SplitArgs a{};
  a.scores = scores;
  a.score_cols = score_cols;
  a.pos = pos;
  a.tokens = tokens;
  a.keep_max = keep_max;
  a.mask = mask;
  a.status = status;
  return launch_split(a, rows, false, workspace, stream);
}

hipError_t launch_select_split_indices(const float* scores, int64_t score_cols, const int32_t* pos,
                                       int64_t rows, int64_t tokens, int keep_max, int32_t* idx,
                                       int64_t idx_stride, int32_t* counts, int32_t* status,
                                       void* workspace, hipStream_t stream, const int32_t* dev_tokens) {
  SplitArgs a{};
  a.scores = scores;
  a.score_cols = score_cols;
  a.pos = pos;
  a.tokens = tokens;
  a.dev_tokens = dev_tokens;
  a.keep_max = keep_max;
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.counts = counts;
  a.status = status;
  return launch_split(a, rows, true, workspace, stream);
}

// ---- scratch for callers that cannot allocate ---------------------------
//
// qsa_select_mask_noalloc runs the split select on this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds
// its own copy (QSA_NOALLOC_SCRATCH_BYTES) until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress, once per device, on the first call
// made with that device current, and only that address reaches the kernels.
// The split kernels write every workspace word they read, so nothing is
// cleared between calls; calls that overlap on one GPU share the array and
// race.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace qsa
