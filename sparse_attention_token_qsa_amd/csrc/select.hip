// Exact top-(budget/4) block select per row and the u8 token visibility mask.
//
// pegainfer pull request 1178 ("select QSA indexer blocks and their tail"),
// "Exact semantics": n = (p+1)/4 complete blocks, tail = (p+1)%4 tokens at
// 4n..p, keep = min(budget/4, n); the keep first blocks under (score
// descending, block index ascending, -0.0 == +0.0) are kept; the mask is 1 on
// their 4 tokens and on the tail.  A row under the budget keeps its whole
// visible prefix.  A non-finite score in the row's prefix is refused.
//
// One workgroup per row; the row's scores live in registers as order-keys
// (KPT per thread, block b = tid + j * NT) for the whole selection:
//  1. four 8-bit LDS histogram passes over the keys matching the prefix found
//     so far give the keep-th largest key K* and the rank `need` of the cut
//     inside the run of keys equal to K*;
//  2. if fewer than all equal keys are taken, the ascending-index tie fill
//     picks the need-th equal key in block order: per-chunk wavefront
//     ballots count the equal keys, a prefix walk finds the chunk, the wave
//     and the lane; that lane's block index is the last taken one, B*;
//  3. block b is kept iff key_b > K* or (key_b == K* and b <= B*); each thread
//     writes its blocks' 4 mask bytes, then the tail and the zero run.
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
  int words;  // mask rows are 4-byte aligned: write them as u32 words
};

// Mask word covering tokens [4w, 4w+4): 1 for every token t <= last.
__device__ __forceinline__ uint32_t prefix_word(int64_t w, int64_t last) {
  const int64_t t0 = 4 * w;
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) v |= (t0 + i <= last ? 1u : 0u) << (8 * i);
  return v;
}

// Bytes [from, tokens) of a mask row: 1 for t <= last, else 0.
template <int NT>
__device__ __forceinline__ void write_run(uint8_t* mrow, int64_t tokens, int64_t from_word,
                                          int64_t last, bool words) {
  if (words) {
    const int64_t nwords = tokens >> 2;
    for (int64_t w = from_word + threadIdx.x; w < nwords; w += NT)
      reinterpret_cast<uint32_t*>(mrow)[w] = prefix_word(w, last);
    const int64_t rest = tokens & 3;
    if (rest && threadIdx.x == 0)
      for (int64_t t = tokens - rest; t < tokens; ++t) mrow[t] = t <= last ? 1 : 0;
  } else {
    for (int64_t t = 4 * from_word + threadIdx.x; t < tokens; t += NT) mrow[t] = t <= last ? 1 : 0;
  }
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_kernel(const SelectArgs a) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t chunk_cnt[KPT];
  __shared__ uint32_t wave_cnt[NW];
  __shared__ uint32_t sh_digit, sh_above, sh_equal, sh_chunk, sh_need, sh_wave;
  __shared__ int sh_bstar;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t T = a.tokens;
  uint8_t* mrow = a.mask + row * T;
  const int64_t p = a.pos[row];

  if (p < 0 || p >= T) {
    write_run<NT>(mrow, T, 0, -1, a.words);
    if (tid == 0) atomicOr(a.status, 1);
    return;
  }
  const int64_t n = (p + 1) / kRatio;
  const int64_t keep = n < a.keep_max ? n : a.keep_max;

  // Load the visible prefix as order-keys.  A finite score's key is at least
  // 0x00800000, so key 0 marks an absent slot and is never counted.
  const float* srow = a.scores + row * a.score_cols;
  const int n32 = static_cast<int>(n);
  uint32_t key[KPT];
  int bad = 0;
  if (n32 > 0) {
    // Every load is issued before any is consumed; slots past the prefix
    // re-read the last visible score and are then discarded.
    float sv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int b = tid + j * NT;
      sv[j] = srow[b < n32 ? b : n32 - 1];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool live = tid + j * NT < n32;
      bad |= live && !is_finite_bits(sv[j]);
      key[j] = live ? score_key(sv[j]) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = 0u;
  }
  if (__syncthreads_or(bad)) {
    write_run<NT>(mrow, T, 0, -1, a.words);
    if (tid == 0) atomicOr(a.status, 2);
    return;
  }
  if (n <= keep) {  // every block kept: the visible prefix [0, p]
    write_run<NT>(mrow, T, 0, p, a.words);
    return;
  }

  // ---- radix select of the keep-th largest key, 8 bits per pass, MSB first.
  uint32_t prefix = 0u, pmask = 0u, k = static_cast<uint32_t>(keep);
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (key[j] != 0u && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l..4l+3; suffix sums from the top bin down
      uint32_t h[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[4 * lane + i];
        tot += h[i];
      }
      uint32_t incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(incl, off);
        if (lane + off < 64) incl += v;
      }
      uint32_t above = incl - tot;  // keys in bins of higher lanes
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < k && above + h[i] >= k) {
          sh_digit = 4 * lane + i;
          sh_above = above;
          sh_equal = h[i];
        }
        above += h[i];
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    k -= sh_above;
  }
  const uint32_t kstar = prefix;
  const uint32_t need = k;  // taken among the keys equal to K*, 1..equal
  const uint32_t equal = sh_equal;

  int bstar = 0x7FFFFFFF;
  if (need < equal) {
    // ---- ascending-index tie fill: the need-th key equal to K* in block order.
    for (int j = tid; j < KPT; j += NT) chunk_cnt[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t bal = __ballot(key[j] == kstar);
      if (lane == 0 && bal) atomicAdd(&chunk_cnt[j], static_cast<uint32_t>(__popcll(bal)));
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0;
      for (int j = 0; j < KPT; ++j) {
        if (cum + chunk_cnt[j] >= need) {
          sh_chunk = j;
          sh_need = need - cum;
          break;
        }
        cum += chunk_cnt[j];
      }
    }
    __syncthreads();
    const int jstar = static_cast<int>(sh_chunk);
    bool eq_here = false;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j == jstar) eq_here = key[j] == kstar;
    const uint64_t bal = __ballot(eq_here);
    if (lane == 0) wave_cnt[wave] = static_cast<uint32_t>(__popcll(bal));
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0;
      const uint32_t need2 = sh_need;
      for (int w = 0; w < NW; ++w) {
        if (cum + wave_cnt[w] >= need2) {
          sh_wave = w;
          sh_need = need2 - cum;
          break;
        }
        cum += wave_cnt[w];
      }
    }
    __syncthreads();
    if (wave == static_cast<int>(sh_wave) && eq_here) {
      const uint64_t below = bal & ((1ull << lane) - 1ull);
      if (static_cast<uint32_t>(__popcll(below)) + 1u == sh_need)
        sh_bstar = tid + jstar * NT;
    }
    __syncthreads();
    bstar = sh_bstar;
  }

  // ---- mask: kept blocks, then the tail [4n, p] and zeros to the end.
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int b = tid + j * NT;
    if (key[j] != 0u) {
      const bool kept = key[j] > kstar || (key[j] == kstar && b <= bstar);
      if (a.words) {
        reinterpret_cast<uint32_t*>(mrow)[b] = kept ? 0x01010101u : 0u;
      } else {
        const uint8_t v = kept ? 1 : 0;
        mrow[4 * b] = v;
        mrow[4 * b + 1] = v;
        mrow[4 * b + 2] = v;
        mrow[4 * b + 3] = v;
      }
    }
  }
  write_run<NT>(mrow, T, n, p, a.words);
}

template <int NT, int KPT>
hipError_t launch_select_t(const SelectArgs& a, int64_t rows, hipStream_t stream) {
  select_kernel<NT, KPT><<<dim3(static_cast<unsigned>(rows)), dim3(NT), 0, stream>>>(a);
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
  a.words = (tokens % 4 == 0) && (reinterpret_cast<uintptr_t>(mask) % 4 == 0);
  const int64_t nmax = tokens / kRatio;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (nmax <= 256) return launch_select_t<256, 1>(a, rows, stream);
  if (nmax <= 512) return launch_select_t<256, 2>(a, rows, stream);
  if (nmax <= 1024) return launch_select_t<256, 4>(a, rows, stream);
  if (nmax <= 2048) return launch_select_t<256, 8>(a, rows, stream);
  if (nmax <= 4096) return launch_select_t<256, 16>(a, rows, stream);
  if (nmax <= 8192) return launch_select_t<1024, 8>(a, rows, stream);
  if (nmax <= 16384) return launch_select_t<1024, 16>(a, rows, stream);
  if (nmax <= 32768) return launch_select_t<1024, 32>(a, rows, stream);
  if (nmax <= 65536) return launch_select_t<1024, 64>(a, rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace qsa
