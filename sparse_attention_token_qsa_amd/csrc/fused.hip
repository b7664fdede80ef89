// Fused score -> select for prefill batches: the per-row top-(budget/4)
// blocks and the u8 token mask, without writing every block score to HBM.
//
// Semantics are those of the score kernel followed by the selector
// (pegainfer pull request 1178, "select QSA indexer blocks and their tail",
// "Exact semantics"; pull request 1160, summary, for the score): the kept
// set is the keep first blocks under (score descending, block index
// ascending).  pegainfer pull request 1160 lists fusing the select into the
// scoring pass as the next step for long prefill; this is one way to do it
// on gfx950, where the prefill score pass is bound by writing its scores.
//
// 1. Sample pass.  The ring scorer scores every 16th block of each row
//    (blocks 0, 16, 32, ...) into a small workspace matrix.
// 2. Threshold.  Per row, T = the r-th largest sampled score (bits read as
//    an unsigned integer), r = max(ceil(2.5 keep / 16), 32): about 2.5 keep
//    blocks of the row score at least T.  Rows under the budget take T =
//    +Inf (only non-finite scores are of interest there); rows with fewer
//    than r samples take T = 0 (every block).
// 3. Emit pass.  The ring scorer scores every block but stores only the
//    (score bits, block) pairs with score >= T, in fixed-capacity regions per
//    (row, workgroup split, 8-block column group), with exact per-region
//    counts.
// 4. Candidate select, one workgroup per row.  If any stored candidate is
//    non-finite the row is refused.  Otherwise, if every region held its
//    blocks and at least keep blocks reached the threshold, the keep-th
//    largest block lies among the candidates (every candidate scores
//    strictly more than any non-candidate), so an exact radix select over
//    the candidates gives the kept set, and the row's mask is written.  Else
//    the row is flagged.
// 5. Fallback, for flagged rows only: the ring scorer writes the flagged row
//    groups' full scores into the workspace and the one-workgroup-per-row
//    selector selects the flagged rows from them.  Both launches exit at
//    once for unflagged groups and rows.
//
// Every stage is exact: a poor threshold costs time (step 5), never a wrong
// block.
#include "../../include/qsa.h"
#include "qsa_device.h"
#include "qsa_launch.h"
#include "select_common.h"

namespace qsa {
namespace {

using namespace sel;

constexpr int kSampleStride = 16;
constexpr int kCandMax = 2048;  // candidates one row's selector holds
constexpr int kSampleTarget = 256;
constexpr int kEmitTarget = 1024;
// The fallback ring pass usually finds no flagged row group and its
// workgroups exit at once; a quarter of the emit pass's workgroups makes
// that idle launch ~2 us cheaper, and a flagged group is scored by 4
// workgroups instead of 16.
constexpr int kFallbackTarget = 256;

int sample_rank(int keep_max) {
  const int r = (5 * keep_max + 2 * kSampleStride - 1) / (2 * kSampleStride);
  return r > 32 ? r : 32;
}

int64_t align256(int64_t x) { return (x + 255) & ~static_cast<int64_t>(255); }

struct Layout {
  int64_t rows_pad, groups, nb, mcols, splits, cap, score_cols;
  int r;
  int64_t off_samp, off_thr, off_cand, off_cnt, off_rflag, off_gflag, off_scores, total;
};

Layout layout(int64_t rows, int64_t tokens, int keep_max) {
  Layout L{};
  L.groups = (rows + kRingRows - 1) / kRingRows;
  L.rows_pad = L.groups * kRingRows;
  L.nb = tokens / kRatio;
  L.mcols = ((L.nb + kSampleStride - 1) / kSampleStride + 3) & ~static_cast<int64_t>(3);
  L.r = sample_rank(keep_max);
  L.splits = ring_splits(rows, L.nb, kEmitTarget);
  // a region (row, split, 8-block column group) holds all its blocks, or
  // three times its expected share of the row's r * 16 candidates, at least 32
  const int64_t tiles = (L.nb + 31) / 32;
  const int64_t bpr = ((tiles + L.splits - 1) / L.splits) * 8;  // blocks per region
  const int64_t expect = static_cast<int64_t>(L.r) * kSampleStride;
  int64_t cap = (3 * expect + 4 * L.splits - 1) / (4 * L.splits);
  cap = cap > 32 ? cap : 32;
  cap = (cap + 3) & ~static_cast<int64_t>(3);
  L.cap = cap < bpr ? cap : bpr;
  L.score_cols = (L.nb + 3) & ~static_cast<int64_t>(3);
  int64_t at = 0;
  L.off_samp = at;
  at = align256(at + L.rows_pad * L.mcols * 4);
  L.off_thr = at;
  at = align256(at + L.rows_pad * 4);
  L.off_cand = at;
  at = align256(at + L.rows_pad * L.splits * 4 * L.cap * 8);
  L.off_cnt = at;
  at = align256(at + L.rows_pad * L.splits * 4 * 4);
  L.off_rflag = at;
  at = align256(at + L.rows_pad * 4);
  L.off_gflag = at;
  at = align256(at + L.groups * 4);
  L.off_scores = at;
  at = align256(at + rows * L.score_cols * 4);
  L.total = at;
  return L;
}

// ---- 2. per-row threshold from the sampled scores ----
struct ThrArgs {
  const float* samp;
  int64_t mcols;
  const int32_t* pos;
  int64_t rows, rows_pad, tokens;
  int keep_max, r;
  uint32_t* thr;
  int32_t* rflag;
  int32_t* gflag;
};

// One wave per row; KPL sampled scores per lane (KPL * 64 >= the row's).
template <int KPL>
__global__ __launch_bounds__(256) void threshold_kernel(const ThrArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.rows_pad) return;
  if (lane == 0) {
    a.rflag[row] = 0;
    if (row % kRingRows == 0) a.gflag[row / kRingRows] = 0;
  }
  uint32_t t = 0xFFFFFFFFu;  // rows without visible blocks keep nothing
  if (row < a.rows) {
    const int64_t p = a.pos[row];
    if (p >= 0 && p < a.tokens) {
      const int n = static_cast<int>((p + 1) / kRatio);
      const int m = (n + kSampleStride - 1) / kSampleStride;
      if (n <= a.keep_max) {
        t = 0x7F800000u;  // non-finite scores only
      } else if (m < a.r) {
        t = 0u;  // every block
      } else {
        const float* srow = a.samp + row * a.mcols;
        uint32_t v[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
          const int j = lane + 64 * k;
          v[k] = j < m ? __float_as_uint(srow[j]) : 0u;
        }
        // The largest x with at least r values >= x, built bit by bit
        // (absent values are 0 and never counted for x >= 1) over the 16
        // bits below the highest bit any value has: a lower bound of the
        // r-th largest (any lower bound is a valid threshold) that keeps 8
        // mantissa bits.
        uint32_t vmax = 0u;
#pragma unroll
        for (int k = 0; k < KPL; ++k) vmax = v[k] > vmax ? v[k] : vmax;
        vmax = wave_max_u32(vmax);
        uint32_t x = 0u;
        const int top = vmax == 0u ? -1 : 31 - __clz(vmax);
        const int stop = top - 16 > -1 ? top - 16 : -1;
        for (int bit = top; bit > stop; --bit) {
          const uint32_t c = x | (1u << bit);
          uint32_t cnt = 0;  // wave-uniform: popcounts of ballots
#pragma unroll
          for (int k = 0; k < KPL; ++k) cnt += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(v[k] >= c)));
          if (cnt >= static_cast<uint32_t>(a.r)) x = c;
        }
        t = x;
      }
    }
  }
  if (lane == 0) a.thr[row] = t < 0x7F800000u || t == 0xFFFFFFFFu ? t : 0x7F800000u;
}

// ---- 4. candidate select and mask ----
struct CandArgs {
  const int32_t* pos;
  int64_t rows, tokens;
  int keep_max;
  const uint2* cand;
  const int32_t* cnt;
  int splits, cap;
  uint8_t* mask;
  int32_t* status;
  int32_t* rflag;
  int32_t* gflag;
};

// One workgroup per row.
template <bool VEC>
__global__ __launch_bounds__(256) void cand_select_kernel(const CandArgs a) {
  constexpr int NT = 256, NW = NT / 64;
  constexpr int KPT = kCandMax / NT;
  __shared__ __attribute__((aligned(16))) uint32_t hist[3 * 256];
  __shared__ uint64_t red64[2 * NW];
  __shared__ uint32_t wsum[NW];
  __shared__ uint16_t owner[kCandMax];
  // sized at launch: offs[4 splits + 1] then the kept-block bitmap
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  int* offs = reinterpret_cast<int*>(dyn);
  uint32_t* kbits = dyn + ((4 * a.splits + 1 + 3) & ~3);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t T = a.tokens;
  uint8_t* mrow = a.mask + row * T;
  const int64_t p = a.pos[row];
  if (p < 0 || p >= T) {
    write_prefix_row<NT, VEC>(mrow, T, -1);
    if (tid == 0) atomicOr(a.status, QSA_STATUS_BAD_POSITION);
    return;
  }
  const int n = static_cast<int>((p + 1) / kRatio);
  const int S = 4 * a.splits;  // regions of the row
  const int32_t* rcnt = a.cnt + row * S;

  // region sizes, an exclusive scan over them, and overflow
  // (thread t owns regions [t * per, t * per + per))
  const int per = (S + NT - 1) / NT;
  uint32_t mine = 0;
  bool ovf = false;
  for (int i = 0; i < per; ++i) {
    const int s = tid * per + i;
    if (s < S) {
      const int c = rcnt[s];
      ovf |= c > a.cap;
      mine += static_cast<uint32_t>(c < a.cap ? c : a.cap);
    }
  }
  const uint32_t incl = wave_incl_sum(mine);
  if (lane == 63) wsum[wave] = incl;
  for (int i = tid; i < 3 * 256; i += NT) hist[i] = 0u;
  const bool any_ovf = __syncthreads_or(ovf ? 1 : 0) != 0;
  uint32_t at = incl - mine, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    at += w < wave ? wsum[w] : 0u;
    total += wsum[w];
  }
  for (int i = 0; i < per; ++i) {
    const int s = tid * per + i;
    if (s < S) {
      offs[s] = static_cast<int>(at);
      const int c = rcnt[s];
      at += static_cast<uint32_t>(c < a.cap ? c : a.cap);
    }
  }
  if (tid == 0) offs[S] = static_cast<int>(total);
  const bool fits = total <= static_cast<uint32_t>(kCandMax);
  const bool complete = !any_ovf && fits;  // every block at or above the threshold is here
  __syncthreads();
  // owner of every candidate slot: wave w fills the slots of regions w, w + NW, ...
  if (fits) {
    for (int s = wave; s < S; s += NW) {
      const int b = offs[s], e = offs[s + 1];
      for (int i = b + lane; i < e; i += 64) owner[i] = static_cast<uint16_t>(s);
    }
  }
  __syncthreads();
  // the candidates as composites, KPT per thread (0 = absent; keys are >= 2^31)
  const uint2* rbase = a.cand + row * S * a.cap;
  uint64_t cv[KPT];
  bool nonfin = false;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * NT;
    cv[j] = 0ull;
    if (fits && i < static_cast<int>(total)) {
      const int s = owner[i];
      const uint2 e = rbase[static_cast<int64_t>(s) * a.cap + (i - offs[s])];
      nonfin |= (e.x & 0x7F800000u) == 0x7F800000u;
      cv[j] = composite(score_key(__uint_as_float(e.x)), static_cast<int>(e.y));
    }
  }
  if (__syncthreads_or(nonfin ? 1 : 0)) {
    write_prefix_row<NT, VEC>(mrow, T, -1);
    if (tid == 0) atomicOr(a.status, QSA_STATUS_NONFINITE_SCORE);
    return;
  }
  if (n <= a.keep_max) {
    // every visible block kept: the prefix [0, p], once every non-finite
    // score is known to be absent (all of them reach the threshold)
    if (complete) {
      write_prefix_row<NT, VEC>(mrow, T, p);
    } else if (tid == 0) {
      a.rflag[row] = 1;
      a.gflag[row / kRingRows] = 1;
    }
    return;
  }
  const int keep = a.keep_max;
  if (!complete || total < static_cast<uint32_t>(keep)) {
    if (tid == 0) {
      a.rflag[row] = 1;
      a.gflag[row / kRingRows] = 1;
    }
    return;  // the fallback writes this row
  }
  // exact C* among the candidates
  uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    lo = cv[j] != 0ull && cv[j] < lo ? cv[j] : lo;
    hi = cv[j] > hi ? cv[j] : hi;
  }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (lane == 0) {
    red64[wave] = lo;
    red64[NW + wave] = hi;
  }
  const int nwords = (n + 31) / 32;
  for (int i = tid; i < nwords; i += NT) kbits[i] = 0u;
  __syncthreads();
  lo = red64[0];
  hi = red64[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = red64[w] < lo ? red64[w] : lo;
    hi = red64[NW + w] > hi ? red64[NW + w] : hi;
  }
  const uint64_t cstar = radix_threshold<NT>(
      [&](auto f) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (cv[j] != 0ull) f(cv[j]);
      },
      static_cast<uint32_t>(keep), lo, hi, hist);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (cv[j] != 0ull && cv[j] >= cstar) {
      const int b = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(cv[j]));
      atomicOr(&kbits[b >> 5], 1u << (b & 31));
    }
  }
  __syncthreads();
  auto bit = [&](int b) { return (kbits[b >> 5] >> (b & 31)) & 1u; };
  if constexpr (VEC) {
    for (int64_t c = tid; c < T / 16; c += NT) {
      uint32_t wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = static_cast<int>(4 * c + i);
        wv[i] = b < n ? (bit(b) ? 0x01010101u : 0u) : prefix_word(b, p);
      }
      store_stream(reinterpret_cast<uint4*>(mrow) + c, wv[0], wv[1], wv[2], wv[3]);
    }
  } else {
    for (int64_t t2 = tid; t2 < T; t2 += NT) {
      const int b = static_cast<int>(t2 / kRatio);
      mrow[t2] = b < n ? static_cast<uint8_t>(bit(b)) : (t2 <= p ? 1 : 0);
    }
  }
}

}  // namespace

int64_t score_select_workspace_bytes(int64_t rows, int64_t tokens, int keep_max) {
  return layout(rows, tokens, keep_max).total;
}

int64_t score_select_flags_offset(int64_t rows, int64_t tokens, int keep_max) {
  return layout(rows, tokens, keep_max).off_rflag;
}

hipError_t launch_score_select(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                               const uint16_t* pooled, int64_t tokens, int keep_max,
                               uint8_t* mask, int32_t* status, void* workspace,
                               hipStream_t stream) {
  const Layout L = layout(rows, tokens, keep_max);
  if (L.splits > 1024 || L.rows_pad / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* samp = reinterpret_cast<float*>(ws + L.off_samp);
  uint32_t* thr = reinterpret_cast<uint32_t*>(ws + L.off_thr);
  uint2* cand = reinterpret_cast<uint2*>(ws + L.off_cand);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.off_cnt);
  int32_t* rflag = reinterpret_cast<int32_t*>(ws + L.off_rflag);
  int32_t* gflag = reinterpret_cast<int32_t*>(ws + L.off_gflag);
  float* fscores = reinterpret_cast<float*>(ws + L.off_scores);
  hipError_t e;

  // 1. sampled scores
  RingJob j{};
  j.qhat = qhat;
  j.pos = pos;
  j.rows = rows;
  j.pooled = pooled;
  j.tokens = tokens;
  j.bstride = kSampleStride;
  j.scores = samp;
  j.score_cols = L.mcols;
  if ((e = launch_ring(j, kSampleTarget, stream)) != hipSuccess) return e;

  // 2. thresholds (and the flags cleared)
  ThrArgs ta{};
  ta.samp = samp;
  ta.mcols = L.mcols;
  ta.pos = pos;
  ta.rows = rows;
  ta.rows_pad = L.rows_pad;
  ta.tokens = tokens;
  ta.keep_max = keep_max;
  ta.r = L.r;
  ta.thr = thr;
  ta.rflag = rflag;
  ta.gflag = gflag;
  const dim3 tgrid(static_cast<unsigned>(L.rows_pad / 4));
  if (L.mcols <= 1024)
    threshold_kernel<16><<<tgrid, dim3(256), 0, stream>>>(ta);
  else
    threshold_kernel<64><<<tgrid, dim3(256), 0, stream>>>(ta);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 3. candidates
  RingJob k = j;
  k.bstride = 1;
  k.scores = nullptr;
  k.score_cols = 0;
  k.status = status;
  k.thr = thr;
  k.cand = cand;
  k.cnt = cnt;
  k.cap = static_cast<int>(L.cap);
  if ((e = launch_ring(k, kEmitTarget, stream)) != hipSuccess) return e;

  // 4. exact select over the candidates
  CandArgs ca{};
  ca.pos = pos;
  ca.rows = rows;
  ca.tokens = tokens;
  ca.keep_max = keep_max;
  ca.cand = cand;
  ca.cnt = cnt;
  ca.splits = static_cast<int>(L.splits);
  ca.cap = static_cast<int>(L.cap);
  ca.mask = mask;
  ca.status = status;
  ca.rflag = rflag;
  ca.gflag = gflag;
  const bool mvec = (tokens % 16 == 0) && (reinterpret_cast<uintptr_t>(mask) % 16 == 0);
  const dim3 rgrid(static_cast<unsigned>(rows));
  const size_t dyn = 4 * (((4 * L.splits + 1 + 3) & ~static_cast<int64_t>(3)) + (L.nb + 31) / 32);
  if (mvec)
    cand_select_kernel<true><<<rgrid, dim3(256), dyn, stream>>>(ca);
  else
    cand_select_kernel<false><<<rgrid, dim3(256), dyn, stream>>>(ca);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 5. fallback for flagged rows
  RingJob f = j;
  f.bstride = 1;
  f.scores = fscores;
  f.score_cols = L.score_cols;
  f.status = nullptr;
  f.group_flag = gflag;
  if ((e = launch_ring(f, kFallbackTarget, stream)) != hipSuccess) return e;
  return launch_select_flagged(fscores, L.score_cols, pos, rows, tokens, keep_max, mask, status, rflag,
                               stream);
}

}  // namespace qsa
