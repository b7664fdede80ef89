// Block scoring: s[r, b] = sum_h relu(qhat_{r,h} . khat_b) / sqrt(128), b < (p_r+1)/4.
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: each of the row's 4 query heads is (1 + w) RMSNorm-ed and
// roped at the row's own position; relu per head, then the head sum, then the
// 1/sqrt(128) scale, in f32; the review keeps relu NaN-propagating.
//
// MFMA mapping (gfx950, v_mfma_f32_32x32x16_bf16).  The contraction is a GEMM
// with M = rows x 4 heads, N = blocks, K = 128.  M is ordered (row, head) with
// the head fastest, so the 32x32 accumulator of one MFMA tile gives every lane
// the four heads of one (row, block) pair in four consecutive registers: the
// relu / head-sum / scale epilogue never leaves the lane.  This is the shape
// the pages' SIMT kernel avoided on 16x8 tiles; 32-row M tiles fit it exactly.
//
// Workgroup: 4 waves.  WM waves stack along M (8 query rows = 32 M-rows per
// wave), WN = 4 / WM waves stack along N (64 blocks = two 32-block MFMA
// tiles per wave).  Query prep runs once per workgroup into LDS; each wave
// keeps its A fragments (8 x 16 B) in registers for the whole block loop.
// Pooled-key tiles are staged in LDS with a 272-byte row pitch so the
// 32 distinct rows one B-fragment read touches fall in distinct banks.
// A workgroup walks a contiguous range of block tiles and stops at the
// largest visible block count of its rows (causal prefill rows are ragged).
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kScoreThreads = 256;
constexpr int kNPerWave = 64;  // two 32-block MFMA tiles per wave and iteration
constexpr int kPitch = 136;    // LDS row pitch in bf16 elements (272 bytes)
constexpr float kScale = static_cast<float>(0.088388347648318440550);  // 1/sqrt(128)

struct ScoreArgs {
  const uint16_t* q;
  int64_t q_stride;
  const int32_t* pos;
  int64_t rows;
  const uint16_t* w;
  const uint16_t* pooled;
  int64_t tokens;
  float* scores;
  int64_t score_cols;
  int32_t* status;
  int64_t tiles_per_split;
  int64_t row_groups;
  int q_vec;
  int pooled_vec;
  RopeParams rp;
};

__device__ __forceinline__ float relu_keep_nan(float x) { return x < 0.0f ? 0.0f : x; }

template <int WM>
struct ScoreSmem {
  static constexpr int WN = 4 / WM;
  static constexpr int RG = 8 * WM;           // query rows per workgroup
  static constexpr int TILE = kNPerWave * WN;  // blocks per iteration
  // prologue: normed + roped queries, the norm's partner buffer, cos/sin
  static constexpr int kQBytes = RG * 4 * kPitch * 2;
  static constexpr int kPrologueBytes = kQBytes + 16 * kHeadDim * 4 + RG * kMaxHalfRotary * 8;
  // block loop: two key tiles
  static constexpr int kTileBytes = TILE * kPitch * 2;
  static constexpr int kBytes = kPrologueBytes > 2 * kTileBytes ? kPrologueBytes : 2 * kTileBytes;
  static constexpr int kChunks = TILE * 16 / kScoreThreads;  // 16-byte loads per thread per tile
};

template <int WM>
__global__ __launch_bounds__(kScoreThreads) void score_mfma_kernel(const ScoreArgs a) {
  using S = ScoreSmem<WM>;
  constexpr int RG = S::RG;
  constexpr int TILE = S::TILE;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
  __shared__ int nvis[RG];
  __shared__ int ppos[RG];
  __shared__ int sh_nmax;

  uint16_t(*qs)[kPitch] = reinterpret_cast<uint16_t(*)[kPitch]>(smem);
  float(*ybuf)[kHeadDim] = reinterpret_cast<float(*)[kHeadDim]>(smem + S::kQBytes);
  float2(*csq)[kMaxHalfRotary] =
      reinterpret_cast<float2(*)[kMaxHalfRotary]>(smem + S::kQBytes + 16 * kHeadDim * 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t rg = static_cast<int64_t>(blockIdx.x) % a.row_groups;
  const int64_t split = static_cast<int64_t>(blockIdx.x) / a.row_groups;
  const int64_t row0 = rg * RG;

  if (tid < RG) {
    const int64_t r = row0 + tid;
    int n = 0, p = 0;
    if (r < a.rows) {
      p = a.pos[r];
      if (p >= 0 && p < a.tokens)
        n = (p + 1) / kRatio;
      else if (split == 0)
        atomicOr(a.status, 1);
    }
    nvis[tid] = n;
    ppos[tid] = p;
  }
  __syncthreads();
  if (tid == 0) {
    int mx = 0;
    for (int i = 0; i < RG; ++i) mx = nvis[i] > mx ? nvis[i] : mx;
    sh_nmax = mx;
  }
  __syncthreads();
  const int64_t nmax = sh_nmax;
  const int64_t blk_begin = split * a.tiles_per_split * TILE;
  if (blk_begin >= nmax) return;  // uniform across the workgroup
  int64_t blk_end = (split + 1) * a.tiles_per_split * TILE;
  if (blk_end > nmax) blk_end = nmax;

  // ---- key tiles: this thread's 16-byte chunks of a tile, loaded to
  // registers one tile ahead of the MFMAs that read them from LDS.
  uint4 pre[S::kChunks];
  auto fetch = [&](int64_t nb0) {
#pragma unroll
    for (int i = 0; i < S::kChunks; ++i) {
      const int idx = tid + i * kScoreThreads;
      const int64_t bb = nb0 + (idx >> 4);
      const int c = idx & 15;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (bb < blk_end) {
        const uint16_t* src = a.pooled + bb * kHeadDim + 8 * c;
        if (a.pooled_vec) {
          v = *reinterpret_cast<const uint4*>(src);
        } else {
          v.x = src[0] | (static_cast<uint32_t>(src[1]) << 16);
          v.y = src[2] | (static_cast<uint32_t>(src[3]) << 16);
          v.z = src[4] | (static_cast<uint32_t>(src[5]) << 16);
          v.w = src[6] | (static_cast<uint32_t>(src[7]) << 16);
        }
      }
      pre[i] = v;
    }
  };
  auto stash = [&](int buf) {
    uint16_t(*bs)[kPitch] = reinterpret_cast<uint16_t(*)[kPitch]>(smem + buf * S::kTileBytes);
#pragma unroll
    for (int i = 0; i < S::kChunks; ++i) {
      const int idx = tid + i * kScoreThreads;
      *reinterpret_cast<uint4*>(&bs[idx >> 4][8 * (idx & 15)]) = pre[i];
    }
  };
  fetch(blk_begin);  // in flight during the query prep

  // ---- query prep: (1 + w) RMSNorm per head, then RoPE at the row's position.
  const int rd = a.rp.rotary_dim;
  const int half = rd >> 1;
  for (int idx = tid; idx < RG * half; idx += kScoreThreads) {
    const int r = idx / half;
    const int i = idx - r * half;
    float c, s;
    rope_cos_sin(ppos[r], a.rp.inv_freq[i], c, s);
    csq[r][i] = make_float2(c, s);
  }
  const int hv_local = tid >> 4;  // head vector handled by this 16-lane group
  const int g = tid & 15;
  float wv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wv[e] = bf16_to_f32(a.w[8 * g + e]);
  for (int pass = 0; pass < RG * 4 / 16; ++pass) {
    const int hv = pass * 16 + hv_local;  // = 4 * local_row + head
    const int lr = hv >> 2;
    const int h = hv & 3;
    float x[8];
    if (row0 + lr < a.rows && ppos[lr] >= 0 && ppos[lr] < a.tokens) {
      const uint16_t* src = a.q + (row0 + lr) * a.q_stride + kHeadDim * h + 8 * g;
      if (a.q_vec) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_to_f32(wd[i] & 0xFFFFu);
          x[2 * i + 1] = bf16_to_f32(wd[i] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(src[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += static_cast<double>(x[e]) * static_cast<double>(x[e]);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const double rinv = inv_rms(ss, a.rp.eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = norm_channel(x[e], rinv, wv[e]);
      ybuf[hv_local][8 * g + e] = y[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * g + e;
      float o = y[e];
      if (c < rd) {
        const bool first = c < half;
        const float xp = ybuf[hv_local][first ? c + half : c - half];
        const float2 cs = csq[lr][first ? c : c - half];
        o = rope_channel(y[e], xp, cs.x, cs.y, first);
      }
      qs[hv][8 * g + e] = static_cast<uint16_t>(f32_to_bf16(o));
    }
    __syncthreads();
  }

  // ---- A fragments: this wave's 32 M-rows (8 query rows x 4 heads), K = 128.
  const int m = wave % WM;
  const int ng = wave / WM;
  const int mrow = 32 * m + (lane & 31);
  const int khalf = 8 * (lane >> 5);
  bf16x8_t afrag[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    afrag[ks] = *reinterpret_cast<const bf16x8_t*>(&qs[mrow][16 * ks + khalf]);

  // per-lane output rows: this lane holds rows 8m + 2 q4 + (lane >> 5)
  float* orow[4];
  int ovis[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int lr = 8 * m + 2 * q4 + (lane >> 5);
    orow[q4] = a.scores + (row0 + lr) * a.score_cols;
    ovis[q4] = nvis[lr];
  }
  __syncthreads();  // every wave holds its A fragments: the LDS becomes key tiles
  stash(0);
  __syncthreads();

  // ---- block loop: MFMAs on tile t (LDS) while tile t+1 is fetched
  int buf = 0;
  for (int64_t nb0 = blk_begin; nb0 < blk_end; nb0 += TILE) {
    const bool more = nb0 + TILE < blk_end;
    if (more) fetch(nb0 + TILE);
    uint16_t(*bs)[kPitch] = reinterpret_cast<uint16_t(*)[kPitch]>(smem + buf * S::kTileBytes);
    const int col0 = ng * kNPerWave + (lane & 31);
    f32x16_t acc0, acc1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc0[v] = 0.0f;
      acc1[v] = 0.0f;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&bs[col0][16 * ks + khalf]);
      const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&bs[col0 + 32][16 * ks + khalf]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ks], b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ks], b1, acc1, 0, 0, 0);
    }
    const int blk0 = static_cast<int>(nb0) + col0;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float s0 = relu_keep_nan(acc0[4 * q4 + 0]) + relu_keep_nan(acc0[4 * q4 + 1]);
      s0 = s0 + relu_keep_nan(acc0[4 * q4 + 2]);
      s0 = s0 + relu_keep_nan(acc0[4 * q4 + 3]);
      float s1 = relu_keep_nan(acc1[4 * q4 + 0]) + relu_keep_nan(acc1[4 * q4 + 1]);
      s1 = s1 + relu_keep_nan(acc1[4 * q4 + 2]);
      s1 = s1 + relu_keep_nan(acc1[4 * q4 + 3]);
      if (blk0 < ovis[q4]) orow[q4][blk0] = s0 * kScale;
      if (blk0 + 32 < ovis[q4]) orow[q4][blk0 + 32] = s1 * kScale;
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

template <int WM>
hipError_t launch_score_wm(const ScoreArgs& base, hipStream_t stream) {
  using S = ScoreSmem<WM>;
  ScoreArgs a = base;
  const int64_t nb_total = a.tokens / kRatio;
  a.row_groups = (a.rows + S::RG - 1) / S::RG;
  // At least one tile: a workgroup per row group still runs, to flag rows
  // whose position is out of range even when no block is complete.
  int64_t n_tiles = (nb_total + S::TILE - 1) / S::TILE;
  if (n_tiles < 1) n_tiles = 1;
  int64_t splits = (1024 + a.row_groups - 1) / a.row_groups;
  if (splits < 1) splits = 1;
  if (splits > n_tiles) splits = n_tiles;
  a.tiles_per_split = (n_tiles + splits - 1) / splits;
  splits = (n_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  const int64_t grid = a.row_groups * splits;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  score_mfma_kernel<WM><<<dim3(static_cast<unsigned>(grid)), dim3(kScoreThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const uint16_t* q, int64_t q_stride, const int32_t* pos, int64_t rows,
                        const uint16_t* w, const RopeParams& rp, const uint16_t* pooled,
                        int64_t tokens, float* scores, int64_t score_cols, int32_t* status,
                        hipStream_t stream) {
  ScoreArgs a{};
  a.q = q;
  a.q_stride = q_stride;
  a.pos = pos;
  a.rows = rows;
  a.w = w;
  a.pooled = pooled;
  a.tokens = tokens;
  a.scores = scores;
  a.score_cols = score_cols;
  a.status = status;
  a.q_vec = (q_stride % 8 == 0) && (reinterpret_cast<uintptr_t>(q) % 16 == 0);
  a.pooled_vec = reinterpret_cast<uintptr_t>(pooled) % 16 == 0;
  a.rp = rp;
  if (rows >= 32) return launch_score_wm<4>(a, stream);
  if (rows > 8) return launch_score_wm<2>(a, stream);
  return launch_score_wm<1>(a, stream);
}

}  // namespace qsa
