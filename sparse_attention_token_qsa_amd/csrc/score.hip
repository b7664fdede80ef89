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
// Workgroup: 4 waves.  WM waves stack along M, each holding MS M-subtiles
// (8 query rows = 32 M-rows each) as A fragments in registers for the whole
// block loop; WN = 4 / WM waves stack along N, one 32-block MFMA tile each
// per step.  Every B fragment read from LDS feeds MS MFMAs.  The queries come
// either prepared (qsa_prep_queries) straight from memory into the A
// fragments, or are normed and roped in a per-workgroup LDS prologue.
//
// Key tiles stream through a ring of D LDS stages, loaded by the memory
// engine straight into LDS (global_load_lds_dwordx4: no register staging)
// D - 1 steps ahead of their MFMAs.  A stage holds TILE 256-byte block rows
// with the 16-byte chunk c of row r stored at chunk c ^ (r & 7), so the 32
// rows one B-fragment read touches spread over all banks.  Loads and the
// branch-free score stores retire in issue order, so each step waits only
// for its own tile's loads, not for the stores issued after them.
// A workgroup walks a contiguous range of block tiles and stops at the
// largest visible block count of its rows (causal prefill rows are ragged).
#include <utility>

#include "prep_body.h"
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kScoreThreads = 256;
constexpr int kPitch = 136;  // prologue LDS row pitch in bf16 elements (272 bytes)
constexpr int kStoreNT = 2;  // buffer-store cache policy: nt

struct ScoreArgs {
  const uint16_t* qhat;  // prepared queries [rows, 4, 128] bf16 (PREP kernels)
  const uint16_t* q;
  int64_t q_stride;
  const int32_t* pos;
  int64_t rows;
  const uint16_t* w;
  const uint16_t* pooled;
  int64_t tokens;             // the ceiling when dev_tokens is set
  const int32_t* dev_tokens;  // optional live cache length on the device
  float* scores;
  int64_t score_cols;
  int32_t* status;
  int64_t splits;  // workgroups per row group; split s takes tiles s, s + splits, ...
  int64_t row_groups;
  int64_t tasks;
  int q_vec;
  RopeParams rp;
};

// Waits on the vector-memory counter only (expcnt / lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Waits until this wave's LDS operations have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (3 << 14)); }

__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
  uint4 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
  o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
  return o;
}

// Workgroup geometry.
template <int WM, int MS, int D, bool PREP>
struct ScoreGeom {
  static constexpr int WN = 4 / WM;
  static constexpr int RG = 8 * MS * WM;       // query rows per workgroup
  static constexpr int TILE = 32 * WN;         // blocks per step
  static constexpr int NPASS = RG * 4 / 16;    // head vectors per 16-lane group (prologue)
  static constexpr int kLoads = TILE / 16;     // 1 KiB LDS loads per wave per tile
  static constexpr int kStores = 4 * MS;       // score stores per wave per step
  static constexpr int kStageBytes = TILE * 256;
  // prologue: normed + roped queries, then packed bf16 (cos, sin) per row and frequency
  static constexpr int kQBytes = RG * 4 * kPitch * 2;
  static constexpr int kPrologueBytes = PREP ? 0 : kQBytes + RG * kMaxHalfRotary * 4;
  static constexpr int kRingBytes = D * kStageBytes;
  static constexpr int kBytes = kPrologueBytes > kRingBytes ? kPrologueBytes : kRingBytes;
};

template <int WM, int MS, int D, bool BUFST, bool PREP>
__global__ __launch_bounds__(kScoreThreads) void score_mfma_kernel(const ScoreArgs a) {
  using G = ScoreGeom<WM, MS, D, PREP>;
  constexpr int RG = G::RG;
  constexpr int TILE = G::TILE;
  constexpr int NPASS = G::NPASS;
  static_assert(RG <= 64, "wave 0 holds one row per lane");
  static_assert(D >= 3, "the ring needs a stage in use, one landing and one ahead");
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::kBytes];
  __shared__ int nvis[RG];
  __shared__ int ppos[RG];
  __shared__ int sh_nmax;
  __shared__ int sh_nmin;

  uint16_t(*qs)[kPitch] = reinterpret_cast<uint16_t(*)[kPitch]>(smem);
  uint32_t(*csq)[kMaxHalfRotary] = reinterpret_cast<uint32_t(*)[kMaxHalfRotary]>(smem + G::kQBytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Task order: the splits of a row group take interleaved tiles, so at any
  // moment they write neighbouring 256-byte pieces of the same score rows;
  // consecutive tasks (the splits of one row group) are kept on one XCD (the
  // hardware deals consecutive workgroups round-robin over 8 XCDs), so those
  // pieces meet in one L2 and leave it as whole lines and pages.
  int64_t task = blockIdx.x;
  {
    const int64_t per = a.tasks >> 3;
    if (task < (per << 3)) task = (task & 7) * per + (task >> 3);
  }
  const int64_t rg = task / a.splits;
  const int64_t split = task - rg * a.splits;
  const int64_t row0 = rg * RG;
  const int blk_begin = static_cast<int>(split) * TILE;
  const int stride = static_cast<int>(a.splits) * TILE;

  const int m = wave % WM;
  const int ng = wave / WM;
  const int khalf = 8 * (lane >> 5);
  bf16x8_t afrag[MS][8];
  if constexpr (PREP) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      int64_t rr = row0 + ((32 * (MS * m + ms) + (lane & 31)) >> 2);
      rr = rr < a.rows ? rr : a.rows - 1;  // rows past the end are never stored
      const uint16_t* src = a.qhat + rr * (kHeads * kHeadDim) + kHeadDim * (lane & 3) + khalf;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        afrag[ms][ks] = *reinterpret_cast<const bf16x8_t*>(src + 16 * ks);
    }
  }
  const int hv_local = tid >> 4;
  const int g = tid & 15;
  uint4 xq[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int hv = p * 16 + hv_local;
    const int64_t r = row0 + (hv >> 2);
    xq[p] = make_uint4(0u, 0u, 0u, 0u);
    if (!PREP && r < a.rows) {
      const uint16_t* src = a.q + r * a.q_stride + kHeadDim * (hv & 3) + 8 * g;
      if (a.q_vec) {
        xq[p] = *reinterpret_cast<const uint4*>(src);
      } else {
        xq[p].x = src[0] | (static_cast<uint32_t>(src[1]) << 16);
        xq[p].y = src[2] | (static_cast<uint32_t>(src[3]) << 16);
        xq[p].z = src[4] | (static_cast<uint32_t>(src[5]) << 16);
        xq[p].w = src[6] | (static_cast<uint32_t>(src[7]) << 16);
      }
    }
  }
  float wv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wv[e] = PREP ? 0.0f : bf16_to_f32(a.w[8 * g + e]);

  // ---- key ring loads.  Wave w loads rows [4 (w kL + i), +4) of a tile, i < kL:
  // lane L of load i fills LDS bytes 1024 (w kL + i) + 16 L, i.e. row
  // 4 (w kL + i) + L / 16 at chunk L % 16, which holds the key's chunk
  // (L % 16) ^ (row & 7).  Block indices are clamped to `last`, so loads
  // never leave the pooled buffer and every step issues the same number of
  // loads.
  constexpr int kL = G::kLoads;
  const int lrow = lane >> 4;
  const int lchunk = lane & 15;
  auto load_tile = [&](int nb0, int stage, int last) {
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int row = 4 * (wave * kL + i) + lrow;
      const int blk = min(nb0 + row, last);
      const uint16_t* src = a.pooled + static_cast<int64_t>(blk) * kHeadDim + 8 * (lchunk ^ (row & 7));
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       static_cast<void*>(smem + stage * G::kStageBytes + 1024 * (wave * kL + i)),
                                       16, 0, 0);
    }
  };

  // ---- positions and visible block counts (wave 0).  With prepared queries
  // the LDS is free from the start, so the first D - 1 tiles are requested
  // right behind the positions, clamped to the pooled buffer's last block
  // instead of the batch's last visible one: the two latencies overlap.  A
  // tile row past every row's prefix feeds only scores that are never stored.
  const int nb_cap = static_cast<int>(a.tokens / kRatio);
  int prow = 0;       // this lane's row position (wave 0)
  int64_t live = 0;   // the live cache length it must lie below
  if (wave == 0 && lane < RG && row0 + lane < a.rows) {
    prow = a.pos[row0 + lane];
    live = live_tokens(a.tokens, a.dev_tokens, a.status);
  }
  if constexpr (PREP) {
    if (nb_cap > 0)  // uniform
#pragma unroll
      for (int t = 0; t < D - 1; ++t) load_tile(blk_begin + t * stride, t, nb_cap - 1);
  }
  if (wave == 0) {
    int n = 0, nlo = 0x7FFFFFFF;
    if (lane < RG) {
      const int64_t r = row0 + lane;
      if (r < a.rows) {
        if (prow >= 0 && prow < live)
          n = (prow + 1) / kRatio;
        else if (split == 0)
          atomicOr(a.status, 1);
      }
      nvis[lane] = n;
      ppos[lane] = prow;
      nlo = n;
    }
    const uint32_t mx = wave_max_u32(static_cast<uint32_t>(n));
    const uint32_t mn = wave_min_u32(static_cast<uint32_t>(nlo));
    if (lane == 0) {
      sh_nmax = static_cast<int>(mx);
      sh_nmin = static_cast<int>(mn);
    }
  }
  __syncthreads();
  const int nmax = sh_nmax;
  const int nmin = sh_nmin;  // blocks every row of the workgroup sees
  if (blk_begin >= nmax) {  // uniform across the workgroup
    if constexpr (PREP) wait_vmcnt<0>();  // no load into LDS outlives the workgroup
    return;
  }
  const int blk_end = nmax;

  if constexpr (!PREP) {
  // ---- cos/sin of every (row, frequency), four per thread in flight
  const int rd = a.rp.rotary_dim;
  const int half = rd >> 1;
  const int ncs = RG * half;
  for (int base = 0; base < ncs; base += 4 * kScoreThreads) {
    uint32_t cs[4];
    int ri[4], fi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int idx = base + u * kScoreThreads + tid;
      idx = idx < ncs ? idx : ncs - 1;
      ri[u] = idx / half;
      fi[u] = idx - ri[u] * half;
      cs[u] = rope_cos_sin_bf16x2(ppos[ri[u]], a.rp.inv_freq[fi[u]]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + u * kScoreThreads + tid < ncs) csq[ri[u]][fi[u]] = cs[u];
  }

  // ---- (1 + w) RMSNorm of every head vector this group holds
  float y[NPASS][8];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int lr = (p * 16 + hv_local) >> 2;
    float x[8];
    unpack_bf16x8(xq[p], x);
    if (!(ppos[lr] >= 0 && ppos[lr] < live_tokens(a.tokens, a.dev_tokens, nullptr))) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += static_cast<double>(x[e]) * static_cast<double>(x[e]);
    const double rinv = inv_rms(row16_sum(ss), a.rp.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[p][e] = norm_channel(x[e], rinv, wv[e]);
  }
  __syncthreads();  // cos/sin table complete
  // ---- RoPE at the row's position.  The group's own row of qs is the
  // exchange buffer: normed values go in, partners are read back, the roped
  // values replace them.  A group lives in one wave, so wave-level ordering
  // of LDS traffic is enough here.
#pragma unroll
  for (int p = 0; p < NPASS; ++p)
    *reinterpret_cast<uint4*>(&qs[p * 16 + hv_local][8 * g]) = pack_bf16x8(y[p]);
  wave_lds_sync();
  uint4 outq[NPASS];
  const bool fast = (half & 7) == 0;  // chunks of 8 never straddle the halves
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int hv = p * 16 + hv_local;
    const int lr = hv >> 2;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = y[p][e];
    if (fast) {
      const int c0 = 8 * g;
      if (c0 < rd) {
        const bool first = c0 < half;
        float xp[8];
        unpack_bf16x8(*reinterpret_cast<const uint4*>(&qs[hv][first ? c0 + half : c0 - half]), xp);
        const int f0 = first ? c0 : c0 - half;
        const uint4 cs0 = *reinterpret_cast<const uint4*>(&csq[lr][f0]);
        const uint4 cs1 = *reinterpret_cast<const uint4*>(&csq[lr][f0 + 4]);
        const uint32_t cs[8] = {cs0.x, cs0.y, cs0.z, cs0.w, cs1.x, cs1.y, cs1.z, cs1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = rope_channel(y[p][e], xp[e], bf16_to_f32(cs[e] & 0xFFFFu), bf16_to_f32(cs[e] >> 16), first);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * g + e;
        if (c < rd) {
          const bool first = c < half;
          const float xp = bf16_to_f32(qs[hv][first ? c + half : c - half]);
          const uint32_t cs = csq[lr][first ? c : c - half];
          o[e] = rope_channel(y[p][e], xp, bf16_to_f32(cs & 0xFFFFu), bf16_to_f32(cs >> 16), first);
        }
      }
    }
    outq[p] = pack_bf16x8(o);
  }
  wave_lds_sync();
#pragma unroll
  for (int p = 0; p < NPASS; ++p) *reinterpret_cast<uint4*>(&qs[p * 16 + hv_local][8 * g]) = outq[p];
  __syncthreads();

  // ---- A fragments: this wave's MS x 32 M-rows (8 query rows x 4 heads each), K = 128.
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      afrag[ms][ks] = *reinterpret_cast<const bf16x8_t*>(
          &qs[32 * (MS * m + ms) + (lane & 31)][16 * ks + khalf]);
  __syncthreads();  // every wave holds its A fragments: the LDS becomes the key ring
  }

  // ---- the first D - 1 tiles (after the prologue, whose LDS they reuse)
  if constexpr (!PREP) {
#pragma unroll
    for (int t = 0; t < D - 1; ++t) load_tile(blk_begin + t * stride, t, blk_end - 1);
  }

  // per-lane output rows: subtile ms holds rows 8 (MS m + ms) + 2 q4 + (lane >> 5).
  // With BUFST the stores go through a buffer resource over the workgroup's
  // rows, the lane's row and column in the vector offset and the step's first
  // block in the scalar offset.  In a step that reaches past some row's
  // prefix, a lane whose block is past its row's prefix gets an offset beyond
  // the resource's end and the hardware drops that store.
  const int col = ng * 32 + (lane & 31);
  float* orow[MS][4];
  int ovis[MS][4];
  int ooff[MS][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int lr = 8 * (MS * m + ms) + 2 * q4 + (lane >> 5);
      orow[ms][q4] = a.scores + (row0 + lr) * a.score_cols;
      ovis[ms][q4] = nvis[lr];
      ooff[ms][q4] = (lr * static_cast<int>(a.score_cols) + col) * 4;
    }
  __amdgpu_buffer_rsrc_t out_rsrc;
  if constexpr (BUFST)
    out_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.scores + row0 * a.score_cols, static_cast<short>(0),
                                                 static_cast<int>(RG * a.score_cols * 4), 0x00020000);
  // B-fragment address of this lane in a stage: row `col`, chunk 2 ks + (lane >> 5), swizzled.
  const int brow = col * 256;
  const int bsw = col & 7;

  // tile 0 landed (the D - 2 later tiles may still be in flight)
  wait_vmcnt<(D - 2) * kL>();
  __builtin_amdgcn_s_barrier();

  // ---- block loop: step t loads tile t + D - 1, runs tile t's MFMAs and
  // stores its scores, then waits for tile t + 1.  Counting what this wave
  // issued after tile t + 1's loads gives at least (D - 2) loads and one
  // step's stores in every step, so vmcnt((D - 2) kL + kStores) retires them.
  int stage = 0;
  for (int nb0 = blk_begin; nb0 < blk_end; nb0 += stride) {
    int lstage = stage + D - 1;
    lstage = lstage >= D ? lstage - D : lstage;
    load_tile(nb0 + (D - 1) * stride, lstage, blk_end - 1);
    const unsigned char* sb = smem + stage * G::kStageBytes + brow;
    f32x16_t acc[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ms][v] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t b =
          *reinterpret_cast<const bf16x8_t*>(sb + 16 * ((2 * ks + (lane >> 5)) ^ bsw));
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        acc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ms][ks], b, acc[ms], 0, 0, 0);
    }
    // relu -> head sum -> scale through the doubled terms (score_fast); a
    // non-finite result, rare, is recomputed exactly.
    float sc[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      uint32_t top = 0u;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        sc[ms][q4] = score_fast(acc[ms][4 * q4 + 0], acc[ms][4 * q4 + 1], acc[ms][4 * q4 + 2],
                                acc[ms][4 * q4 + 3]);
        top = max(top, __float_as_uint(sc[ms][q4]));
      }
      if (top >= 0x7F800000u) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          sc[ms][q4] = score_exact(acc[ms][4 * q4 + 0], acc[ms][4 * q4 + 1], acc[ms][4 * q4 + 2],
                                   acc[ms][4 * q4 + 3]);
      }
    }
    const int blk = nb0 + col;
    if (nb0 + TILE <= nmin) {  // every lane's block is inside its row's prefix
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if constexpr (BUFST) {
            // non-temporal: the score stream is written once and read back once
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc[ms][q4]), out_rsrc, ooff[ms][q4],
                                                  4 * nb0, kStoreNT);
          } else {
            orow[ms][q4][blk] = sc[ms][q4];
          }
        }
    } else {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if constexpr (BUFST) {
            const int off = blk < ovis[ms][q4] ? ooff[ms][q4] : static_cast<int>(0x80000000u);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc[ms][q4]), out_rsrc, off, 4 * nb0,
                                                  kStoreNT);
          } else {
            if (blk < ovis[ms][q4]) orow[ms][q4][blk] = sc[ms][q4];
          }
        }
    }
    wait_lgkm0();
    if constexpr (BUFST)
      wait_vmcnt<(D - 2) * kL + G::kStores>();
    else
      wait_vmcnt<0>();  // branchy stores: their count per step is not fixed
    __builtin_amdgcn_s_barrier();
    stage = stage + 1 == D ? 0 : stage + 1;
  }
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup
}


// ---------------------------------------------------------------------------
// Ring scorer for prepared queries.
//
// WM waves along M, each holding 32 query rows as four 32 x 128 A-fragment
// sets (MS = 4) for the whole block loop: 32 WM rows per workgroup.  The
// other 4 / WM wave columns split each step's tile of 32 (4 / WM) blocks,
// 32 blocks per wave.  Prefill batches take WM = 4 (128 rows, 32-block
// tiles).  The pooled keys stream through a D-stage LDS ring
// filled by buffer loads straight to LDS (blocks at or past the workgroup's
// longest prefix read as zeros and are never stored); every wave reads its
// eight B fragments of a step once and feeds each to four MFMAs.
//
// Two details keep the ring pipelined.  The B-fragment reads are inline
// assembly: a compiler-visible LDS read behind an in-flight load to LDS makes
// the compiler drain every outstanding memory operation first, scores
// included.  And each step waits with vmcnt for exactly the next tile's
// loads: a wave's loads and score stores retire in issue order, and the
// stores issued since that tile's loads are counted (at most 63).
//
// Epilogue: phase A stores the previous step's acc[2..3] scores before
// acc[0..1]'s MFMAs; phase B stores acc[0..1]'s, threaded between
// acc[2..3]'s MFMAs on interior tiles, so relu / head sum / scale of one
// pair overlaps the other pair's MFMAs.
// ---------------------------------------------------------------------------

template <int WM>
struct RingGeom {
  static constexpr int WN = 4 / WM;
  static constexpr int RG = 32 * WM;          // query rows per workgroup
  static constexpr int TILE = 32 * WN;        // blocks per step
  static constexpr int STAGE = TILE * 256;    // bytes per ring stage
  static constexpr int kL = STAGE / 4096;     // 1 KiB ring loads per wave per tile
  static constexpr int kStores = 16;          // score stores per wave per step
  static constexpr int D = WM == 4 ? 4 : 3;   // ring stages
};

struct RingArgs {
  const uint16_t* qhat;
  const int32_t* pos;
  int64_t rows;
  const uint16_t* pooled;
  int64_t tokens;             // the ceiling when dev_tokens is set
  const int32_t* dev_tokens;  // optional live cache length on the device
  int bstride;  // column j scores the pooled key of block j * bstride
  float* scores;
  int64_t score_cols;
  int32_t* status;              // may be null: bad positions are then not flagged
  const int32_t* group_flag;    // non-null: only row groups with a nonzero flag run
  const uint32_t* thr;          // EMIT: per-row thresholds (score bits), 128-row padded
  uint2* cand;                  // EMIT: [rows][splits][4][cap] (score bits, block)
  int32_t* cnt;                 // EMIT: [rows][splits][4] blocks at or above the threshold
  int cap;
  int splits;  // workgroups per row group; split s takes tiles s, s + splits, ...
  int tasks;
};

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}
// One 16-byte LDS read as inline assembly (see above); the value may only be
// used after lds_wait8.
template <int OFF>
__device__ __forceinline__ bf16x8_t lds_read16(uint32_t addr) {
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
  return v;
}
// Waits for this wave's LDS reads; the fragments become usable after it.
__device__ __forceinline__ void lds_wait8(bf16x8_t (&b)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7])
               :
               : "memory");
}
// One LDS word read and its wait, as inline assembly.
__device__ __forceinline__ int lds_read_word(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// In-register transpose of one emit phase.  On entry slot s (0..7) of lane
// (r, h) = lane % 32, lane / 32 holds phase row 2 s + h at tile block r.
// Three exchanges trade the slot index bits s2, s1, s0 for the lane bits 4,
// 1, 0: a permlane16 swap (lane bit 4), then quad permutations taken by the
// lanes whose bit is set (lane bits 1 and 0).  On exit lane l holds, in slot
// j, phase row 8 l[4] + 4 l[1] + 2 l[0] + l[5] at tile block
// 16 j[2] + 4 ((l >> 2) & 3) + (j & 3).
__device__ __forceinline__ void emit_transpose(uint32_t (&v)[8], int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const auto p = __builtin_amdgcn_permlane16_swap(v[s], v[s + 4], false, false);
    v[s] = p[0];
    v[s + 4] = p[1];
  }
  const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = (k & 1) + 4 * (k >> 1);  // 0, 1, 4, 5: partners s + 2
    const uint32_t pa = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v[s]), 0x4E, 0xF, 0xF, false));
    const uint32_t pb = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v[s + 2]), 0x4E, 0xF, 0xF, false));
    const uint32_t na = b1 ? pb : v[s];
    const uint32_t nb = b1 ? v[s + 2] : pa;
    v[s] = na;
    v[s + 2] = nb;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = 2 * k;  // partners s + 1
    const uint32_t pa = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v[s]), 0xB1, 0xF, 0xF, false));
    const uint32_t pb = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v[s + 1]), 0xB1, 0xF, 0xF, false));
    const uint32_t na = b0 ? pb : v[s];
    const uint32_t nb = b0 ? v[s + 1] : pa;
    v[s] = na;
    v[s + 1] = nb;
  }
}

// EMIT: instead of storing the scores, the kernel keeps the blocks whose
// score, read as an unsigned integer, is at least the row's threshold
// thr[row] (score bits).  Scores are +-0 or positive or NaN: for finite
// thresholds this is their order (a -0.0 score, from an all -0.0 head set,
// reads as large and is kept, which only adds a candidate), and NaN / +Inf
// bits lie above every threshold up to +Inf: non-finite scores are always
// kept, for the selector to refuse.  Each epilogue phase (16 rows x 32
// blocks of a wave) is transposed in registers (emit_transpose) so that each
// lane owns one row of the phase and eight blocks of the tile: its threshold
// and its running count stay in the lane, and a kept block is one compare and
// one store, with no cross-lane work.  Kept blocks go to the region of (row,
// split, block group), cap entries of (score bits, block); the counts, which
// may exceed cap (the excess overwrote the region's last entry), finally go
// to cnt[row][split][block group].
template <int WM, bool EMIT>
__global__ __launch_bounds__(256, 2) void score_ring_kernel(const RingArgs a) {
  using G = RingGeom<WM>;
  constexpr int RG = G::RG, TILE = G::TILE, STAGE = G::STAGE, kL = G::kL, kStores = G::kStores, D = G::D;
  static_assert(!EMIT || WM == 4, "emission assumes 32 rows per wave, 32 blocks per step");
  __shared__ __attribute__((aligned(16))) unsigned char ring[D * STAGE];
  __shared__ int nvis[RG];
  __shared__ int sh_nmax, sh_nmin;
  __shared__ uint32_t sthr[EMIT ? RG : 1];  // EMIT: per-row thresholds

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = wave % WM;   // 32-row slice of the group
  const int ng = wave / WM;  // 32-block slice of the tile
  // The splits of one row group share an XCD (the hardware deals workgroups
  // round-robin over 8 XCDs: XCD b % 8 takes workgroups b, b + 8, ...), so
  // their neighbouring pieces of the same score rows meet in one L2.  With a
  // multiple of 8 row groups, XCD x's j-th workgroup is split j % splits of
  // its share's entry j / splits (xcd_share_group: shares of equal length on
  // causal batches; 8192 prefill rows over 64k: 138.3 -> 134.9 us, the step
  // 322.5 -> 316.4 us in one A/B); otherwise
  // each XCD takes a contiguous eighth of the tasks.
  int rg, split;
  {
    const int groups = a.tasks / a.splits;
    if ((groups & 7) == 0) {
      const int j = static_cast<int>(blockIdx.x >> 3);
      const int k = j / a.splits;
      split = j - k * a.splits;
      rg = xcd_share_group(static_cast<int>(blockIdx.x & 7), k, groups);
    } else {
      int task = blockIdx.x;
      const int per = a.tasks >> 3;
      if (task < (per << 3)) task = (task & 7) * per + (task >> 3);
      rg = task / a.splits;
      split = task - rg * a.splits;
    }
  }
  if (a.group_flag != nullptr && a.group_flag[rg] == 0) return;  // uniform
  const int64_t row0 = static_cast<int64_t>(rg) * RG;
  const int blk_begin = split * TILE;
  const int stride = a.splits * TILE;

  // EMIT: after emit_transpose lane l's rows are 32 m + er (phase of
  // acc[0..1]) and 32 m + 16 + er (acc[2..3]), its blocks of a tile
  // 4 cg + {0, 1, 2, 3, 16, 17, 18, 19}
  const int er = 8 * ((lane >> 4) & 1) + 4 * ((lane >> 1) & 1) + 2 * (lane & 1) + (lane >> 5);
  const int cg = (lane >> 2) & 3;
  uint32_t ecnt0 = 0u, ecnt1 = 0u;

  auto store_counts = [&]() {
    const int64_t r0 = row0 + 32 * m + er, r1 = r0 + 16;
    if (r0 < a.rows) a.cnt[(r0 * a.splits + split) * 4 + cg] = static_cast<int32_t>(ecnt0);
    if (r1 < a.rows) a.cnt[(r1 * a.splits + split) * 4 + cg] = static_cast<int32_t>(ecnt1);
  };

  // A fragments: subtile ms = rows 32 m + 8 ms .. + 7 as 32 M-rows (row, head)
  bf16x8_t afrag[4][8];
  {
    const int khalf = 8 * (lane >> 5);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      int64_t rr = row0 + 32 * m + 8 * ms + ((lane & 31) >> 2);
      rr = rr < a.rows ? rr : a.rows - 1;  // rows past the end are never stored
      const uint16_t* src = a.qhat + rr * (kHeads * kHeadDim) + kHeadDim * (lane & 3) + khalf;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) afrag[ms][ks] = *reinterpret_cast<const bf16x8_t*>(src + 16 * ks);
    }
  }
  // visible columns (wave 0, lane l: rows l and l + 64): blocks (p + 1) / 4,
  // of which every bstride-th is a column
  if constexpr (EMIT)
    if (tid < RG) sthr[tid] = a.thr[row0 + tid];
  if (wave == 0) {
    uint32_t mx = 0u, mn = 0x7FFFFFFFu;
#pragma unroll
    for (int hh = 0; hh < (RG + 63) / 64; ++hh) {
      const int lr = lane + 64 * hh;
      if (lr < RG) {
        int n = 0;
        const int64_t r = row0 + lr;
        if (r < a.rows) {
          const int p = a.pos[r];
          if (p >= 0 && p < live_tokens(a.tokens, a.dev_tokens, a.status))
            n = ((p + 1) / kRatio + a.bstride - 1) / a.bstride;
          else if (split == 0 && a.status != nullptr)
            atomicOr(a.status, 1);
        }
        nvis[lr] = n;
        mx = max(mx, static_cast<uint32_t>(n));
        mn = min(mn, static_cast<uint32_t>(n));
      }
    }
    mx = wave_max_u32(mx);
    mn = wave_min_u32(mn);
    if (lane == 0) {
      sh_nmax = static_cast<int>(mx);
      sh_nmin = static_cast<int>(mn);
    }
  }
  __syncthreads();
  const int nmax = sh_nmax;
  const int nmin = sh_nmin;  // columns every row of the workgroup sees
  if (blk_begin >= nmax) {   // uniform; nothing in flight
    if constexpr (EMIT) store_counts();
    return;
  }

  // ---- key ring.  Load i of wave w fills tile rows 4 (w kL + i) + lane / 16
  // with the key's 16-byte chunk (lane % 16) ^ (row & 7) at chunk lane % 16,
  // so a B-fragment read (32 rows, one chunk each) spreads over all banks.
  const int kbytes = 256 * a.bstride;  // bytes from one column's key to the next
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.pooled), static_cast<short>(0), nmax * kbytes, 0x00020000);
  const int lrow = lane >> 4, lchunk = lane & 15;
  auto load_tile = [&](int nb0, int stage) {
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int row = 4 * (wave * kL + i) + lrow;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krsrc, (__attribute__((address_space(3))) void*)(ring + stage * STAGE + 1024 * (wave * kL + i)), 16,
          row * kbytes + 16 * (lchunk ^ (row & 7)), nb0 * kbytes, 0, 0);
    }
  };
  // B fragment ks of lane (r, h): stage row 32 ng + r, logical chunk 2 ks + h
  // at chunk (2 ks + h) ^ (r & 7) = 2 ((ks & 3) ^ s2) + (h ^ s1) + 8 (ks >> 2).
  const int r = lane & 31, h = lane >> 5;
  const int col = 32 * ng + r;  // the lane's block within the tile
  const int s2 = (r & 7) >> 1, s1 = r & 1;
  const uint32_t bbase = lds_addr(ring) + col * 256 + 16 * (h ^ s1);
  const uint32_t s2x = 32 * s2;
  const uint32_t nvis_lane = lds_addr(nvis) + 4 * (32 * m + h);

  // score stores through a resource over the group's rows: lane (r, h) of
  // subtile ms writes row 32 m + 8 ms + 2 q4 + h, column nb0 + col.  An
  // offset past the resource drops the store (blocks outside a row's prefix).
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      EMIT ? nullptr : a.scores + row0 * a.score_cols, static_cast<short>(0),
      EMIT ? 0 : static_cast<int>(RG * a.score_cols * 4), 0x00020000);
  const int vbase = EMIT ? 0 : ((32 * m + h) * static_cast<int>(a.score_cols) + col) * 4;
  const int rowbytes = EMIT ? 0 : static_cast<int>(a.score_cols) * 4;
  constexpr int kDrop = static_cast<int>(0x80000000u);

  // Fast pass: scores through score_fast, and `seen` (a wave-uniform mask in
  // scalar registers: the ring loop has no vector register to spare) records
  // the lanes that produced a non-finite one; exact pass: score_exact (see
  // the end).
  uint64_t seen = 0u;
  // fast_c: every column of the tile is visible to every row of the group
  // (a compile-time choice, so the fast form is straight-line code; a
  // run-time flag left a branch and exec-mask bookkeeping around each store)
  auto store_off = [&](int ms, int q4, int nb0, bool live, auto fast_c) {
    if constexpr (decltype(fast_c)::value) {
      return vbase;
    } else {
      const int nv = lds_read_word(nvis_lane + 4 * (8 * ms + 2 * q4));
      return (live && nb0 + col < nv) ? vbase : kDrop;
    }
  };
  auto phase_score = [&](const f32x16_t& x, int q4, auto exact_c) {
    if constexpr (decltype(exact_c)::value)
      return score_exact(x[4 * q4 + 0], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
    else
      return score_fast(x[4 * q4 + 0], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
  };
  // the largest bits of a phase's eight fast scores into `seen`
  auto note_phase = [&](const float (&sc)[8]) {
    uint32_t t = max(max(__float_as_uint(sc[0]), __float_as_uint(sc[1])), __float_as_uint(sc[2]));
    t = max(max(t, __float_as_uint(sc[3])), __float_as_uint(sc[4]));
    t = max(max(t, __float_as_uint(sc[5])), __float_as_uint(sc[6]));
    t = max(t, __float_as_uint(sc[7]));
    seen |= __builtin_amdgcn_ballot_w64(t >= 0x7F800000u);
  };
  auto pair_store = [&](const f32x16_t& x0, const f32x16_t& x1, int m0, int nb0, bool live, auto fast,
                        auto exact_c) {
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ms = m0 + (j >> 2), q4 = j & 3;
      sc[j] = phase_score(j < 4 ? x0 : x1, q4, exact_c);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc[j]), orsrc, store_off(ms, q4, nb0, live, fast),
                                            (8 * ms + 2 * q4) * rowbytes + 4 * nb0, 0);
    }
    if constexpr (!decltype(exact_c)::value) note_phase(sc);
  };

  // EMIT: regions of the group's rows, [row][split][4][cap]
  const int crow = EMIT ? a.splits * 4 * a.cap * 8 : 0;  // bytes of one row's regions
  const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
      EMIT ? a.cand + row0 * a.splits * 4 * a.cap : nullptr, static_cast<short>(0), RG * crow, 0x00020000);
  const int ebase = EMIT ? (32 * m + er) * crow + (split * 4 + cg) * a.cap * 8 : 0;
  const uint32_t capm1 = EMIT ? static_cast<uint32_t>(a.cap - 1) : 0u;
  auto pair_emit = [&](const f32x16_t& x0, const f32x16_t& x1, auto m0c, int nb0, bool live, bool fast,
                       auto exact_c) {
    constexpr int m0 = decltype(m0c)::value;
    // slot s = 4 (ms - m0) + q4 of lane (r, h): phase row 2 s + h, block r
    float sc[8];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      sc[q4] = phase_score(x0, q4, exact_c);
      sc[4 + q4] = phase_score(x1, q4, exact_c);
    }
    if constexpr (!decltype(exact_c)::value) note_phase(sc);
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __float_as_uint(sc[j]);
    emit_transpose(v, lane);
    const uint32_t t = static_cast<uint32_t>(lds_read_word(lds_addr(sthr) + 4 * (32 * m + 8 * m0 + er)));
    const uint32_t blk0 = static_cast<uint32_t>(nb0 + 4 * cg);
    uint32_t& cnt = m0 == 0 ? ecnt0 : ecnt1;
    const int soff = m0 == 0 ? 0 : 16 * crow;
    // each path issues exactly 8 stores (the ring's vmcnt accounting)
    auto emit8 = [&](auto visc) {
      uint32_t nv = 0u;
      if constexpr (decltype(visc)::value) nv = static_cast<uint32_t>(lds_read_word(lds_addr(nvis) + 4 * (32 * m + 8 * m0 + er)));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t blk = blk0 + 16 * (j >> 2) + (j & 3);
        bool c = v[j] >= t;
        if constexpr (decltype(visc)::value) c = c & live & (blk < nv);
        const uint32_t slot = cnt < capm1 ? cnt : capm1;  // past capacity: the row falls back
        const int voff = c ? ebase + 8 * static_cast<int>(slot) : kDrop;
        __attribute__((ext_vector_type(2))) uint32_t e = {v[j], blk};
        __builtin_amdgcn_raw_buffer_store_b64(e, crsrc, voff, soff, 0);
        cnt += c ? 1u : 0u;
      }
    };
    if (fast)  // every block of the tile visible to every row of the group
      emit8(std::integral_constant<bool, false>{});
    else
      emit8(std::integral_constant<bool, true>{});
  };
  auto epilogue = [&](const f32x16_t& x0, const f32x16_t& x1, auto m0c, int nb0, bool live, bool fast,
                      auto exact_c) {
    if constexpr (EMIT) {
      pair_emit(x0, x1, m0c, nb0, live, fast, exact_c);
    } else {
      if (fast)
        pair_store(x0, x1, decltype(m0c)::value, nb0, live, std::true_type{}, exact_c);
      else
        pair_store(x0, x1, decltype(m0c)::value, nb0, live, std::false_type{}, exact_c);
    }
  };

#pragma unroll
  for (int t = 0; t < D - 1; ++t) load_tile(blk_begin + t * stride, t);
  f32x16_t acc[4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ms][v] = 0.0f;

  wait_vmcnt<(D - 2) * kL>();  // tile 0 landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  int stage = 0, step = 0;
  int prev_nb0 = blk_begin;
  for (int nb0 = blk_begin; nb0 < nmax; nb0 += stride) {
    int lstage = stage + D - 1;
    lstage = lstage >= D ? lstage - D : lstage;
    load_tile(nb0 + (D - 1) * stride, lstage);
    bf16x8_t bf[8];
    {
      const uint32_t bb = bbase + stage * STAGE;
      const uint32_t b0 = bb + s2x, b1 = bb + (32u ^ s2x), b2 = bb + (64u ^ s2x), b3 = bb + (96u ^ s2x);
      bf[0] = lds_read16<0>(b0);
      bf[1] = lds_read16<0>(b1);
      bf[2] = lds_read16<0>(b2);
      bf[3] = lds_read16<0>(b3);
      bf[4] = lds_read16<128>(b0);
      bf[5] = lds_read16<128>(b1);
      bf[6] = lds_read16<128>(b2);
      bf[7] = lds_read16<128>(b3);
    }
    // phase A: the previous step's acc[2..3] (dropped in the first step)
    epilogue(acc[2], acc[3], std::integral_constant<int, 2>{}, prev_nb0, step > 0, step > 0 && prev_nb0 + TILE <= nmin,
             std::false_type{});
    lds_wait8(bf);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[0][ks], bf[ks], ks ? acc[0] : f32x16_t{}, 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[1][ks], bf[ks], ks ? acc[1] : f32x16_t{}, 0, 0, 0);
    }
    // phase B: this step's acc[0..1]
    // Interior tile: acc[0..1]'s score math and stores are threaded between
    // acc[2..3]'s MFMAs (one MFMA, six VALU, a store every second MFMA), so a
    // wave issues its own epilogue while its matrix pipe is busy; left to
    // itself the compiler issued all 32 MFMAs first.  8192 prefill rows over
    // 64k: 133.8 -> 128.1 and 129.0 -> 123.9 us in one-process A/Bs on two
    // boxes, scores bit-identical.
    if (!EMIT && nb0 + TILE <= nmin) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[2][ks], bf[ks], ks ? acc[2] : f32x16_t{}, 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[3][ks], bf[ks], ks ? acc[3] : f32x16_t{}, 0, 0, 0);
      }
      pair_store(acc[0], acc[1], 0, nb0, true, std::true_type{}, std::false_type{});
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
        if (i & 1) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);  // a store every second MFMA
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[2][ks], bf[ks], ks ? acc[2] : f32x16_t{}, 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[3][ks], bf[ks], ks ? acc[3] : f32x16_t{}, 0, 0, 0);
      }
      epilogue(acc[0], acc[1], std::integral_constant<int, 0>{}, nb0, true, nb0 + TILE <= nmin, std::false_type{});
    }
    // Tile t + 1 has landed once at most N of this wave's memory operations
    // are outstanding, N = what was issued after its loads: the loads of
    // (D - 2) tiles and the stores of each step since (D - 1 steps in the
    // steady state, step + 1 in the first D - 2 steps).  Smaller N is safe.
    // Both epilogues issue kStores stores per step, whatever they keep.
    {
      constexpr int NA0 = (D - 2) * kL + (D - 1) * kStores;
      constexpr int NA = NA0 > 63 ? 63 : NA0;
      constexpr int N0 = (D - 2) * kL + kStores;
      constexpr int N1 = (D - 2) * kL + 2 * kStores;
      constexpr int N2 = (D - 2) * kL + 3 * kStores;
      static_assert(D <= 5, "steps before the steady state: at most three");
      if (step >= D - 2) wait_vmcnt<NA>();
      else if (step == 0) wait_vmcnt<(N0 > 63 ? 63 : N0)>();
      else if (step == 1) wait_vmcnt<(N1 > 63 ? 63 : N1)>();
      else wait_vmcnt<(N2 > 63 ? 63 : N2)>();
    }
    __builtin_amdgcn_s_barrier();  // the stage read this step may be refilled
    asm volatile("" ::: "memory");
    prev_nb0 = nb0;
    ++step;
    stage = stage + 1 == D ? 0 : stage + 1;
  }
  epilogue(acc[2], acc[3], std::integral_constant<int, 2>{}, prev_nb0, true, prev_nb0 + TILE <= nmin, std::false_type{});
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup

  // score_fast equals score_exact wherever it is finite.  If any lane of the
  // workgroup produced a non-finite score (rare: NaN or infinite inputs, or
  // a head dot beyond half the f32 range), the workgroup scores its tiles
  // again with score_exact, overwriting every score (or re-emitting every
  // candidate) it wrote.  This pass loads its B fragments straight from
  // memory, without the ring.
  if (__syncthreads_or(seen != 0u ? 1 : 0)) {
    ecnt0 = 0u;
    ecnt1 = 0u;
    // lane values recomputed here, so that none of them stays live across
    // the ring loop above
    int t2 = threadIdx.x;
    asm volatile("" : "+v"(t2));
    const int col2 = 32 * ((t2 >> 6) / WM) + (t2 & 31), h2 = (t2 & 63) >> 5;
    for (int nb0 = blk_begin; nb0 < nmax; nb0 += stride) {
      const int c = min(nb0 + col2, nmax - 1);  // columns past nmax are never stored
      const uint16_t* krow = a.pooled + static_cast<int64_t>(c) * a.bstride * kHeadDim + 8 * h2;
      bf16x8_t bf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) bf[ks] = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ks);
      f32x16_t x[4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        x[ms] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) x[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ms][ks], bf[ks], x[ms], 0, 0, 0);
      }
      const bool fast = nb0 + TILE <= nmin;
      epilogue(x[0], x[1], std::integral_constant<int, 0>{}, nb0, true, fast, std::true_type{});
      epilogue(x[2], x[3], std::integral_constant<int, 2>{}, nb0, true, fast, std::true_type{});
    }
  }
  if constexpr (EMIT) store_counts();
}

// Workgroups: `target` in all, at least one tile each; a row group's splits
// take interleaved tiles.  When that would leave a workgroup a tile or two
// (short caches), it keeps four (the ring depth) while 256 workgroups
// remain: 4096 rows over 4k tokens score in 14 instead of 24 us.
int64_t ring_splits_for(int64_t row_groups, int64_t cols, int tile, int64_t target) {
  int64_t n_tiles = (cols + tile - 1) / tile;
  if (n_tiles < 1) n_tiles = 1;
  int64_t splits = (target + row_groups - 1) / row_groups;
  const int64_t wide = (256 + row_groups - 1) / row_groups;
  const int64_t deep = n_tiles / 4 > wide ? n_tiles / 4 : wide;
  if (splits > deep) splits = deep;
  if (splits < 1) splits = 1;
  if (splits > n_tiles) splits = n_tiles;
  return splits;
}

template <int WM, bool EMIT>
hipError_t launch_score_ring_geom(RingArgs a, int64_t target, hipStream_t stream) {
  using G = RingGeom<WM>;
  const int64_t nb_total = a.tokens / kRatio;
  const int64_t cols = (nb_total + a.bstride - 1) / a.bstride;
  const int64_t row_groups = (a.rows + G::RG - 1) / G::RG;
  const int64_t splits = ring_splits_for(row_groups, cols, G::TILE, target);
  if (row_groups * splits > 0x7FFFFFFF) return hipErrorInvalidValue;
  a.splits = static_cast<int>(splits);
  a.tasks = static_cast<int>(row_groups * splits);
  score_ring_kernel<WM, EMIT><<<dim3(static_cast<unsigned>(a.tasks)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

// The ring's store resource spans 32 WM rows of scores, within 2^31 bytes.
bool ring_fits(const ScoreArgs& a, int rows_per_group) {
  return a.score_cols <= 0x7FFFFFFF / (4 * rows_per_group);
}

hipError_t launch_score_ring(const ScoreArgs& s, hipStream_t stream) {
  RingArgs a{};
  a.qhat = s.qhat;
  a.pos = s.pos;
  a.rows = s.rows;
  a.pooled = s.pooled;
  a.tokens = s.tokens;
  a.dev_tokens = s.dev_tokens;
  a.bstride = 1;
  a.scores = s.scores;
  a.score_cols = s.score_cols;
  a.status = s.status;
  return launch_score_ring_geom<4, false>(a, 1024, stream);
}

// ---- one decode row: a streaming scorer -----------------------------------
//
// pegainfer pull request 1160 ("score QSA token-indexer blocks in native
// CUDA"), summary: with one row the 4 heads are a sliver of a matrix tile's
// M side, and the row's scoring is bound by the stream of pooled keys itself
// (256 B per block, read once).  Each block is owned by 16 lanes of a wave,
// 8 channels each.  A lane keeps its 8 channels of the 4 prepared heads as
// packed bf16 pairs, forms each head dot product with bf16 pair dots
// accumulated in f32, and the 16 lanes reduce it with DPP; lane 0 of the
// group stores the block's score.  Keys are 16-byte streaming loads,
// kStreamU per lane in flight; no LDS ring.  Without prepared queries the
// workgroup first prepares the row into LDS (prep_body.h), so both entry
// points run the same loop and give the same scores bit for bit.
constexpr int kStreamU = 4;                   // blocks per 16-lane group per step
constexpr int kStreamBlocks = 16 * kStreamU;  // blocks per workgroup step

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Sum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row16_sum_f32(float v) {
#define QSA_ROR_STEP_F(CTRL) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  QSA_ROR_STEP_F(0x128)
  QSA_ROR_STEP_F(0x124)
  QSA_ROR_STEP_F(0x122)
  QSA_ROR_STEP_F(0x121)
#undef QSA_ROR_STEP_F
  return v;
}

template <bool PREP>
__global__ __launch_bounds__(kScoreThreads) void score_stream_kernel(const ScoreArgs a) {
  static_assert(kScoreThreads == kPrepThreads, "the prep body runs on the whole workgroup");
  __shared__ __attribute__((aligned(16))) uint16_t qs[PREP ? 8 : kPrepRows * kHeads * kHeadDim];
  const int tid = threadIdx.x;
  const int grp = tid >> 4;  // block slot of this lane's 16-lane group
  const int g = tid & 15;    // channels 8g .. 8g + 7
  if constexpr (!PREP) {
    PrepArgs pa{};
    pa.q = a.q;
    pa.q_stride = a.q_stride;
    pa.pos = a.pos;
    pa.rows = 1;
    pa.w = a.w;
    pa.tokens = a.tokens;
    pa.dev_tokens = a.dev_tokens;
    pa.qhat = qs;
    pa.status = a.status;
    pa.q_vec = a.q_vec;
    pa.rp = a.rp;
    prep_group(pa, 0);
    __syncthreads();
  }
  const uint16_t* qsrc = PREP ? a.qhat : qs;

  // The workgroup's first keys are requested before the row's position
  // arrives, clamped to the pooled buffer -- or, with a device cache length,
  // to its live blocks -- and the visible count only gates the stores.
  const int64_t live = live_tokens(a.tokens, a.dev_tokens, a.status);
  const int64_t nb_cap = live / kRatio;
  typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
  u32x4_nt kv[kStreamU];
  auto load_keys = [&](int64_t b0) {
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const int64_t b = b0 + grp + 16 * u;
      const int64_t bc = b < nb_cap ? b : nb_cap - 1;
      kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(a.pooled + bc * kHeadDim + 8 * g));
    }
  };
  int64_t b0 = static_cast<int64_t>(blockIdx.x) * kStreamBlocks;
  if (b0 < nb_cap) load_keys(b0);  // uniform

  // this lane's channels of the 4 heads (also requested ahead of the position)
  uint32_t qv[kHeads][4];
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(qsrc + h * kHeadDim + 8 * g);
    qv[h][0] = v.x;
    qv[h][1] = v.y;
    qv[h][2] = v.z;
    qv[h][3] = v.w;
  }
  // the row's visible block count (uniform across the workgroup)
  const int p = a.pos[0];
  int n = 0;
  if (p >= 0 && p < live)
    n = (p + 1) / kRatio;
  else if (blockIdx.x == 0 && tid == 0)
    atomicOr(a.status, 1);

  // n <= nb_cap, so a workgroup that skipped its loads never enters
  while (b0 < n) {
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const int64_t b = b0 + grp + 16 * u;
      float d[kHeads];
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        float acc = dot2_bf16(qv[h][0], kv[u][0], 0.0f);
        acc = dot2_bf16(qv[h][1], kv[u][1], acc);
        acc = dot2_bf16(qv[h][2], kv[u][2], acc);
        acc = dot2_bf16(qv[h][3], kv[u][3], acc);
        d[h] = row16_sum_f32(acc);
      }
      if (g == 0 && b < n) {
        float sc = score_fast(d[0], d[1], d[2], d[3]);
        if (!(__float_as_uint(sc) < 0x7F800000u)) sc = score_exact(d[0], d[1], d[2], d[3]);
        a.scores[b] = sc;
      }
    }
    b0 += static_cast<int64_t>(gridDim.x) * kStreamBlocks;
    if (b0 < n) load_keys(b0);
  }
}

template <bool PREP>
hipError_t launch_score_stream(const ScoreArgs& a, hipStream_t stream) {
  const int64_t nb = a.tokens / kRatio;
  int64_t grid = (nb + kStreamBlocks - 1) / kStreamBlocks;
  grid = grid < 1 ? 1 : (grid > 4096 ? 4096 : grid);  // one workgroup still flags bad positions
  const dim3 g(static_cast<unsigned>(grid)), b(kScoreThreads);
  score_stream_kernel<PREP><<<g, b, 0, stream>>>(a);
  return hipGetLastError();
}

template <int WM, int MS, int D, bool PREP>
hipError_t launch_score_geom(const ScoreArgs& base, hipStream_t stream) {
  using G = ScoreGeom<WM, MS, D, PREP>;
  ScoreArgs a = base;
  const int64_t nb_total = a.tokens / kRatio;
  a.row_groups = (a.rows + G::RG - 1) / G::RG;
  // At least one tile: a workgroup per row group still runs, to flag rows
  // whose position is out of range even when no block is complete.
  int64_t n_tiles = (nb_total + G::TILE - 1) / G::TILE;
  if (n_tiles < 1) n_tiles = 1;
  // About 1024 workgroups in all; but when few row groups would leave each
  // workgroup a tile or two, keep at least D tiles per workgroup (the ring
  // then overlaps its loads) as long as 256 workgroups remain.
  int64_t splits = (1024 + a.row_groups - 1) / a.row_groups;
  const int64_t deep = n_tiles / D > (256 + a.row_groups - 1) / a.row_groups
                           ? n_tiles / D
                           : (256 + a.row_groups - 1) / a.row_groups;
  if (splits > deep) splits = deep;
  if (splits < 1) splits = 1;
  if (splits > n_tiles) splits = n_tiles;
  a.splits = splits;
  a.tasks = a.row_groups * splits;
  if (a.tasks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.tasks));
  const dim3 block(kScoreThreads);
  // buffer-resource stores need the workgroup's rows within 2^31 bytes
  if (a.score_cols <= 0x7FFFFFFF / (4 * G::RG))
    score_mfma_kernel<WM, MS, D, true, PREP><<<grid, block, 0, stream>>>(a);
  else
    score_mfma_kernel<WM, MS, D, false, PREP><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool PREP>
hipError_t launch_score_rows(const ScoreArgs& a, hipStream_t stream) {
  // The one-call path keeps 8 rows per wave, which bounds its query-prep LDS.
  // Prepared queries in batches of 128 rows and more: the ring scorer, when
  // its store resource fits.  (Its 1- and 2-wave-row layouts measured slower
  // than the kernels below on decode batches: 32 A-fragment loads and a
  // 96 KiB ring per workgroup outweigh the shared key tiles there.)
  // One row: the streaming scorer (64k: 3.0 us per launch against 4.2 for
  // the padded-M matrix kernel).  From two rows its per-row lane reductions
  // make it VALU-bound (two rows over 256k: 7.3 us against 5.0), and the
  // matrix kernels below take over.
  if (a.rows == 1) return launch_score_stream<PREP>(a, stream);
  if constexpr (PREP)
    if (a.rows >= 128 && ring_fits(a, 128)) return launch_score_ring(a, stream);
  // 64..127 prepared rows: one 64-row group, each wave 16 rows (two
  // subtiles) of a 32-block tile, so no two waves load the same A fragments
  // (64 rows over 64k: 7.9 -> 6.0 us against 32 rows per wave and 64-block
  // tiles, whose waves load every fragment twice).
  if constexpr (PREP)
    if (a.rows >= 64) return launch_score_geom<4, 2, 4, PREP>(a, stream);
  if (a.rows >= 32) return launch_score_geom<4, 1, 4, PREP>(a, stream);
  if (a.rows > 8) return launch_score_geom<2, 1, 4, PREP>(a, stream);
  return launch_score_geom<1, 1, 3, PREP>(a, stream);
}

}  // namespace

int64_t ring_splits(int64_t rows, int64_t cols, int64_t target) {
  return ring_splits_for((rows + kRingRows - 1) / kRingRows, cols, 32, target);
}

hipError_t launch_ring(const RingJob& j, int64_t target, hipStream_t stream) {
  RingArgs a{};
  a.qhat = j.qhat;
  a.pos = j.pos;
  a.rows = j.rows;
  a.pooled = j.pooled;
  a.tokens = j.tokens;
  a.bstride = j.bstride;
  a.scores = j.scores;
  a.score_cols = j.score_cols;
  a.status = j.status;
  a.group_flag = j.group_flag;
  a.thr = j.thr;
  a.cand = j.cand;
  a.cnt = j.cnt;
  a.cap = j.cap;
  if (j.cand != nullptr) return launch_score_ring_geom<4, true>(a, target, stream);
  return launch_score_ring_geom<4, false>(a, target, stream);
}

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
  a.rp = rp;
  return launch_score_rows<false>(a, stream);
}

hipError_t launch_score_prepped(const uint16_t* qhat, const int32_t* pos, int64_t rows,
                                const uint16_t* pooled, int64_t tokens, float* scores,
                                int64_t score_cols, int32_t* status, hipStream_t stream,
                                const int32_t* dev_tokens) {
  ScoreArgs a{};
  a.dev_tokens = dev_tokens;
  a.qhat = qhat;
  a.pos = pos;
  a.rows = rows;
  a.pooled = pooled;
  a.tokens = tokens;
  a.scores = scores;
  a.score_cols = score_cols;
  a.status = status;
  return launch_score_rows<true>(a, stream);
}

}  // namespace qsa
