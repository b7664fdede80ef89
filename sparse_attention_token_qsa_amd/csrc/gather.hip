// Decode K/V gather: each row's selected tokens' K and V vectors, copied out
// of a paged cache into contiguous per-row scratch, and the identity page
// table that lets a paged decode attention read the scratch as its cache.
//
// metrale model layers, layers/qsa.rs (module notes and decode_select): the
// kept token list indexes the sequence's paged cache; the listed tokens'
// vectors land, in list order, in a contiguous NHD scratch read through an
// identity block table.  Layout and bounds: include/qsa.h, qsa_gather_kv.
//
// One wave per (row, entry), or per two consecutive entries of a row in
// batches that fill the chip: the entry's token is resolved to (page, slot)
// (the only dependent loads: count, list entry, page-table entry) and the K
// and V vectors (kv_dim bf16 each) move as 16-byte chunks, lane l taking
// chunks l, l + 64, ..., every entry's loads in flight before its stores.  Entries past
// the row's count are written as zeros, so the scratch holds exactly the
// selection.  The stage is HBM-bound: 4 kv_dim bytes read and written per
// entry (K and V), from 2 kv_dim-byte runs.
#include "../../include/qsa.h"
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

struct GatherArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t n_pages;
  int page_size;
  int kv_dim;
  const int32_t* table;
  int64_t table_stride;
  int64_t table_len;
  const int32_t* idx;
  int64_t idx_stride;
  const int32_t* counts;
  int64_t rows;
  int64_t slots;
  uint16_t* ko;
  uint16_t* vo;
  int32_t* otable;
  int32_t* status;
};

constexpr int kGatherWaves = 4;

template <bool VEC>
__global__ __launch_bounds__(64 * kGatherWaves) void gather_kernel(const GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kGatherWaves + (threadIdx.x >> 6);
  if (e >= a.rows * a.slots) return;  // uniform per wave
  const int64_t r = e / a.slots;
  const int64_t i = e - r * a.slots;
  const int64_t ppr = a.slots / a.page_size;
  if (i % a.page_size == 0 && lane == 0) {
    const int64_t j = i / a.page_size;
    a.otable[r * ppr + j] = static_cast<int32_t>(r * ppr + j);
  }
  // a list holds at most min(slots, idx_stride) entries
  const int64_t cmax = a.slots < a.idx_stride ? a.slots : a.idx_stride;
  int64_t c = a.counts[r];
  if (c < 0 || c > cmax) {
    if (i == 0 && lane == 0) atomicOr(a.status, QSA_STATUS_BAD_INDEX);
    c = c < 0 ? 0 : cmax;
  }
  // source row of the cache, or -1 for a zero entry
  int64_t src = -1;
  if (i < c) {
    const int64_t t = a.idx[r * a.idx_stride + i];
    const int64_t lp = t >= 0 ? t / a.page_size : -1;
    if (t >= 0 && lp < a.table_len) {
      const int64_t page = a.table[r * a.table_stride + lp];
      if (page >= 0 && page < a.n_pages) src = page * a.page_size + (t - lp * a.page_size);
    }
    if (src < 0 && lane == 0) atomicOr(a.status, QSA_STATUS_BAD_INDEX);
  }
  const int64_t dst = e * a.kv_dim;
  if constexpr (VEC) {
    const int chunks = a.kv_dim / 8;
    const uint4* ks = reinterpret_cast<const uint4*>(a.k + (src < 0 ? 0 : src) * a.kv_dim);
    const uint4* vs = reinterpret_cast<const uint4*>(a.v + (src < 0 ? 0 : src) * a.kv_dim);
    uint4* kd = reinterpret_cast<uint4*>(a.ko + dst);
    uint4* vd = reinterpret_cast<uint4*>(a.vo + dst);
    for (int ch = lane; ch < chunks; ch += 64) {
      uint4 kx = make_uint4(0u, 0u, 0u, 0u), vx = kx;
      if (src >= 0) {
        kx = ks[ch];
        vx = vs[ch];
      }
      kd[ch] = kx;
      vd[ch] = vx;
    }
  } else {
    const uint16_t* ks = a.k + (src < 0 ? 0 : src) * a.kv_dim;
    const uint16_t* vs = a.v + (src < 0 ? 0 : src) * a.kv_dim;
    for (int x = lane; x < a.kv_dim; x += 64) {
      a.ko[dst + x] = src >= 0 ? ks[x] : 0;
      a.vo[dst + x] = src >= 0 ? vs[x] : 0;
    }
  }
}

// Source row of the cache for entry i of row r (i < slots), or -1 for a
// zero entry; `flag`: set the status bit for a listed entry that does not
// resolve.
__device__ __forceinline__ int64_t resolve(const GatherArgs& a, int64_t r, int64_t i, int64_t c, bool flag) {
  if (i >= c) return -1;
  const int64_t t = a.idx[r * a.idx_stride + i];
  const int64_t lp = t >= 0 ? t / a.page_size : -1;
  int64_t src = -1;
  if (t >= 0 && lp < a.table_len) {
    const int64_t page = a.table[r * a.table_stride + lp];
    if (page >= 0 && page < a.n_pages) src = page * a.page_size + (t - lp * a.page_size);
  }
  if (src < 0 && flag) atomicOr(a.status, QSA_STATUS_BAD_INDEX);
  return src;
}

// Large batches: one wave per E consecutive entries of one row.  Lane j < E
// resolves entry j (count, list entry, page-table entry: the only dependent
// loads), then all 64 lanes move the entries' K and V vectors as 16-byte
// chunks (lane l takes chunks l, l + 64, ...), the loads of all E entries
// issued before their stores.
template <bool VEC, int E>
__global__ __launch_bounds__(64 * kGatherWaves) void gather_batch_kernel(const GatherArgs a) {
  constexpr int kEntriesPerWave = E, kInFlight = E;
  const int lane = threadIdx.x & 63;
  const int64_t wpr = (a.slots + kEntriesPerWave - 1) / kEntriesPerWave;  // waves per row
  const int64_t wv = static_cast<int64_t>(blockIdx.x) * kGatherWaves + (threadIdx.x >> 6);
  if (wv >= a.rows * wpr) return;  // uniform per wave
  const int64_t r = wv / wpr;
  const int64_t i0 = (wv - r * wpr) * kEntriesPerWave;
  const int64_t ppr = a.slots / a.page_size;
  // a list holds at most min(slots, idx_stride) entries
  const int64_t cmax = a.slots < a.idx_stride ? a.slots : a.idx_stride;
  int64_t c = a.counts[r];
  if (c < 0 || c > cmax) {
    if (i0 == 0 && lane == 0) atomicOr(a.status, QSA_STATUS_BAD_INDEX);
    c = c < 0 ? 0 : cmax;
  }
  const int64_t il = i0 + lane;
  int64_t src_l = -1;
  if (lane < E && il < a.slots) {
    src_l = resolve(a, r, il, c, true);
    if (il % a.page_size == 0) a.otable[r * ppr + il / a.page_size] = static_cast<int32_t>(r * ppr + il / a.page_size);
  }
  const int n_ent = static_cast<int>(a.slots - i0 < kEntriesPerWave ? a.slots - i0 : kEntriesPerWave);
  auto src_of = [&](int e) {  // entry e's source row, uniform across the wave
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(src_l), e));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(src_l >> 32), e));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  const int64_t dst0 = (r * a.slots + i0) * a.kv_dim;
  if constexpr (VEC) {
    const int chunks = a.kv_dim / 8;
    for (int ch = lane; ch < chunks; ch += 64) {
      for (int e0 = 0; e0 < n_ent; e0 += kInFlight) {
        uint4 kx[kInFlight], vx[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
          kx[u] = make_uint4(0u, 0u, 0u, 0u);
          vx[u] = kx[u];
          if (e0 + u < n_ent) {
            const int64_t src = src_of(e0 + u);
            if (src >= 0) {
              kx[u] = reinterpret_cast<const uint4*>(a.k + src * a.kv_dim)[ch];
              vx[u] = reinterpret_cast<const uint4*>(a.v + src * a.kv_dim)[ch];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
          if (e0 + u < n_ent) {
            const int64_t dst = dst0 + static_cast<int64_t>(e0 + u) * a.kv_dim;
            reinterpret_cast<uint4*>(a.ko + dst)[ch] = kx[u];
            reinterpret_cast<uint4*>(a.vo + dst)[ch] = vx[u];
          }
        }
      }
    }
  } else {
    for (int e = 0; e < n_ent; ++e) {
      const int64_t src = src_of(e);
      const int64_t dst = dst0 + static_cast<int64_t>(e) * a.kv_dim;
      const uint16_t* ks = a.k + (src < 0 ? 0 : src) * a.kv_dim;
      const uint16_t* vs = a.v + (src < 0 ? 0 : src) * a.kv_dim;
      for (int x = lane; x < a.kv_dim; x += 64) {
        a.ko[dst + x] = src >= 0 ? ks[x] : 0;
        a.vo[dst + x] = src >= 0 ? vs[x] : 0;
      }
    }
  }
}

}  // namespace

hipError_t launch_gather_kv(const uint16_t* k, const uint16_t* v, int64_t n_pages, int page_size,
                            int kv_dim, const int32_t* table, int64_t table_stride, int64_t table_len,
                            const int32_t* idx, int64_t idx_stride, const int32_t* counts, int64_t rows,
                            int64_t slots, uint16_t* ko, uint16_t* vo, int32_t* otable, int32_t* status,
                            hipStream_t stream) {
  GatherArgs a{k, v, n_pages, page_size, kv_dim, table, table_stride, table_len, idx, idx_stride,
               counts, rows, slots, ko, vo, otable, status};
  // Two entries per wave once the batch fills the chip (64 rows x 2064
  // entries: 95 -> 86 us back to back, 89 -> 83 us cold); one for smaller
  // batches, where more waves in flight win (one row: 3.4 against 3.8 us).
  const int ent = rows * slots >= 65536 ? 2 : 1;
  const int64_t waves = rows * ((slots + ent - 1) / ent);
  const int64_t groups = (waves + kGatherWaves - 1) / kGatherWaves;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const uintptr_t al = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                       reinterpret_cast<uintptr_t>(ko) | reinterpret_cast<uintptr_t>(vo);
  const bool vec = kv_dim % 8 == 0 && al % 16 == 0;
  const dim3 grid(static_cast<unsigned>(groups)), block(64 * kGatherWaves);
  if (vec && ent == 2)
    gather_batch_kernel<true, 2><<<grid, block, 0, stream>>>(a);
  else if (vec)
    gather_kernel<true><<<grid, block, 0, stream>>>(a);
  else if (ent == 2)
    gather_batch_kernel<false, 2><<<grid, block, 0, stream>>>(a);
  else
    gather_kernel<false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
