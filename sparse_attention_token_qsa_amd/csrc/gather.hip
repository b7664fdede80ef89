// Decode K/V gather: each row's selected tokens' K and V vectors, copied out
// of a paged cache into contiguous per-row scratch, and the identity page
// table that lets a paged decode attention read the scratch as its cache.
//
// metrale model layers, layers/qsa.rs (module notes and decode_select): the
// kept token list indexes the sequence's paged cache; the listed tokens'
// vectors land, in list order, in a contiguous NHD scratch read through an
// identity block table.  Layout and bounds: include/qsa.h, qsa_gather_kv.
//
// One wave per (row, entry): it resolves the entry's token to (page, slot)
// and moves the K and V vectors (kv_dim bf16 each) as 16-byte chunks, lane
// l taking chunks l, l + 64, ...; K and V loads are both in flight before
// either store.  Entries past the row's count are written as zeros, so the
// scratch holds exactly the selection.  The stage is HBM-bound: 4 kv_dim
// bytes read and written per entry (K and V), from 2 kv_dim-byte runs.
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

}  // namespace

hipError_t launch_gather_kv(const uint16_t* k, const uint16_t* v, int64_t n_pages, int page_size,
                            int kv_dim, const int32_t* table, int64_t table_stride, int64_t table_len,
                            const int32_t* idx, int64_t idx_stride, const int32_t* counts, int64_t rows,
                            int64_t slots, uint16_t* ko, uint16_t* vo, int32_t* otable, int32_t* status,
                            hipStream_t stream) {
  GatherArgs a{k, v, n_pages, page_size, kv_dim, table, table_stride, table_len, idx, idx_stride,
               counts, rows, slots, ko, vo, otable, status};
  const int64_t waves = rows * slots;
  const int64_t groups = (waves + kGatherWaves - 1) / kGatherWaves;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const uintptr_t al = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                       reinterpret_cast<uintptr_t>(ko) | reinterpret_cast<uintptr_t>(vo);
  const bool vec = kv_dim % 8 == 0 && al % 16 == 0;
  const dim3 grid(static_cast<unsigned>(groups)), block(64 * kGatherWaves);
  if (vec)
    gather_kernel<true><<<grid, block, 0, stream>>>(a);
  else
    gather_kernel<false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
