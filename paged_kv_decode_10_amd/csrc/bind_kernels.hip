// Per-step bind: the steady +1 update, the kv_indptr prefix sum and the
// kv_indices slot fill.
//
// AstrAI commit cbc58447 (cache.py view): kv_indptr is the prefix sum of
// seq_lens, built once per decode step and reused by every layer; in the steady
// state (same requests, one more token each) seq_lens / kv_indptr are advanced
// in place and position_ids moves by +1 instead of being rebuilt.  The flat
// kv_indices list is the slot of each cached token, looked up through the
// request's page list (the request -> token pool of the same page).
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kScanThreads = 1024;  // one thread per request (max_batch <= 1024)

__device__ inline int64_t wave_inclusive_scan(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ inline int wave_max_int(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  return x;
}

// One workgroup.  Thread b owns request b.
__global__ void __launch_bounds__(kScanThreads)
bind_scan_kernel(BindArgs a) {
  __shared__ int64_t wave_tot[kScanThreads / 64];
  __shared__ int wave_maxp[kScanThreads / 64];
  const int b = threadIdx.x;
  const int lane = b & 63, wave = b >> 6;
  const int B = active_batch(a.active, a.batch);
  uint32_t flags = 0;
  int64_t len = 0;
  if (b < B) {
    int32_t L = a.seq_lens[b];
    if (a.mode == PD_BIND_STEADY) {
      L += 1;
      a.seq_lens[b] = L;
      if (a.position_ids) a.position_ids[b] += 1;
    }
    const int64_t cap = (int64_t)a.max_pages_per_req * a.page_size;
    len = L;
    if (len < 0) { len = 0; flags |= PD_ERR_NEG_SEQ_LEN; }
    if (len > cap) { len = cap; flags |= PD_ERR_SEQ_OVER_TABLE; }
  }
  // Block-wide exclusive scan of the lengths (int64: no overflow before the
  // capacity clip).
  int64_t incl = wave_inclusive_scan(len);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const int64_t excl = before + incl - len;
  // Clip to the kv_indices capacity so every later read stays in bounds.
  const int64_t lo = min(excl, a.max_total_tokens);
  const int64_t hi = min(excl + len, a.max_total_tokens);
  if (b < B && hi - lo < len) flags |= PD_ERR_TOTAL_OVER_CAP;
  if (b == B - 1) a.meta[kMetaTotalTokens] = (int32_t)hi;
  const int pages = (b < B) ? (int)((hi - lo + a.page_size - 1) / a.page_size) : 0;
  if (b < B) {
    a.kv_indptr[b + 1] = (int32_t)hi;
    if (b == 0) a.kv_indptr[0] = 0;
  }
  int mp = wave_max_int(pages);
  // Second scan: page counts (the split plan walks rows page by page).
  const int64_t pincl = wave_inclusive_scan(pages);
  __syncthreads();  // wave_tot is reused
  if (lane == 63) wave_tot[wave] = pincl;
  if (lane == 0) wave_maxp[wave] = mp;
  __syncthreads();
  int64_t pbefore = 0;
  for (int w = 0; w < wave; ++w) pbefore += wave_tot[w];
  if (b < B) {
    a.page_indptr[b + 1] = (int32_t)(pbefore + pincl);
    if (b == 0) a.page_indptr[0] = 0;
  }
  if (b == 0) {
    int m = 0;
    int64_t ptotal = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      m = max(m, wave_maxp[w]);
      ptotal += wave_tot[w];
    }
    a.meta[kMetaMaxPages] = m;
    a.meta[kMetaTotalPages] = (int32_t)ptotal;
  }
  if (a.extend_lens != nullptr) {
    // Extend / prefill: the last n_b of the (clipped) tokens are new, one
    // query row each; qo_indptr is the prefix sum of n_b.  The prefill work
    // items (n_kv_heads * ceil(n_b * group / kPrefillRows) per request) are
    // listed request by request in order of decreasing length (req_order;
    // item_indptr is their prefix sum in that order), so the long items come
    // first in the prefill's schedule.
    __shared__ int32_t s_key[kScanThreads];
    __shared__ int32_t s_idx[kScanThreads];
    int64_t nb = 0;
    if (b < B) {
      nb = a.extend_lens[b];
      if (nb < 0) { nb = 0; flags |= PD_ERR_NEG_SEQ_LEN; }
      if (nb > hi - lo) { nb = hi - lo; flags |= PD_ERR_EXTEND_OVER_LEN; }
    }
    const int64_t items = (int64_t)a.n_kv_heads * ((nb * a.group + kPrefillRows - 1) / kPrefillRows);
    const int64_t qincl = wave_inclusive_scan(nb);
    __syncthreads();  // wave_tot is reused
    if (lane == 63) wave_tot[wave] = qincl;
    __syncthreads();
    int64_t qbefore = 0;
    for (int w = 0; w < wave; ++w) qbefore += wave_tot[w];
    if (b < B) {
      a.qo_indptr[b + 1] = (int32_t)(qbefore + qincl);
      if (b == 0) a.qo_indptr[0] = 0;
      if (b == B - 1) a.meta[kMetaTotalQ] = (int32_t)(qbefore + qincl);
    }
    // Bitonic sort of (length, request) over the first P2 = 2^ceil(log2 B)
    // entries: descending length, ascending request on ties; requests without
    // items and padding last.  Entries from P2 on are padding and stay put.
    s_key[b] = (b < B && items > 0) ? (int32_t)(hi - lo) : -1;
    s_idx[b] = b;
    int P2 = 1;
    while (P2 < B) P2 <<= 1;
    __syncthreads();
    for (int size = 2; size <= P2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const int partner = b ^ stride;
        if (partner > b) {
          const bool first_block = (b & size) == 0;  // this half is sorted "first-before-second"
          const int32_t k0 = s_key[b], k1 = s_key[partner];
          const int32_t i0 = s_idx[b], i1 = s_idx[partner];
          const bool before = (k0 > k1) || (k0 == k1 && i0 < i1);  // (k0, i0) goes first
          if (before != first_block) {
            s_key[b] = k1; s_key[partner] = k0;
            s_idx[b] = i1; s_idx[partner] = i0;
          }
        }
        __syncthreads();
      }
    }
    // thread p now holds the p-th request of the schedule
    const int rb = s_idx[b];
    __syncthreads();
    // items of request rb, counted by the thread that owns rb
    __shared__ int32_t s_items[kScanThreads];
    s_items[b] = (int32_t)items;
    __syncthreads();
    const int64_t my_items = (b < B) ? s_items[rb] : 0;
    const int64_t iincl = wave_inclusive_scan(my_items);
    __syncthreads();
    if (lane == 63) wave_tot[wave] = iincl;
    __syncthreads();
    int64_t ibefore = 0;
    for (int w = 0; w < wave; ++w) ibefore += wave_tot[w];
    if (b < B) {
      a.item_indptr[b + 1] = (int32_t)(ibefore + iincl);
      a.req_order[b] = rb;
      if (b == 0) a.item_indptr[0] = 0;
      if (b == B - 1) a.meta[kMetaTotalItems] = (int32_t)(ibefore + iincl);
    }
  }
  if (flags) atomicOr(a.error_word, flags);
}

constexpr int kFillThreads = 256;

// Grid (batch, Y): block (b, y) fills tokens y*256 + tid, stepping 256*Y, of
// request b.  The token range comes from the (already clipped) kv_indptr.
// Paged cache: slot = page * page_size + t % page_size through the request's
// page list.  Contiguous cache (AstrAI cache.py view: a contiguous per-request
// buffer next to the paged one): slot = base_b + t.
__global__ void __launch_bounds__(kFillThreads)
bind_fill_kernel(BindArgs a) {
  const int b = blockIdx.x;
  if (b >= active_batch(a.active, a.batch)) return;
  const int32_t start = a.kv_indptr[b];
  const int32_t len = a.kv_indptr[b + 1] - start;
  uint32_t flags = 0;
  if (a.req_base != nullptr) {
    const int64_t base = a.req_base[b];
    for (int32_t t = blockIdx.y * kFillThreads + threadIdx.x; t < len;
         t += kFillThreads * gridDim.y) {
      int64_t slot = base + t;
      if (base < 0 || slot >= a.num_slots) {
        flags |= PD_ERR_BAD_PAGE;
        slot = 0;
      }
      a.kv_indices[start + t] = (int32_t)slot;
    }
  } else {
    const int32_t* row = a.req_to_page + (int64_t)b * a.max_pages_per_req;
    for (int32_t t = blockIdx.y * kFillThreads + threadIdx.x; t < len;
         t += kFillThreads * gridDim.y) {
      const int32_t page = row[t / a.page_size];
      int64_t slot;
      if (page < 0 || (int64_t)page >= a.num_pages) {
        flags |= PD_ERR_BAD_PAGE;
        slot = 0;
      } else {
        slot = (int64_t)page * a.page_size + t % a.page_size;
      }
      a.kv_indices[start + t] = (int32_t)slot;
    }
  }
  if (flags) atomicOr(a.error_word, flags);
}

}  // namespace

hipError_t launch_bind(const BindArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(bind_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)a.max_pages_per_req * a.page_size;
  int y = (int)((cap + 4 * kFillThreads - 1) / (4 * kFillThreads));
  y = y < 1 ? 1 : (y > 256 ? 256 : y);
  hipLaunchKernelGGL(bind_fill_kernel, dim3(a.batch, y), dim3(kFillThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
