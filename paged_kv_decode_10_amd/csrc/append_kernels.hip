// Per-layer KV append: the new token's K and V rows go into the stores.
//
// AstrAI commit cbc58447 (cache.py view): the per-layer cache write is a
// single advanced-index store buffer[layer_id, loc], and the slot
// bookkeeping moved into the once-per-step bind.  Here the bind has already
// counted the new token in seq_lens, so it is position L_b - 1 of request b
// and its slot is the request's last kv_indices entry.
//
// One workgroup per request copies the request's [n_kv_heads, D] K row and
// V row (16-byte vector loads and stores).  A request with no tokens has no
// new token and is skipped.
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kAppendThreads = 256;

__global__ void __launch_bounds__(kAppendThreads) append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  if (b >= active_batch(a.active, a.batch)) return;
  const int32_t end = a.kv_indptr[b + 1];
  if (end == a.kv_indptr[b]) return;
  const int64_t slot = a.kv_indices[end - 1];
  const int n16 = a.row_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(a.k_new) + (int64_t)b * n16;
  const uint4* vs = reinterpret_cast<const uint4*>(a.v_new) + (int64_t)b * n16;
  uint4* kd = reinterpret_cast<uint4*>(a.k_layer) + slot * n16;
  uint4* vd = reinterpret_cast<uint4*>(a.v_layer) + slot * n16;
  for (int i = threadIdx.x; i < n16; i += kAppendThreads) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(a.batch), dim3(kAppendThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
