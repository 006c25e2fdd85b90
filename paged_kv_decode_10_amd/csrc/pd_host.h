// Host-side internals shared by the C ABI (paged_decode.cpp) and the graph
// pool (graph_pool.cpp): the handle and the launch helpers, which also take the
// graph pool's active-request word (null outside the pool).
#pragma once

#include "pd_internal.h"

struct pd_handle {
  pd_config cfg;
  pd_layout lay;
  char* arena;
  int device;
  // The batch of the last bind call (0: none since init, when kv_indptr,
  // page_indptr and the meta words are all zero and any batch reads a
  // consistent empty step), and whether it was an extend bind.  The kernels
  // walk page_indptr / kv_indptr up to the batch they are given, so a
  // per-layer call must use the bound batch.
  int32_t bound_batch;
  int bound_extend;
  void* scratch;  // this device's static scratch array (no-allocation entry point)
};

namespace pdh {

template <typename T>
T* at(const pd_handle* h, size_t off) {
  return reinterpret_cast<T*>(h->arena + off);
}

inline pd_status hip_status(hipError_t e) { return e == hipSuccess ? PD_OK : PD_E_HIP; }

// A per-layer call must take the batch of the last bind (any batch before the
// first one).  Checked on the host, so it holds under graph capture too.
inline bool batch_matches_bind(const pd_handle* h, int32_t batch) {
  return h->bound_batch == 0 || batch == h->bound_batch;
}

int32_t auto_splits(const pd_handle* h, int32_t batch);

pd_status bind_launch(pd_handle* h, int32_t batch, int32_t mode, int32_t* d_seq_lens, int32_t* d_position_ids,
                      const int32_t* d_req_to_page, const int32_t* d_req_base, const int32_t* d_active,
                      hipStream_t stream, const int32_t* d_extend_lens = nullptr);

// The split partials go to the arena's o_part / ml_part (split stride
// max_splits), or, when o_part is given, to o_part / ml_part at split stride
// part_stride (the no-allocation entry point's scratch array).
pd_status attn_launch(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits, const void* d_q,
                      const void* d_k_new, const void* d_v_new, const void* d_k_store, const void* d_v_store,
                      float scale, const int32_t* d_active, hipStream_t stream, float* o_part = nullptr,
                      float* ml_part = nullptr, int32_t part_stride = 0);

pd_status merge_launch(pd_handle* h, int32_t batch, int32_t num_splits, void* d_out, const int32_t* d_active,
                       hipStream_t stream, const float* o_part = nullptr, const float* ml_part = nullptr,
                       int32_t part_stride = 0);

}  // namespace pdh

namespace pd {
// Device address of this device's static scratch array (noalloc.hip); call
// with `device` current.
hipError_t scratch_address(int device, void** out);
}  // namespace pd

namespace pdh {

}  // namespace pdh
