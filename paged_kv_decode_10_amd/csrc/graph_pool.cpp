// Batch-size graph pool: one captured decode step per batch-size key.
//
// AstrAI commit e0f7fa8e (executor.py view): graphs are pre-captured at init
// for power-of-two batch sizes, one graph per batch-size key with every input
// at a fixed workspace address, in a warmup -> capture -> replay lifecycle,
// and a graph is used only when its warmup succeeded.
//
// Here a step is [steady bind, n_layers x (attention (with the fused KV append
// when new rows are given), merge)] over the caller's fixed buffers.  Keys are
// 1, 2, 4, ... below max_batch, and max_batch.  A step for `batch` requests
// runs the smallest key >= batch: the pool first writes `batch` into the
// arena's active-request word, and every kernel of the step works on that many
// requests, so the padding requests batch .. key-1 are left untouched (their
// lengths are not advanced and their outputs are not written).  A key whose
// capture or instantiation failed runs the same launches eagerly.  Capture
// executes nothing, so warmup does not touch the caller's buffers; the kernels
// allocate nothing, so no live run is needed before capture.
#include <new>

#include "pd_host.h"

namespace {

constexpr int kMaxKeys = 16;

__global__ void set_word_kernel(int32_t* p, int32_t v) { *p = v; }

}  // namespace

struct pd_graph_pool {
  pd_handle* h;
  pd_step_buffers buf;
  uint32_t flags;
  int n_keys;
  int32_t keys[kMaxKeys];
  int32_t splits[kMaxKeys];
  hipGraphExec_t exec[kMaxKeys];
  hipStream_t capture_stream;
  int32_t* active;
};

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The launches of one step at key index i (captured, or run eagerly).
pd_status launch_step(pd_graph_pool* p, int i, hipStream_t stream) {
  const pd_config& c = p->h->cfg;
  const pd_step_buffers& b = p->buf;
  const int32_t key = p->keys[i], S = p->splits[i];
  pd_status s = pdh::bind_launch(p->h, key, PD_BIND_STEADY, b.seq_lens, b.position_ids, b.req_to_page,
                                 b.req_base, p->active, stream);
  const int64_t q_stride = (int64_t)c.max_batch * c.n_heads * c.head_dim * 2;      // bytes per layer
  const int64_t new_stride = (int64_t)c.max_batch * c.n_kv_heads * c.head_dim * 2;
  for (int l = 0; l < c.n_layers && s == PD_OK; ++l) {
    const char* q = static_cast<const char*>(b.q) + l * q_stride;
    char* out = static_cast<char*>(b.out) + l * q_stride;
    const void* kn = b.k_new ? static_cast<const char*>(b.k_new) + l * new_stride : nullptr;
    const void* vn = b.v_new ? static_cast<const char*>(b.v_new) + l * new_stride : nullptr;
    s = pdh::attn_launch(p->h, key, l, S, q, kn, vn, b.k_store, b.v_store, b.scale, p->active, stream);
    if (s == PD_OK) s = pdh::merge_launch(p->h, key, S, out, p->active, stream);
  }
  return s;
}

void release_graphs(pd_graph_pool* p) {
  for (int i = 0; i < p->n_keys; ++i) {
    if (p->exec[i]) (void)hipGraphExecDestroy(p->exec[i]);
    p->exec[i] = nullptr;
  }
}

}  // namespace

extern "C" {

pd_status paged_decode_graph_pool_create(pd_handle* h, const pd_step_buffers* bufs, uint32_t flags,
                                         pd_graph_pool** out) {
  if (!out) return PD_E_INVALID;
  *out = nullptr;
  if (!h || !bufs || (flags & ~(uint32_t)PD_POOL_EAGER)) return PD_E_INVALID;
  const pd_step_buffers& b = *bufs;
  if (!b.seq_lens || !b.position_ids || !b.q || !b.k_store || !b.v_store || !b.out) return PD_E_INVALID;
  if ((b.req_to_page == nullptr) == (b.req_base == nullptr)) return PD_E_INVALID;  // exactly one layout
  if ((b.k_new == nullptr) != (b.v_new == nullptr)) return PD_E_INVALID;
  if (!aligned(b.q, 16) || !aligned(b.k_store, 16) || !aligned(b.v_store, 16) || !aligned(b.out, 16) ||
      (b.k_new && (!aligned(b.k_new, 16) || !aligned(b.v_new, 16))) || !aligned(b.seq_lens, 4) ||
      !aligned(b.position_ids, 4))
    return PD_E_INVALID;
  pd_graph_pool* p = new (std::nothrow) pd_graph_pool;
  if (!p) return PD_E_CAPACITY;
  p->h = h;
  p->buf = b;
  p->flags = flags;
  p->n_keys = 0;
  for (int32_t k = 1; k < h->cfg.max_batch && p->n_keys < kMaxKeys - 1; k *= 2) p->keys[p->n_keys++] = k;
  p->keys[p->n_keys++] = h->cfg.max_batch;
  for (int i = 0; i < p->n_keys; ++i) {
    p->splits[i] = pdh::auto_splits(h, p->keys[i]);
    p->exec[i] = nullptr;
  }
  p->active = pdh::at<int32_t>(h, h->lay.meta) + pd::kMetaActive;
  p->capture_stream = nullptr;
  if (hipStreamCreateWithFlags(&p->capture_stream, hipStreamNonBlocking) != hipSuccess) {
    delete p;
    return PD_E_HIP;
  }
  *out = p;
  return PD_OK;
}

pd_status paged_decode_graph_pool_warmup(pd_graph_pool* p) {
  if (!p) return PD_E_INVALID;
  release_graphs(p);
  if (p->flags & PD_POOL_EAGER) return PD_OK;
  // Capturing runs the host side of every launch, which records each key's
  // bind as the handle's bound batch; nothing reaches the device, so the
  // handle keeps the bind it had.
  const int32_t bound_batch = p->h->bound_batch;
  const int bound_extend = p->h->bound_extend;
  for (int i = 0; i < p->n_keys; ++i) {
    hipGraph_t g = nullptr;
    if (hipStreamBeginCapture(p->capture_stream, hipStreamCaptureModeThreadLocal) != hipSuccess) continue;
    const pd_status s = launch_step(p, i, p->capture_stream);
    const hipError_t e = hipStreamEndCapture(p->capture_stream, &g);
    if (s == PD_OK && e == hipSuccess && g) {
      hipGraphExec_t ex = nullptr;
      if (hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) == hipSuccess) p->exec[i] = ex;
    }
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();  // a failed key runs eagerly; clear its error
  }
  p->h->bound_batch = bound_batch;
  p->h->bound_extend = bound_extend;
  return PD_OK;
}

pd_status paged_decode_graph_pool_step(pd_graph_pool* p, int32_t batch, hipStream_t stream) {
  if (!p || batch < 1) return PD_E_INVALID;
  if (batch > p->h->cfg.max_batch) return PD_E_CAPACITY;
  int i = 0;
  while (p->keys[i] < batch) ++i;
  hipLaunchKernelGGL(set_word_kernel, dim3(1), dim3(1), 0, stream, p->active, batch);
  if (hipGetLastError() != hipSuccess) return PD_E_HIP;
  const pd_status s = p->exec[i] ? pdh::hip_status(hipGraphLaunch(p->exec[i], stream)) : launch_step(p, i, stream);
  // The step's bind covers requests 0 .. batch-1 (the active word): those are
  // what a per-layer call made after it may walk.
  if (s == PD_OK) {
    p->h->bound_batch = batch;
    p->h->bound_extend = 0;
  }
  return s;
}

pd_status paged_decode_graph_pool_num_keys(const pd_graph_pool* p, int32_t* n_keys) {
  if (!p || !n_keys) return PD_E_INVALID;
  *n_keys = p->n_keys;
  return PD_OK;
}

pd_status paged_decode_graph_pool_key(const pd_graph_pool* p, int32_t index, int32_t* key, int32_t* num_splits,
                                      int32_t* is_graph) {
  if (!p || index < 0 || index >= p->n_keys) return PD_E_INVALID;
  if (key) *key = p->keys[index];
  if (num_splits) *num_splits = p->splits[index];
  if (is_graph) *is_graph = p->exec[index] != nullptr;
  return PD_OK;
}

pd_status paged_decode_graph_pool_destroy(pd_graph_pool* p) {
  if (!p) return PD_E_INVALID;
  release_graphs(p);
  if (p->capture_stream) (void)hipStreamDestroy(p->capture_stream);
  delete p;
  return PD_OK;
}

}  // extern "C"
