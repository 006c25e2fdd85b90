// Host side of libpaged_decode.so: config validation, arena carve-up, split
// heuristic and the extern "C" entry points declared in include/paged_decode.h.
//
// AstrAI commit 0b661bae (workspace.py view): every per-step buffer is
// preallocated once (at executor init) at a fixed address, so nothing in the
// decode loop allocates and the step can be graph-captured.  Here the caller
// hands over one device arena and the library only carves it.
#include <math.h>
#include <new>
#include <string.h>

#include "pd_host.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxBatch = 1024;  // one scan workgroup covers the batch
constexpr int kMaxSplits = 256;
constexpr int kMaxGroup = 16;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

pd_status check_config(const pd_config* c) {
  if (!c) return PD_E_INVALID;
  if (c->n_layers < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->page_size < 1 ||
      c->max_batch < 1 || c->max_splits < 1 || c->max_pages_per_req < 1 ||
      c->num_slots < c->page_size || c->max_total_tokens < 1)
    return PD_E_INVALID;
  if (c->head_dim != 64 && c->head_dim != 128) return PD_E_UNSUPPORTED;
  if (c->n_heads % c->n_kv_heads != 0) return PD_E_UNSUPPORTED;
  if (c->n_heads / c->n_kv_heads > kMaxGroup) return PD_E_UNSUPPORTED;
  if (c->max_batch > kMaxBatch || c->max_splits > kMaxSplits) return PD_E_UNSUPPORTED;
  // Slot ids, token offsets and per-request capacities are int32.
  if (c->num_slots > INT32_MAX || c->max_total_tokens > INT32_MAX ||
      (int64_t)c->max_pages_per_req * c->page_size > INT32_MAX)
    return PD_E_UNSUPPORTED;
  return PD_OK;
}

pd_layout make_layout(const pd_config* c) {
  pd_layout l;
  memset(&l, 0, sizeof(l));
  size_t off = 0;
  l.kv_indptr = off;
  off = align_up(off + (size_t)(c->max_batch + 1) * 4);
  l.kv_indices = off;
  off = align_up(off + (size_t)c->max_total_tokens * 4);
  l.page_indptr = off;
  off = align_up(off + (size_t)(c->max_batch + 1) * 4);
  const size_t rows = (size_t)c->max_batch * c->n_heads * c->max_splits;
  l.o_part = off;
  off = align_up(off + rows * c->head_dim * 4);
  l.ml_part = off;
  off = align_up(off + rows * 2 * 4);
  l.qo_indptr = off;
  off = align_up(off + (size_t)(c->max_batch + 1) * 4);
  l.item_indptr = off;
  off = align_up(off + (size_t)(c->max_batch + 1) * 4);
  l.req_order = off;
  off = align_up(off + (size_t)c->max_batch * 4);
  l.meta = off;
  off = align_up(off + 16 * 4);
  l.error_word = off;
  off = align_up(off + 4);
  l.arena_bytes = off;
  return l;
}

}  // namespace

using pdh::at;
using pdh::hip_status;

extern "C" {

pd_status paged_decode_workspace_bytes(const pd_config* cfg, size_t* bytes) {
  if (!bytes) return PD_E_INVALID;
  pd_status s = check_config(cfg);
  if (s != PD_OK) return s;
  *bytes = make_layout(cfg).arena_bytes;
  return PD_OK;
}

pd_status paged_decode_init_workspace(const pd_config* cfg, void* d_arena, size_t arena_bytes,
                                      pd_handle** out) {
  if (!out) return PD_E_INVALID;
  *out = nullptr;
  pd_status s = check_config(cfg);
  if (s != PD_OK) return s;
  if (!d_arena || !aligned(d_arena, kAlign)) return PD_E_INVALID;
  pd_layout lay = make_layout(cfg);
  if (arena_bytes < lay.arena_bytes) return PD_E_CAPACITY;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PD_E_HIP;
  pd_handle* h = new (std::nothrow) pd_handle;
  if (!h) return PD_E_CAPACITY;
  h->cfg = *cfg;
  h->lay = lay;
  h->arena = static_cast<char*>(d_arena);
  h->device = dev;
  h->bound_batch = 0;
  h->bound_extend = 0;
  h->scratch = nullptr;
  // This device's static scratch array (the no-allocation entry point),
  // looked up with the device current.
  if (pd::scratch_address(dev, &h->scratch) != hipSuccess) {
    delete h;
    return PD_E_HIP;
  }
  // Start from an empty step: zero kv_indptr, meta and the error word so an
  // attention call before the first bind sees no tokens.
  hipError_t e = hipMemsetAsync(h->arena + lay.kv_indptr, 0, (size_t)(cfg->max_batch + 1) * 4, nullptr);
  if (e == hipSuccess)
    e = hipMemsetAsync(h->arena + lay.page_indptr, 0, (size_t)(cfg->max_batch + 1) * 4, nullptr);
  if (e == hipSuccess) e = hipMemsetAsync(h->arena + lay.meta, 0, 16 * 4, nullptr);
  if (e == hipSuccess) e = hipMemsetAsync(h->arena + lay.qo_indptr, 0, (size_t)(cfg->max_batch + 1) * 4, nullptr);
  if (e == hipSuccess) e = hipMemsetAsync(h->arena + lay.item_indptr, 0, (size_t)(cfg->max_batch + 1) * 4, nullptr);
  if (e == hipSuccess) e = hipMemsetAsync(h->arena + lay.req_order, 0, (size_t)cfg->max_batch * 4, nullptr);
  if (e == hipSuccess) e = hipMemsetAsync(h->arena + lay.error_word, 0, 4, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) {
    delete h;
    return PD_E_HIP;
  }
  *out = h;
  return PD_OK;
}

pd_status paged_decode_layout(const pd_handle* h, pd_layout* out) {
  if (!h || !out) return PD_E_INVALID;
  *out = h->lay;
  return PD_OK;
}

pd_status paged_decode_num_splits(const pd_handle* h, int32_t batch, int32_t requested,
                                  int32_t* num_splits) {
  if (!h || !num_splits || batch < 1 || requested < 0) return PD_E_INVALID;
  if (batch > h->cfg.max_batch) return PD_E_CAPACITY;
  if (requested > 0) {
    if (requested > h->cfg.max_splits) return PD_E_CAPACITY;
    *num_splits = requested;
    return PD_OK;
  }
  *num_splits = pdh::auto_splits(h, batch);
  return PD_OK;
}

}  // extern "C"

int32_t pdh::auto_splits(const pd_handle* h, int32_t batch) {
  // The plan cuts the page sequence into 2048 equal chunks when no row needs
  // more than S splits for it; rows average 2048 / (batch * n_kv_heads) chunks,
  // so allow about twice that.  More splits than pages buys nothing.
  const int64_t rows = (int64_t)batch * h->cfg.n_kv_heads;
  int64_t S = 1 + (2LL * pd::kSplitChunks + rows - 1) / rows;
  if (S > h->cfg.max_pages_per_req) S = h->cfg.max_pages_per_req;
  if (S > h->cfg.max_splits) S = h->cfg.max_splits;
  if (S < 2) S = h->cfg.max_splits >= 2 ? 2 : 1;
  return (int32_t)S;
}

pd_status pdh::bind_launch(pd_handle* h, int32_t batch, int32_t mode, int32_t* d_seq_lens,
                           int32_t* d_position_ids, const int32_t* d_req_to_page, const int32_t* d_req_base,
                           const int32_t* d_active, hipStream_t stream, const int32_t* d_extend_lens) {
  if (!h || !d_seq_lens || (!d_req_to_page && !d_req_base) || batch < 1) return PD_E_INVALID;
  if (mode != PD_BIND_FULL && mode != PD_BIND_STEADY) return PD_E_INVALID;
  if (mode == PD_BIND_STEADY && !d_position_ids) return PD_E_INVALID;
  if (!aligned(d_seq_lens, 4) || (d_req_to_page && !aligned(d_req_to_page, 4)) ||
      (d_req_base && !aligned(d_req_base, 4)) || (d_position_ids && !aligned(d_position_ids, 4)))
    return PD_E_INVALID;
  if (batch > h->cfg.max_batch) return PD_E_CAPACITY;
  pd::BindArgs a{};
  a.batch = batch;
  a.mode = mode;
  a.page_size = h->cfg.page_size;
  a.max_pages_per_req = h->cfg.max_pages_per_req;
  a.num_pages = h->cfg.num_slots / h->cfg.page_size;
  a.num_slots = h->cfg.num_slots;
  a.max_total_tokens = h->cfg.max_total_tokens;
  a.seq_lens = d_seq_lens;
  a.position_ids = d_position_ids;
  a.req_to_page = d_req_to_page;
  a.req_base = d_req_base;
  a.active = d_active;
  a.kv_indptr = at<int32_t>(h, h->lay.kv_indptr);
  a.kv_indices = at<int32_t>(h, h->lay.kv_indices);
  a.page_indptr = at<int32_t>(h, h->lay.page_indptr);
  a.meta = at<int32_t>(h, h->lay.meta);
  a.error_word = at<uint32_t>(h, h->lay.error_word);
  if (d_extend_lens) {
    if (!aligned(d_extend_lens, 4)) return PD_E_INVALID;
    a.extend_lens = d_extend_lens;
    a.qo_indptr = at<int32_t>(h, h->lay.qo_indptr);
    a.item_indptr = at<int32_t>(h, h->lay.item_indptr);
    a.req_order = at<int32_t>(h, h->lay.req_order);
    a.group = h->cfg.n_heads / h->cfg.n_kv_heads;
    a.n_kv_heads = h->cfg.n_kv_heads;
  }
  const pd_status s = hip_status(pd::launch_bind(a, stream));
  if (s == PD_OK) {
    h->bound_batch = batch;
    h->bound_extend = d_extend_lens != nullptr;
  }
  return s;
}

extern "C" {

pd_status paged_decode_bind(pd_handle* h, int32_t batch, int32_t mode, int32_t* d_seq_lens,
                            int32_t* d_position_ids, const int32_t* d_req_to_page,
                            hipStream_t stream) {
  if (!d_req_to_page) return PD_E_INVALID;
  return pdh::bind_launch(h, batch, mode, d_seq_lens, d_position_ids, d_req_to_page, nullptr, nullptr, stream);
}

pd_status paged_decode_bind_contiguous(pd_handle* h, int32_t batch, int32_t mode, int32_t* d_seq_lens,
                                       int32_t* d_position_ids, const int32_t* d_req_base,
                                       hipStream_t stream) {
  if (!d_req_base) return PD_E_INVALID;
  return pdh::bind_launch(h, batch, mode, d_seq_lens, d_position_ids, nullptr, d_req_base, nullptr, stream);
}

}  // extern "C"

// Shared by paged_decode_attn and paged_decode_append_attn (k_new == nullptr:
// no append) and the graph pool.
pd_status pdh::attn_launch(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits, const void* d_q,
                           const void* d_k_new, const void* d_v_new, const void* d_k_store,
                           const void* d_v_store, float scale, const int32_t* d_active, hipStream_t stream,
                           float* o_part, float* ml_part, int32_t part_stride) {
  if (!h || !d_q || !d_k_store || !d_v_store || batch < 1 || num_splits < 1 || layer < 0)
    return PD_E_INVALID;
  if (!aligned(d_q, 16) || !aligned(d_k_store, 16) || !aligned(d_v_store, 16))
    return PD_E_INVALID;
  if (d_k_new && (!aligned(d_k_new, 16) || !aligned(d_v_new, 16))) return PD_E_INVALID;
  const pd_config& c = h->cfg;
  if (batch > c.max_batch || num_splits > c.max_splits || layer >= c.n_layers)
    return PD_E_CAPACITY;
  if (!pdh::batch_matches_bind(h, batch)) return PD_E_INVALID;
  const int64_t layer_elems = c.num_slots * c.n_kv_heads * c.head_dim;
  pd::AttnArgs a{};
  a.batch = batch;
  a.n_heads = c.n_heads;
  a.n_kv_heads = c.n_kv_heads;
  a.group = c.n_heads / c.n_kv_heads;
  a.page_size = c.page_size;
  a.num_splits = num_splits;
  a.team = pd::kv_team(c.n_kv_heads);
  a.max_splits = o_part ? part_stride : c.max_splits;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  a.q = static_cast<const uint16_t*>(d_q);
  a.k_layer = static_cast<const uint16_t*>(d_k_store) + (int64_t)layer * layer_elems;
  a.v_layer = static_cast<const uint16_t*>(d_v_store) + (int64_t)layer * layer_elems;
  a.kv_indptr = at<int32_t>(h, h->lay.kv_indptr);
  a.kv_indices = at<int32_t>(h, h->lay.kv_indices);
  a.page_indptr = at<int32_t>(h, h->lay.page_indptr);
  a.meta = at<int32_t>(h, h->lay.meta);
  a.o_part = o_part ? o_part : at<float>(h, h->lay.o_part);
  a.ml_part = o_part ? ml_part : at<float>(h, h->lay.ml_part);
  a.k_new = static_cast<const uint16_t*>(d_k_new);
  a.v_new = static_cast<const uint16_t*>(d_v_new);
  a.k_dst = const_cast<uint16_t*>(a.k_layer);
  a.v_dst = const_cast<uint16_t*>(a.v_layer);
  a.active = d_active;
  return hip_status(pd::launch_attn(a, c.head_dim, stream));
}

extern "C" {

pd_status paged_decode_attn(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits,
                            const void* d_q, const void* d_k_store, const void* d_v_store,
                            float scale, hipStream_t stream) {
  return pdh::attn_launch(h, batch, layer, num_splits, d_q, nullptr, nullptr, d_k_store, d_v_store, scale,
                          nullptr, stream);
}

pd_status paged_decode_append_attn(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits,
                                   const void* d_q, const void* d_k_new, const void* d_v_new,
                                   void* d_k_store, void* d_v_store, float scale, hipStream_t stream) {
  if (!d_k_new || !d_v_new) return PD_E_INVALID;
  return pdh::attn_launch(h, batch, layer, num_splits, d_q, d_k_new, d_v_new, d_k_store, d_v_store, scale,
                          nullptr, stream);
}

pd_status paged_decode_append_kv(pd_handle* h, int32_t batch, int32_t layer, const void* d_k_new,
                                 const void* d_v_new, void* d_k_store, void* d_v_store, hipStream_t stream) {
  if (!h || !d_k_new || !d_v_new || !d_k_store || !d_v_store || batch < 1 || layer < 0) return PD_E_INVALID;
  if (!aligned(d_k_new, 16) || !aligned(d_v_new, 16) || !aligned(d_k_store, 16) || !aligned(d_v_store, 16))
    return PD_E_INVALID;
  const pd_config& c = h->cfg;
  if (batch > c.max_batch || layer >= c.n_layers) return PD_E_CAPACITY;
  if (!pdh::batch_matches_bind(h, batch)) return PD_E_INVALID;
  const int64_t layer_elems = c.num_slots * c.n_kv_heads * c.head_dim;
  pd::AppendArgs a{};
  a.batch = batch;
  a.row_bytes = c.n_kv_heads * c.head_dim * 2;
  a.kv_indptr = at<int32_t>(h, h->lay.kv_indptr);
  a.kv_indices = at<int32_t>(h, h->lay.kv_indices);
  a.k_new = static_cast<const uint16_t*>(d_k_new);
  a.v_new = static_cast<const uint16_t*>(d_v_new);
  a.k_layer = static_cast<uint16_t*>(d_k_store) + (int64_t)layer * layer_elems;
  a.v_layer = static_cast<uint16_t*>(d_v_store) + (int64_t)layer * layer_elems;
  return hip_status(pd::launch_append(a, stream));
}

pd_status paged_decode_bind_extend(pd_handle* h, int32_t batch, int32_t* d_seq_lens, const int32_t* d_extend_lens,
                                   const int32_t* d_req_to_page, const int32_t* d_req_base, hipStream_t stream) {
  if (!d_extend_lens || (d_req_to_page == nullptr) == (d_req_base == nullptr)) return PD_E_INVALID;
  return pdh::bind_launch(h, batch, PD_BIND_FULL, d_seq_lens, nullptr, d_req_to_page, d_req_base, nullptr, stream,
                          d_extend_lens);
}

pd_status paged_decode_prefill_attn(pd_handle* h, int32_t batch, int32_t layer, const void* d_q, int32_t q_rows,
                                    const void* d_k_store, const void* d_v_store, float scale, void* d_out,
                                    hipStream_t stream) {
  if (!h || !d_q || !d_k_store || !d_v_store || !d_out || batch < 1 || layer < 0 || q_rows < 0)
    return PD_E_INVALID;
  if (!aligned(d_q, 16) || !aligned(d_k_store, 16) || !aligned(d_v_store, 16) || !aligned(d_out, 16))
    return PD_E_INVALID;
  const pd_config& c = h->cfg;
  if (batch > c.max_batch || layer >= c.n_layers) return PD_E_CAPACITY;
  // The work list (qo_indptr, item_indptr, req_order, item count) comes from
  // an extend bind of this batch; a decode bind leaves it stale.
  if (h->bound_batch != 0 && (!h->bound_extend || batch != h->bound_batch)) return PD_E_INVALID;
  const int64_t layer_elems = c.num_slots * c.n_kv_heads * c.head_dim;
  pd::PrefillArgs a{};
  a.batch = batch;
  a.n_heads = c.n_heads;
  a.n_kv_heads = c.n_kv_heads;
  a.group = c.n_heads / c.n_kv_heads;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  a.q = static_cast<const uint16_t*>(d_q);
  a.q_rows = q_rows;
  a.k_layer = static_cast<const uint16_t*>(d_k_store) + (int64_t)layer * layer_elems;
  a.v_layer = static_cast<const uint16_t*>(d_v_store) + (int64_t)layer * layer_elems;
  a.kv_indptr = at<int32_t>(h, h->lay.kv_indptr);
  a.kv_indices = at<int32_t>(h, h->lay.kv_indices);
  a.qo_indptr = at<int32_t>(h, h->lay.qo_indptr);
  a.error_word = at<uint32_t>(h, h->lay.error_word);
  a.item_indptr = at<int32_t>(h, h->lay.item_indptr);
  a.req_order = at<int32_t>(h, h->lay.req_order);
  a.meta = at<int32_t>(h, h->lay.meta);
  a.claim = at<int32_t>(h, h->lay.meta) + pd::kMetaPrefillClaim;
  a.out = static_cast<uint16_t*>(d_out);
  a.off32 = (uint64_t)layer_elems * 2 <= 0xffffffffull && (uint64_t)c.max_total_tokens * 4 <= 0xffffffffull;
  return hip_status(pd::launch_prefill(a, c.head_dim, stream));
}

pd_status paged_decode_merge(pd_handle* h, int32_t batch, int32_t num_splits, void* d_out,
                             hipStream_t stream) {
  return pdh::merge_launch(h, batch, num_splits, d_out, nullptr, stream);
}

pd_status paged_decode_read_error(pd_handle* h, uint32_t* flags, hipStream_t stream) {
  if (!h || !flags) return PD_E_INVALID;
  uint32_t v = 0;
  void* w = h->arena + h->lay.error_word;
  hipError_t e = hipMemcpyAsync(&v, w, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemsetAsync(w, 0, 4, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return PD_E_HIP;
  *flags = v;
  return PD_OK;
}

pd_status paged_decode_destroy(pd_handle* h) {
  if (!h) return PD_E_INVALID;
  delete h;
  return PD_OK;
}

const char* paged_decode_strerror(int status) {
  switch (status) {
    case PD_OK: return "ok";
    case PD_E_INVALID: return "invalid argument (null or misaligned pointer, bad dimension or mode)";
    case PD_E_UNSUPPORTED: return "unsupported configuration (head_dim, head grouping or limits)";
    case PD_E_CAPACITY: return "capacity exceeded (batch, splits, layer or arena size)";
    case PD_E_HIP: return "HIP runtime error";
    case PD_E_SCRATCH:
      return "request exceeds the 32 MiB static scratch array of paged_decode_attn_merge_noalloc "
             "(batch * n_heads * num_splits * (head_dim + 2) * 4 bytes)";
    default: return "unknown status";
  }
}

}  // extern "C"

pd_status pdh::merge_launch(pd_handle* h, int32_t batch, int32_t num_splits, void* d_out, const int32_t* d_active,
                            hipStream_t stream, const float* o_part, const float* ml_part, int32_t part_stride) {
  if (!h || !d_out || batch < 1 || num_splits < 1) return PD_E_INVALID;
  if (!aligned(d_out, 16)) return PD_E_INVALID;
  if (batch > h->cfg.max_batch || num_splits > h->cfg.max_splits) return PD_E_CAPACITY;
  if (!pdh::batch_matches_bind(h, batch)) return PD_E_INVALID;
  pd::MergeArgs a{};
  a.batch = batch;
  a.active = d_active;
  a.n_heads = h->cfg.n_heads;
  a.num_splits = num_splits;
  a.max_splits = o_part ? part_stride : h->cfg.max_splits;
  a.o_part = o_part ? o_part : at<float>(h, h->lay.o_part);
  a.ml_part = o_part ? ml_part : at<float>(h, h->lay.ml_part);
  a.out = static_cast<uint16_t*>(d_out);
  return hip_status(pd::launch_merge(a, h->cfg.head_dim, stream));
}
