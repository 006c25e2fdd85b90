// Internal declarations shared by the host ABI and the kernel translation
// units of libpaged_decode.so.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/paged_decode.h"

namespace pd {

// Words of the arena's meta block written by the bind scan.
enum MetaWord : int {
  kMetaMaxPages = 0,     // max over requests of ceil(L_b / page_size)
  kMetaTotalTokens = 1,  // sum of the (clamped) lengths
  kMetaTotalPages = 2,   // sum over requests of ceil(L_b / page_size)
  kMetaActive = 4,       // active requests of a padded graph-pool step (graph pool only)
  kMetaTotalQ = 5,       // extend bind: sum of the (clamped) new-token counts
  kMetaTotalItems = 6,   // extend bind: prefill work items (request, kv head, query rows)
  kMetaPrefillClaim = 7, // prefill: work-item counter (0 between launches)
};

// The attention launches this many waves.  They work in teams of
// kv_team(n_kv_heads) waves; a team walks one chunk of the page sequence and
// each of its waves reads one kv head of those pages.
constexpr int kSplitChunks = PD_PLAN_WAVES;
constexpr int kTeamMax = PD_PLAN_TEAM_MAX;  // waves per workgroup

// Waves per team = kv heads per bundle: gcd(n_kv_heads, kTeamMax).
static_assert(kTeamMax == 4, "kv_team below is gcd(n, 4)");
inline __host__ __device__ int kv_team(int n_kv_heads) {
  return (n_kv_heads % 4 == 0) ? 4 : (n_kv_heads % 2 == 0) ? 2 : 1;
}

// Requests a kernel works on: `batch`, or in a graph-pool step (captured at a
// padded batch) the active count the pool wrote into the arena, clamped to
// [1, batch].  Requests past it are left untouched.
__device__ __forceinline__ int active_batch(const int32_t* active, int batch) {
  if (active == nullptr) return batch;
  const int n = *active;
  return n < 1 ? 1 : (n > batch ? batch : n);
}

struct BindArgs {
  int32_t batch;
  const int32_t* active;      // null, or the graph pool's active-request word
  int32_t mode;
  int32_t page_size;
  int32_t max_pages_per_req;
  int64_t num_pages;          // num_slots / page_size
  int64_t max_total_tokens;
  int32_t* seq_lens;
  int32_t* position_ids;      // may be null
  const int32_t* req_to_page;  // paged cache: [batch, max_pages_per_req] page ids
  const int32_t* req_base;     // contiguous cache: [batch] first slot of each request (else null)
  int64_t num_slots;
  int32_t* kv_indptr;
  int32_t* kv_indices;
  int32_t* page_indptr;       // [batch + 1]: prefix sum of ceil(L_b / page_size)
  int32_t* meta;
  uint32_t* error_word;
  // extend bind only (else null): new tokens per request, and the prefix sums
  // of the new-token counts and of the prefill work items per request
  // (n_kv_heads * ceil(n_b * group / kPrefillRows)).
  const int32_t* extend_lens;
  int32_t* qo_indptr;
  int32_t* item_indptr;       // over the requests in req_order
  int32_t* req_order;         // requests by decreasing length (prefill schedule)
  int32_t group;
  int32_t n_kv_heads;
};

struct AttnArgs {
  int32_t batch;
  const int32_t* active;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t group;              // n_heads / n_kv_heads
  int32_t page_size;
  int32_t num_splits;         // S used for this launch
  int32_t team;               // kv_team(n_kv_heads)
  int32_t max_splits;         // stride of the partial buffers
  float scale_log2;           // scale * log2(e)
  const uint16_t* q;          // bf16 [batch, n_heads, D]
  const uint16_t* k_layer;    // bf16 [num_slots, n_kv_heads, D] of this layer
  const uint16_t* v_layer;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* page_indptr;
  const int32_t* meta;
  float* o_part;              // [max_batch, n_heads, max_splits, D]
  float* ml_part;             // [max_batch, n_heads, max_splits, 2]
  // KV append fused into the launch (null when not appending): the new
  // token's rows, bf16 [batch, n_kv_heads, D], and the writable layer stores
  // (the same addresses as k_layer / v_layer).
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_dst;
  uint16_t* v_dst;
};

struct MergeArgs {
  int32_t batch;
  const int32_t* active;
  int32_t n_heads;
  int32_t num_splits;
  int32_t max_splits;
  const float* o_part;
  const float* ml_part;
  uint16_t* out;              // bf16 [batch, n_heads, D]
};

struct AppendArgs {
  int32_t batch;
  const int32_t* active;
  int32_t row_bytes;          // n_kv_heads * head_dim * 2
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const uint16_t* k_new;      // bf16 [batch, n_kv_heads, D]
  const uint16_t* v_new;
  uint16_t* k_layer;          // bf16 [num_slots, n_kv_heads, D] of this layer
  uint16_t* v_layer;
};

// Prefill work item: one request, one kv head, kPrefillRows query rows.  A
// wave holds kPrefillTiles MFMA tiles of 16 (new token, query head) rows, and
// the four waves of a workgroup share one item (and its K/V, staged in LDS).
constexpr int kPrefillTiles = 2;
constexpr int kPrefillWavesPerItem = 4;
constexpr int kPrefillRows = 16 * kPrefillTiles * kPrefillWavesPerItem;

struct PrefillArgs {
  int32_t batch;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t group;
  float scale_log2;
  const uint16_t* q;          // bf16 [q_rows, n_heads, D], ragged by qo_indptr
  int32_t q_rows;             // rows of q and out: rows at or past it are not computed
  const uint16_t* k_layer;
  const uint16_t* v_layer;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* qo_indptr;
  const int32_t* item_indptr;
  const int32_t* req_order;
  const int32_t* meta;
  int32_t* claim;             // the work-item counter (a meta word)
  uint16_t* out;              // bf16 [q_rows, n_heads, D]
  uint32_t* error_word;
  int32_t off32;              // a layer's K (and V) store and kv_indices each span < 4 GiB:
                              // 32-bit byte offsets from a uniform base address them
};

hipError_t launch_bind(const BindArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream);

}  // namespace pd
