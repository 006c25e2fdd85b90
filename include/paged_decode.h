/*
 * paged_decode.h -- C ABI of libpaged_decode.so: split-KV paged decode
 * attention for MI355X (gfx950).
 *
 * One decode step of an LLM inference engine: a batch of B single-token
 * queries attends over a paged bf16 KV cache.  The operations follow the
 * AstrAI engine as described on three commit pages:
 *   [WS] AstrAI commit 0b661bae, astrai/inference/core/workspace.py view
 *   [CA] AstrAI commit cbc58447, astrai/inference/core/cache.py view
 *   [EX] AstrAI commit e0f7fa8e, astrai/inference/core/executor.py view
 *
 * Conventions for every entry point:
 *   - Returns a pd_status; nothing aborts, throws or prints.
 *   - Every device pointer is borrowed: the caller allocates and frees it
 *     (typically with PyTorch).  Device pointers must be 16-byte aligned.
 *   - The library never calls hipMalloc/hipFree.  All per-step buffers live in
 *     one caller-supplied device arena carved at fixed offsets at init, so the
 *     kernel arguments of a step never change and a whole multi-layer step can
 *     be captured into a hipGraph and replayed ([WS]: buffers preallocated at
 *     executor init, no allocation in the decode hot loop, fixed addresses as
 *     the prerequisite for graph capture).
 *   - Work is enqueued on the given stream only; no call except
 *     paged_decode_read_error reads device memory back or synchronises.
 *   - A handle is not thread-safe; use one per thread or serialise.
 *   - Identical inputs and split count give bit-identical results.
 *
 * Index conventions (all int32): kv_indptr and kv_indices are token-granular.
 * Page p owns storage slots [p*page_size, (p+1)*page_size).  A request's t-th
 * cached token is in page req_to_page[b][t / page_size] at offset
 * t % page_size.  Query head h reads kv head h / (n_heads / n_kv_heads).
 */
#ifndef PAGED_DECODE_H
#define PAGED_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pd_status {
  PD_OK = 0,
  PD_E_INVALID = 1,     /* null / misaligned pointer, bad dimension or mode,
                           a batch other than the last bind's               */
  PD_E_UNSUPPORTED = 2, /* head_dim not 64/128, n_heads % n_kv_heads != 0,
                           group size above 16 ([EX]: graphs only for a
                           supported head_dim)                                */
  PD_E_CAPACITY = 3,    /* batch > max_batch, splits > max_splits, arena too
                           small, layer out of range                          */
  PD_E_HIP = 4,         /* a HIP launch or copy failed                        */
  PD_E_SCRATCH = 5      /* paged_decode_attn_merge_noalloc: the partials do not
                           fit its 32 MiB static scratch array                */
} pd_status;

/* Bits of the device error word (see paged_decode_read_error).  A kernel that
 * meets a bad value records it here and clamps instead of reading out of
 * bounds; outputs of a step with a nonzero word are undefined. */
enum {
  PD_ERR_NEG_SEQ_LEN = 1u << 0,    /* seq_lens[b] < 0: treated as 0          */
  PD_ERR_SEQ_OVER_TABLE = 1u << 1, /* seq_lens[b] > max_pages_per_req*page_size:
                                      clamped to that                          */
  PD_ERR_TOTAL_OVER_CAP = 1u << 2, /* sum(seq_lens) > max_total_tokens: the
                                      lengths are clipped to fit               */
  PD_ERR_BAD_PAGE = 1u << 3,       /* a page id outside [0, num_slots/page_size):
                                      its slots are redirected to slot 0       */
  PD_ERR_EXTEND_OVER_LEN = 1u << 4 /* extend bind: extend_lens[b] > seq_lens[b]
                                      (after clipping): treated as seq_lens[b] */
};

/* Launch constants of the split plan (part of the ABI: the partition that
 * paged_decode_attn documents is defined in terms of them, and the same
 * values hold on every device).  One attention launch runs PD_PLAN_WAVES
 * waves (512 workgroups of 4: two per compute unit on a 256-CU MI355X); kv
 * heads are bundled T = gcd(n_kv_heads, PD_PLAN_TEAM_MAX) at a time and the
 * page sequence is cut into C = PD_PLAN_WAVES / T chunks. */
#define PD_PLAN_WAVES 2048
#define PD_PLAN_TEAM_MAX 4

/* Bind modes ([CA]: steady-state detection lets bind increment seq_lens and
 * kv_indptr in place and reuse the request map; [WS]: position_ids, seq_lens
 * and kv_indptr are updated in place instead of rebuilt). */
enum {
  PD_BIND_FULL = 0,   /* the caller has written seq_lens for this step        */
  PD_BIND_STEADY = 1  /* same requests, each one token longer: the device adds
                         1 to seq_lens[b] and position_ids[b] first           */
};

typedef struct pd_config {
  int32_t n_layers;          /* layers in the K/V stores                        */
  int32_t n_heads;           /* query heads H                                   */
  int32_t n_kv_heads;        /* kv heads Hkv; H % Hkv == 0, H / Hkv <= 16       */
  int32_t head_dim;          /* D: 64 or 128                                    */
  int32_t page_size;         /* tokens per page, >= 1                           */
  int32_t max_batch;         /* 1 .. 1024                                       */
  int32_t max_splits;        /* 1 .. 256: capacity of the split partials        */
  int32_t max_pages_per_req; /* row width of req_to_page, >= 1                  */
  int64_t num_slots;         /* slots per layer in each store, >= page_size     */
  int64_t max_total_tokens;  /* capacity of kv_indices (sum of seq_lens), >= 1  */
} pd_config;

/* Byte offsets into the arena and the shapes behind them. */
typedef struct pd_layout {
  size_t arena_bytes;
  size_t kv_indptr;   /* int32 [max_batch + 1]                                 */
  size_t kv_indices;  /* int32 [max_total_tokens]                              */
  size_t page_indptr; /* int32 [max_batch + 1]: prefix sum of ceil(L_b / page_size)
                         (pages per request, used by the split plan)           */
  size_t o_part;      /* fp32  [max_batch, n_heads, max_splits, head_dim]:
                         each split's output normalised by its own softmax sum
                         ([WS] decode_o_part)                                  */
  size_t ml_part;     /* fp32  [max_batch, n_heads, max_splits, 2]: (m, ln l)
                         with m the split's max scaled score and
                         l = sum exp(s - m); lse = m + ln l; an empty split
                         holds (-inf, -inf) and its o_part row is
                         unspecified ([WS] decode_ml_part)                     */
  size_t qo_indptr;   /* int32 [max_batch + 1]: extend bind: prefix sum of the
                         new-token counts (prefill query rows)                 */
  size_t item_indptr; /* int32 [max_batch + 1]: extend bind: prefix sum of the
                         prefill work items per request, in req_order          */
  size_t req_order;   /* int32 [max_batch]: extend bind: requests by decreasing
                         length (the prefill schedule)                         */
  size_t meta;        /* int32 [16]: [0] = max pages of any request this step,
                         [1] = total tokens, [2] = total pages this step       */
  size_t error_word;  /* uint32: PD_ERR_* bits                                 */
} pd_layout;

typedef struct pd_handle pd_handle;

/* Arena size for a config (pure host).  Every sub-buffer is 256-byte aligned.
 * ([WS]: the workspace owns decode_o_part / decode_ml_part / decode_out and
 * the bind metadata, all sized once at executor init; this call sizes the
 * library's share of that workspace.) */
pd_status paged_decode_workspace_bytes(const pd_config* cfg, size_t* bytes);

/* ([WS]: every per-step buffer is preallocated at executor init, at a fixed
 * address, so the decode loop allocates nothing and can be graph-captured.)
 * Validates cfg and carves the caller's device arena (d_arena, arena_bytes >=
 * paged_decode_workspace_bytes) at fixed offsets.  Allocates only the small
 * host handle; never device memory.  The arena must stay alive and untouched
 * by the caller (except through read-only views) until destroy.  Zeroes the
 * step metadata (kv_indptr, page_indptr, the extend-bind arrays, the meta
 * words) and the error word on the null stream and waits for it, so a call
 * before the first bind sees an empty step; looks up this device's static
 * scratch array (paged_decode_attn_merge_noalloc) with the device current;
 * PD_E_HIP if either fails. */
pd_status paged_decode_init_workspace(const pd_config* cfg, void* d_arena,
                                      size_t arena_bytes, pd_handle** out);

/* Offsets of the arena's sub-buffers, for read-only views (tests, tools).
 * No passage defines this call: it exposes the [WS] workspace buffers'
 * placement, which the pages leave to the implementation. */
pd_status paged_decode_layout(const pd_handle* h, pd_layout* out);

/* No passage defines a split count: the pages name the split partials
 * ([WS] decode_o_part / decode_ml_part) but not how many splits a request
 * gets, so the rule below is this library's own.
 * Resolves the split count S for a batch: requested > 0 is honoured (it must be
 * <= max_splits); requested == 0 picks S = 1 + ceil(4096 / (batch*n_kv_heads)),
 * capped at max_splits and max_pages_per_req (at least 2), so that the split
 * plan below can give all chunks the same number of pages.
 * Pass the same S to paged_decode_attn and paged_decode_merge. */
pd_status paged_decode_num_splits(const pd_handle* h, int32_t batch, int32_t requested,
                                  int32_t* num_splits);

/* Per-step metadata ([CA]: kv_indptr is the prefix sum of seq_lens, built once
 * per step and shared by every layer; steady +1 update).
 *   d_seq_lens      int32 [batch], in/out (incremented in PD_BIND_STEADY)
 *   d_position_ids  int32 [batch], in/out (incremented in PD_BIND_STEADY; may
 *                   be NULL in PD_BIND_FULL)
 *   d_req_to_page   int32 [batch, max_pages_per_req] row-major page ids
 * Writes the arena's kv_indptr [batch+1] and kv_indices [sum seq_lens] and the
 * meta words, and makes `batch` the batch of the per-layer calls that follow.
 * Two kernels on `stream`; no host sync. */
pd_status paged_decode_bind(pd_handle* h, int32_t batch, int32_t mode, int32_t* d_seq_lens,
                            int32_t* d_position_ids, const int32_t* d_req_to_page,
                            hipStream_t stream);

/* The same bind for a contiguous cache ([CA]: a contiguous per-request buffer
 * next to the paged one): request b's tokens occupy slots base_b, base_b + 1,
 * ... of the stores, so kv_indices[kv_indptr[b] + t] = d_req_base[b] + t.
 *   d_req_base  int32 [batch]: the first slot of each request's buffer
 * Lengths are capped at max_pages_per_req * page_size as in the paged bind
 * (the per-request capacity); a token whose slot falls outside
 * [0, num_slots) sets PD_ERR_BAD_PAGE and reads slot 0.  The split plan and
 * the attention are unchanged (they count pages of page_size tokens). */
pd_status paged_decode_bind_contiguous(pd_handle* h, int32_t batch, int32_t mode, int32_t* d_seq_lens,
                                       int32_t* d_position_ids, const int32_t* d_req_base,
                                       hipStream_t stream);

/* Split-KV attention for one layer ([WS]: attn_paged_decode writes split
 * partials into decode_o_part / decode_ml_part).
 *   d_q        bf16 [batch, n_heads, head_dim] queries of this layer
 *   d_k_store  bf16 [n_layers, num_slots, n_kv_heads, head_dim] (base of the
 *   d_v_store  whole store; the library adds the 64-bit offset of `layer`)
 *   scale      softmax scale applied to q.k (float32)
 * Split plan (S = num_splits, P_b = ceil(L_b / page_size)): the kv heads
 * form bundles of T = gcd(n_kv_heads, PD_PLAN_TEAM_MAX) consecutive heads, and
 * the bundle rows (request b, bundle gs) are laid end to end, request-major,
 * each as its P_b pages.  S = 1: each row is one split.  S >= 2: the page
 * sequence is cut into chunks of Qp = max(ceil(TP / C), ceil(P_max / (S - 1)), 1)
 * pages (C = PD_PLAN_WAVES / T, TP = (n_kv_heads / T) * sum P_b,
 * P_max = max P_b), and split
 * j of row (b, g) is the intersection of bundle row (b, g / T) with the j-th
 * chunk that touches it -- a contiguous, page-aligned token range; a row
 * never has more than S splits.  For every
 * query head h of kv head g, o_part[b,h,j,:] and ml_part[b,h,j,:] describe
 * split j; splits past a row's last one are empty: ml = (-inf, -inf) and
 * o_part is left unspecified.  Reads kv_indptr / kv_indices / page_indptr
 * from the last bind; batch must be the last bind's (else PD_E_INVALID).
 * One launch of PD_PLAN_WAVES waves (the T waves of a team read the T heads
 * of one bundle over the same chunk). */
pd_status paged_decode_attn(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits,
                            const void* d_q, const void* d_k_store, const void* d_v_store,
                            float scale, hipStream_t stream);

/* Per-layer KV append ([CA]: the per-layer cache write is the single-index
 * store buffer[layer_id, loc]; the slot bookkeeping lives in the per-step
 * bind).  Call after paged_decode_bind, which has counted the new token in
 * seq_lens: the token is position L_b - 1 of request b and its slot is that
 * request's last kv_indices entry.  Copies
 *   k_store[layer, slot_b, :, :] = d_k_new[b, :, :]   (and the same for V)
 * for every request with L_b >= 1 (a request with no tokens is skipped).
 *   d_k_new, d_v_new   bf16 [batch, n_kv_heads, head_dim], this layer's new rows
 *   d_k_store, d_v_store  the whole [n_layers, num_slots, n_kv_heads, head_dim]
 *                      stores, written in place (the library adds the layer
 *                      offset)
 * Slots of distinct requests must differ (a valid page table).  One kernel on
 * `stream`; all pointers 16-byte aligned.  batch must be the last bind's
 * (else PD_E_INVALID). */
pd_status paged_decode_append_kv(pd_handle* h, int32_t batch, int32_t layer, const void* d_k_new,
                                 const void* d_v_new, void* d_k_store, void* d_v_store, hipStream_t stream);

/* The KV append fused into the attention launch: the same writes as
 * paged_decode_append_kv followed by the same partials as paged_decode_attn
 * (bit for bit), in one kernel.  The wave that reads a row's newest token takes
 * its K/V from d_k_new / d_v_new and writes them into the stores, so no wave
 * reads a slot while it is being written.  Arguments as in those two calls. */
pd_status paged_decode_append_attn(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits,
                                   const void* d_q, const void* d_k_new, const void* d_v_new,
                                   void* d_k_store, void* d_v_store, float scale, hipStream_t stream);

/* ---- Paged prefill / extend ([WS]/[CA]: the prefill qo_indptr is built once
 * per step in the workspace and reused by every layer's prefill) ---- */

/* Extend bind: request b holds L_b = d_seq_lens[b] cached tokens (K/V of all
 * of them already in the stores), of which the last n_b = d_extend_lens[b]
 * are new and have query rows.  Writes kv_indptr / kv_indices (as
 * paged_decode_bind in PD_BIND_FULL mode, through d_req_to_page, or as
 * paged_decode_bind_contiguous through d_req_base: exactly one non-NULL),
 * qo_indptr = prefix sum of n_b, and the prefill work list.  n_b is clamped
 * to [0, L_b] (PD_ERR_NEG_SEQ_LEN / PD_ERR_EXTEND_OVER_LEN). */
pd_status paged_decode_bind_extend(pd_handle* h, int32_t batch, int32_t* d_seq_lens, const int32_t* d_extend_lens,
                                   const int32_t* d_req_to_page, const int32_t* d_req_base, hipStream_t stream);

/* Causal attention of every new token over its request's cache, one layer:
 * new token i of request b (query row qo_indptr[b] + i, position
 * p = L_b - n_b + i) attends to that request's tokens 0 .. p:
 *   out[row, h, :] = sum_t softmax_t(scale * q[row, h] . K_t) V_t   (t <= p),
 * kv head of query head h = h / (n_heads / n_kv_heads); rounded to bf16.
 *   d_q     bf16 [q_rows, n_heads, head_dim] (rows ragged by qo_indptr)
 *   q_rows  rows the caller allocated in d_q and d_out: query rows at or past
 *           it (sum n_b > q_rows) are not computed and set PD_ERR_TOTAL_OVER_CAP
 *   d_out   bf16 [q_rows, n_heads, head_dim], caller-owned
 *   stores as in paged_decode_attn.  Reads the last bind, which must be an
 * extend bind of the same batch (else PD_E_INVALID; before any bind the
 * arena holds an empty work list and nothing is computed).  One
 * persistent launch: 512 workgroups of 4 waves over work items (request,
 * kv head, 128 query rows), longest requests first. */
pd_status paged_decode_prefill_attn(pd_handle* h, int32_t batch, int32_t layer, const void* d_q, int32_t q_rows,
                                    const void* d_k_store, const void* d_v_store, float scale, void* d_out,
                                    hipStream_t stream);

/* Log-sum-exp merge of the S partials into decode_out ([WS]: decode_out is
 * preallocated in the workspace):
 *   out[b,h,:] = sum_j exp(lse_j - LSE) o_j,  LSE = log sum_j exp(lse_j),
 * empty splits skipped, rounded to bf16 (nearest-even).  A request with no
 * tokens gets zeros.  d_out bf16 [batch, n_heads, head_dim], caller-owned.
 * batch must be the last bind's (else PD_E_INVALID). */
pd_status paged_decode_merge(pd_handle* h, int32_t batch, int32_t num_splits, void* d_out,
                             hipStream_t stream);

/* No-allocation variant of paged_decode_attn followed by paged_decode_merge,
 * for callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * the same results, bit for bit, but the split partials live in a file-scope
 * device array of the library (32 MiB per GPU, held until the process ends)
 * instead of the workspace arena, at split stride num_splits.  The caller
 * passes the inputs (as paged_decode_attn) and d_out (as paged_decode_merge);
 * the arena's o_part / ml_part are not touched.  Allocates nothing, ever.
 * Returns PD_E_SCRATCH when batch * n_heads * num_splits * (head_dim + 2) * 4
 * bytes (o rows 256-byte aligned) exceed 32 MiB.  Every call on a GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (other streams,
 * handles or threads) race.  Nothing in the array needs clearing between
 * calls: each call writes every partial statistic it reads. */
pd_status paged_decode_attn_merge_noalloc(pd_handle* h, int32_t batch, int32_t layer, int32_t num_splits,
                                          const void* d_q, const void* d_k_store, const void* d_v_store,
                                          float scale, void* d_out, hipStream_t stream);

/* ---- Batch-size graph pool ([EX]: graphs pre-captured at init for
 * power-of-two batch sizes, one graph per batch-size key with all inputs at
 * fixed workspace addresses, a warmup -> capture -> replay lifecycle, graphs
 * used only when warmup succeeds) ---- */

/* The caller's fixed buffers of a decode step, each sized for max_batch. */
typedef struct pd_step_buffers {
  int32_t* seq_lens;          /* int32 [max_batch], advanced +1 per step       */
  int32_t* position_ids;      /* int32 [max_batch], advanced +1 per step       */
  const int32_t* req_to_page; /* int32 [max_batch, max_pages_per_req] (paged)  */
  const int32_t* req_base;    /* int32 [max_batch] (contiguous); exactly one of
                                 req_to_page and req_base is non-NULL           */
  const void* q;              /* bf16 [n_layers, max_batch, n_heads, head_dim] */
  void* k_store;              /* bf16 [n_layers, num_slots, n_kv_heads, head_dim] */
  void* v_store;
  const void* k_new;          /* bf16 [n_layers, max_batch, n_kv_heads, head_dim]:
                                 the new tokens' rows, appended in the attention
                                 launch; NULL (with v_new) for no append        */
  const void* v_new;
  void* out;                  /* bf16 [n_layers, max_batch, n_heads, head_dim] */
  float scale;
} pd_step_buffers;

typedef struct pd_graph_pool pd_graph_pool;

enum { PD_POOL_EAGER = 1 };   /* capture nothing: every key runs eagerly       */

/* A pool over the handle's workspace.  Keys are 1, 2, 4, ... below max_batch,
 * and max_batch; key k uses S = paged_decode_num_splits(k, 0).  Holds the
 * pointers (the buffers must outlive the pool) and one private capture stream.
 * No device memory is allocated. */
pd_status paged_decode_graph_pool_create(pd_handle* h, const pd_step_buffers* bufs, uint32_t flags,
                                         pd_graph_pool** out);

/* Captures the step of every key:
 *   steady bind, then per layer l: attention (append_attn with k_new/v_new
 *   layer l, else attn) of q layer l, and the merge into out layer l.
 * Capture executes nothing, so the buffers are not touched and the handle
 * keeps the bind it had.  A key whose capture or instantiation fails runs
 * eagerly afterwards (see _key). */
pd_status paged_decode_graph_pool_warmup(pd_graph_pool* p);

/* One steady decode step of requests 0 .. batch-1 (1 <= batch <= max_batch) on
 * `stream`: writes `batch` into the workspace's active-request word, then
 * replays (or runs eagerly) the step of the smallest key >= batch.  Every
 * kernel stops at `batch` requests: the padding requests batch .. key-1 keep
 * their lengths and their output rows.  The results equal those of the eager
 * calls with the same batch and the key's split count, bit for bit.  Counts
 * as a bind of `batch` requests: per-layer calls made after it take `batch`. */
pd_status paged_decode_graph_pool_step(pd_graph_pool* p, int32_t batch, hipStream_t stream);

pd_status paged_decode_graph_pool_num_keys(const pd_graph_pool* p, int32_t* n_keys);
/* Key `index`: its batch size, split count and whether it replays a graph. */
pd_status paged_decode_graph_pool_key(const pd_graph_pool* p, int32_t index, int32_t* key, int32_t* num_splits,
                                      int32_t* is_graph);
/* Destroys the graphs and the capture stream (not the buffers). */
pd_status paged_decode_graph_pool_destroy(pd_graph_pool* p);

/* Diagnostics, never in the hot path: synchronises `stream`, returns the
 * device error word (PD_ERR_* bits) and clears it.  No passage defines it:
 * the pages say nothing of error reporting; here capacity violations are
 * recorded on the device so that nothing in a step reads device memory back. */
pd_status paged_decode_read_error(pd_handle* h, uint32_t* flags, hipStream_t stream);

/* Frees the host handle; the arena belongs to the caller.  No passage:
 * lifetime management of this library's own handle. */
pd_status paged_decode_destroy(pd_handle* h);

/* Static description of a status code.  No passage: this library's error
 * reporting. */
const char* paged_decode_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_DECODE_H */
