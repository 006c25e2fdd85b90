// Attention + merge of one layer with the split partials in a file-scope
// device array instead of the workspace arena, for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The kernels are the ones of paged_decode_attn and
// paged_decode_merge; only the partials' address and row stride differ.
//
// The array is `scratch` below.  Each GPU the library runs on holds its own
// copy for the life of the process; its device address is looked up once per
// device, at paged_decode_init_workspace with that device current, and kept in
// g_scratch_ptr.  Host code never passes the array's name itself to a kernel
// (on the host it is only a stand-in symbol): the kernels get the looked-up
// address.
//
// Nothing in the array has to start at zero: every call's attention writes
// (m, ln l) of every split of every (request, query head) it merges, empty
// splits included, and the merge never reads the o rows of empty splits.  All
// calls on one GPU share the array, so calls that overlap in time on that GPU
// (two streams, two handles, two threads) race.
#include <mutex>

#include "pd_host.h"

namespace pd {

// 32 MiB: o rows [batch, n_heads, S, head_dim] fp32 plus (m, ln l)
// [batch, n_heads, S, 2] fp32, each 256-byte aligned.  Enough for
// batch * n_heads * S * (head_dim + 2) * 4 bytes up to ~32 MiB, e.g. 4 x 64
// heads x 129 splits x 128 (17 MB) or 32 x 32 heads x 17 splits x 128 (9 MB).
constexpr size_t kScratchBytes = size_t(32) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Called by paged_decode_init_workspace with `device` current: the device
// address of this device's copy of `scratch`, looked up on the device's first
// workspace and reused afterwards.
hipError_t scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace pd

extern "C" pd_status paged_decode_attn_merge_noalloc(pd_handle* h, int32_t batch, int32_t layer,
                                                     int32_t num_splits, const void* d_q, const void* d_k_store,
                                                     const void* d_v_store, float scale, void* d_out,
                                                     hipStream_t stream) {
  if (!h || !d_out || batch < 1 || num_splits < 1) return PD_E_INVALID;
  const pd_config& c = h->cfg;
  if (batch > c.max_batch || num_splits > c.max_splits) return PD_E_CAPACITY;
  const size_t rows = (size_t)batch * c.n_heads * num_splits;
  const size_t o_bytes = pd::align256(rows * c.head_dim * 4);
  if (o_bytes + rows * 2 * 4 > pd::kScratchBytes) return PD_E_SCRATCH;
  if (h->scratch == nullptr) return PD_E_HIP;
  float* o_part = static_cast<float*>(h->scratch);
  float* ml_part = reinterpret_cast<float*>(static_cast<char*>(h->scratch) + o_bytes);
  // Partials at split stride num_splits (compact), in the scratch array.
  pd_status s = pdh::attn_launch(h, batch, layer, num_splits, d_q, nullptr, nullptr, d_k_store, d_v_store, scale,
                                 nullptr, stream, o_part, ml_part, num_splits);
  if (s == PD_OK) s = pdh::merge_launch(h, batch, num_splits, d_out, nullptr, stream, o_part, ml_part, num_splits);
  return s;
}
