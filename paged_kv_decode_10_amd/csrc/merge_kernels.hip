// Log-sum-exp merge of the split partials into decode_out.
//
// AstrAI commit 0b661bae (workspace.py view): the split partials
// decode_o_part / decode_ml_part are combined into the preallocated
// decode_out.  With lse_j = m_j + ln l_j of split j and LSE = log sum_j
// exp(lse_j), out = sum_j exp(lse_j - LSE) o_j; empty splits (lse = -inf)
// carry no weight and a request with no tokens yields zeros.
//
// One wave per (request, query head): lane j reads split j's statistics, the
// wave reduces max and sum with shuffles, then every lane accumulates its
// D/64 columns over the non-empty splits (one coalesced row load per split).
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kMergeWaves = 4;

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int D>
__global__ void __launch_bounds__(kMergeWaves * 64)
merge_kernel(MergeArgs a) {
  constexpr int E = D / 64;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (item >= a.batch * a.n_heads) return;
  const int64_t base = (int64_t)item * a.max_splits;  // row of split 0
  const float* ml = a.ml_part + base * 2;
  const float* op = a.o_part + base * D;

  // Pass 1: max of lse over splits.
  float M = -INFINITY;
  for (int j0 = 0; j0 < a.num_splits; j0 += 64) {
    const int j = j0 + lane;
    float lse = -INFINITY;
    if (j < a.num_splits) {
      const float m = ml[2 * j], ln_l = ml[2 * j + 1];
      lse = (m == -INFINITY) ? -INFINITY : m + ln_l;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lse = fmaxf(lse, __shfl_xor(lse, off, 64));
    M = fmaxf(M, lse);
  }

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int j0 = 0; j0 < a.num_splits; j0 += 64) {
      const int j = j0 + lane;
      float w = 0.f;
      if (j < a.num_splits) {
        const float m = ml[2 * j], ln_l = ml[2 * j + 1];
        w = (m == -INFINITY) ? 0.f : __expf(m + ln_l - M);
      }
      float ws = w;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off, 64);
      wsum += ws;
      // Rows in batches of 8 with unconditional loads (indices clamped to the
      // last split, whose weight is then 0), so the loads overlap.
      const int n = min(64, a.num_splits - j0);
      for (int jb = 0; jb < n; jb += 8) {
        float v[8][E];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int jj = jb + u < n ? jb + u : n - 1;
          wj[u] = jb + u < n ? __shfl(w, jj, 64) : 0.f;
          const float* row = op + (int64_t)(j0 + jj) * D + lane * E;
          if constexpr (E == 2) {
            const float2 t = *reinterpret_cast<const float2*>(row);
            v[u][0] = t.x;
            v[u][E - 1] = t.y;
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = row[e];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = fmaf(wj[u], wj[u] == 0.f ? 0.f : v[u][e], acc[e]);
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  uint16_t* out = a.out + (int64_t)item * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = f32_to_bf16_rne(acc[e] * inv);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  const int items = a.batch * a.n_heads;
  dim3 grid((items + kMergeWaves - 1) / kMergeWaves);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
