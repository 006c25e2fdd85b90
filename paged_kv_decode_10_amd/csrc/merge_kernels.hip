// Log-sum-exp merge of the split partials into decode_out.
//
// AstrAI commit 0b661bae (workspace.py view): the split partials
// decode_o_part / decode_ml_part are combined into the preallocated
// decode_out.  With lse_j = m_j + ln l_j of split j and LSE = log sum_j
// exp(lse_j), out = sum_j exp(lse_j - LSE) o_j; empty splits (lse = -inf)
// carry no weight and a request with no tokens yields zeros.
//
// Up to 64 splits: one wave per (request, query head): lane j reads split j's
// statistics, the wave reduces max and sum with shuffles, then every lane
// accumulates its D/64 columns over the non-empty splits (one coalesced row
// load per split, the loads of a batch issued together).  More splits: the
// workgroup-per-head kernel below.
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

template <int D, int NB>
__device__ __forceinline__ void load_rows(const float* op, int j0, int n, int lane, float (&v)[NB][D / 64]) {
  constexpr int E = D / 64;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int jj = j0 + (u < n ? u : n - 1);
    const float* row = op + (int64_t)jj * D + lane * E;
    if constexpr (E == 2) {
      const float2 t = *reinterpret_cast<const float2*>(row);
      v[u][0] = t.x;
      v[u][E - 1] = t.y;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = row[e];
    }
  }
}

template <int D, int NB>
__device__ __forceinline__ void accumulate(float (&acc)[D / 64], const float (&v)[NB][D / 64], float w,
                                           int u0, int n) {
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const float wj = u < n ? __shfl(w, u0 + u, 64) : 0.f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] = wj == 0.f ? acc[e] : fmaf(wj, v[u][e], acc[e]);
  }
}

template <int D>
__global__ void __launch_bounds__(kMergeWaves * 64)
merge_kernel(MergeArgs a) {
  constexpr int E = D / 64;  // columns per lane
  constexpr int kSpec = 8;   // split rows read together with the statistics
  constexpr int kBatch = 16;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (item >= active_batch(a.active, a.batch) * a.n_heads) return;
  const int64_t base = (int64_t)item * a.max_splits;  // row of split 0
  const float* ml = a.ml_part + base * 2;
  const float* op = a.o_part + base * D;

  // One round trip for the common case: the statistics of the first 64
  // splits (lane j holds split j) and, speculatively, the rows of the first
  // kSpec splits.  An empty split's row is unspecified data; its weight is 0
  // and it is never added.
  const int s0 = a.num_splits < 64 ? a.num_splits : 64;
  float lse = -INFINITY;
  if (lane < s0) {
    const float m = ml[2 * lane], ln_l = ml[2 * lane + 1];
    lse = (m == -INFINITY) ? -INFINITY : m + ln_l;
  }
  float spec[kSpec][E];
  load_rows<D, kSpec>(op, 0, s0 < kSpec ? s0 : kSpec, lane, spec);
  float M = lse;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  for (int j0 = 64; j0 < a.num_splits; j0 += 64) {  // more than 64 splits (rare)
    const int j = j0 + lane;
    float l2 = -INFINITY;
    if (j < a.num_splits) {
      const float m = ml[2 * j], ln_l = ml[2 * j + 1];
      l2 = (m == -INFINITY) ? -INFINITY : m + ln_l;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l2 = fmaxf(l2, __shfl_xor(l2, off, 64));
    M = fmaxf(M, l2);
  }

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int j0 = 0; j0 < a.num_splits; j0 += 64) {
      const int j = j0 + lane;
      float w = 0.f;
      if (j0 == 0) {
        w = lse == -INFINITY ? 0.f : __expf(lse - M);
      } else if (j < a.num_splits) {
        const float m = ml[2 * j], ln_l = ml[2 * j + 1];
        w = (m == -INFINITY) ? 0.f : __expf(m + ln_l - M);
      }
      float ws = w;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off, 64);
      wsum += ws;
      const uint64_t nonempty = __builtin_amdgcn_ballot_w64(w != 0.f);
      const int n = 64 - __clzll(nonempty);  // one past the last non-empty split
      int jb = 0;
      if (j0 == 0) {
        accumulate<D, kSpec>(acc, spec, w, 0, n < kSpec ? n : kSpec);
        jb = kSpec;
      }
      for (; jb < n; jb += kBatch) {
        float v[kBatch][E];
        load_rows<D, kBatch>(op, j0 + jb, n - jb, lane, v);
        accumulate<D, kBatch>(acc, v, w, jb, n - jb);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  uint16_t* out = a.out + (int64_t)item * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = f32_to_bf16_rne(acc[e] * inv);
}

// Many splits (S > 64): kWideSlices workgroups per (request, query head),
// each owning D / kWideSlices columns, with wave k taking splits
// [32k, 32k + 32).  A wave requests its statistics and its splits' column
// slices in one round trip: lanes 16-byte apart in a slice, LPS lanes per
// split, so one load instruction covers 64 / LPS splits.  It combines them
// relative to its own maximum, reduces over the splits a lane row holds with
// shuffles, and wave 0 joins the waves' sums through LDS:
//   M = max_k M_k,  out = sum_k e^(M_k - M) acc_k / sum_k e^(M_k - M) wsum_k.
constexpr int kWideSplits = 32;  // splits per wave
constexpr int kWideWaves = 8;    // at most 256 splits
constexpr int kWideSlices = 4;   // column slices per head (workgroups per head); 8 measured slower
constexpr int kWideFrom = 64;    // S above which the wide kernel is used: it reads every
                                 // split's row at once, empty ones too, which costs more
                                 // than the single wave's second round trip for fewer splits

template <int D>
__global__ void __launch_bounds__(kWideWaves * 64)
merge_wide_kernel(MergeArgs a) {
  constexpr int SW = D / kWideSlices;   // columns of this workgroup
  constexpr int LPS = SW / 4;           // lanes per split (a float4 each)
  constexpr int SPI = 64 / LPS;         // splits per load instruction
  constexpr int NI = kWideSplits / SPI; // load instructions per wave
  __shared__ float s_acc[kWideWaves][SW];
  __shared__ float s_m[kWideWaves], s_w[kWideWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int item = blockIdx.x / kWideSlices, slice = blockIdx.x % kWideSlices;
  if (item >= active_batch(a.active, a.batch) * a.n_heads) return;  // whole workgroup
  const int64_t base = (int64_t)item * a.max_splits;
  const float* ml = a.ml_part + base * 2;
  const float* op = a.o_part + base * D + slice * SW;
  const int j0 = wave * kWideSplits;
  int n = a.num_splits - j0;  // >= 1: the launch has ceil(S / 32) waves
  n = n < kWideSplits ? n : kWideSplits;
  const int sg = lane / LPS, cq = lane % LPS;  // split within a load, column quad
  float lse = -INFINITY;
  if (lane < n) {
    const float m = ml[2 * (j0 + lane)], ln_l = ml[2 * (j0 + lane) + 1];
    lse = (m == -INFINITY) ? -INFINITY : m + ln_l;
  }
  float4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int jj = i * SPI + sg;
    v[i] = *reinterpret_cast<const float4*>(op + (int64_t)(j0 + (jj < n ? jj : n - 1)) * D + 4 * cq);
  }
  float M = lse;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float w = (lse == -INFINITY) ? 0.f : __expf(lse - M);
  float ws = w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off, 64);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int jj = i * SPI + sg;
    const float wj = __shfl(w, jj < n ? jj : 0, 64);
    if (jj < n && wj != 0.f) {  // an empty split's row is unspecified data: never touched
      acc.x = fmaf(wj, v[i].x, acc.x);
      acc.y = fmaf(wj, v[i].y, acc.y);
      acc.z = fmaf(wj, v[i].z, acc.z);
      acc.w = fmaf(wj, v[i].w, acc.w);
    }
  }
  // sum over the lanes holding the same column quad (lane bits above LPS)
#pragma unroll
  for (int off = LPS; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, 64);
    acc.y += __shfl_xor(acc.y, off, 64);
    acc.z += __shfl_xor(acc.z, off, 64);
    acc.w += __shfl_xor(acc.w, off, 64);
  }
  if (lane < LPS) *reinterpret_cast<float4*>(&s_acc[wave][4 * lane]) = acc;
  if (lane == 0) {
    s_m[wave] = M;
    s_w[wave] = ws;
  }
  __syncthreads();
  if (wave != 0 || lane >= SW) return;
  float Mt = -INFINITY;
  for (int k = 0; k < nw; ++k) Mt = fmaxf(Mt, s_m[k]);
  float tot = 0.f, wsum = 0.f;
  if (Mt != -INFINITY) {
    for (int k = 0; k < nw; ++k) {
      if (s_m[k] == -INFINITY) continue;  // a wave whose splits are all empty
      const float f = __expf(s_m[k] - Mt);
      wsum = fmaf(f, s_w[k], wsum);
      tot = fmaf(f, s_acc[k][lane], tot);
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  a.out[(int64_t)item * D + slice * SW + lane] = f32_to_bf16_rne(tot * inv);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  const int items = a.batch * a.n_heads;
  if (a.num_splits > kWideFrom) {
    const int waves = (a.num_splits + kWideSplits - 1) / kWideSplits;  // <= 8 (S <= 256)
    if (head_dim == 64)
      hipLaunchKernelGGL(merge_wide_kernel<64>, dim3(items * kWideSlices), dim3(waves * 64), 0, stream, a);
    else
      hipLaunchKernelGGL(merge_wide_kernel<128>, dim3(items * kWideSlices), dim3(waves * 64), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid((items + kMergeWaves - 1) / kMergeWaves);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
