// Split-KV paged decode attention for gfx950, matrix-core path.
//
// Same contract as the VALU path (AstrAI commit 0b661bae, workspace.py view:
// per-split partials into decode_o_part / decode_ml_part); this file is the
// CDNA4 design that moves both contractions onto MFMA so that the VALU only
// does the softmax and the bf16 -> fp32 conversion of V.
//
// One workgroup (4 waves) per (request b, kv head g, split j); a wave takes
// every 4th 16-token tile of the split.  Per tile:
//   scores  S[token][head] = K[16 x D] . Q^T[D x 16]  with
//           v_mfma_f32_16x16x32_bf16, D/32 steps.  The K rows are loaded
//           straight into the A operand (lane l: token l%16, 16-byte chunks at
//           byte 16*(l/16) + 64*s), so one load instruction reads 64
//           contiguous bytes of 16 rows.  The B operand is Q of the G heads
//           of this kv head, replicated over the 16 columns (column c holds
//           head c % GP), loaded once.
//           Lane l then holds the scores of tokens 4*(l/16)+i (i = 0..3) for
//           head column l%16.
//   p       exp2(score * scale*log2(e) - mref) in place, with a per-head
//           reference max that is only raised when a score exceeds it by more
//           than kSlack (rare), and the true max tracked for the output.
//   p.V     v_mfma_f32_16x16x4_f32: for token group i the A operand is lane
//           l's p register i (A[head l%16][token 4k+i]) -- exactly where the
//           score MFMA left it -- and the B operand is element e of a V row
//           chunk loaded as lane l: token 4*(l/16)+i, chunk l%16 (whole rows
//           per load instruction).  D/16 accumulators hold O[head][8n+e].
// Two tiles of K/V are in flight per wave while the current one is used.
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kSlack = 8.0f;  // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int VE>
struct VChunk;
template <>
struct VChunk<8> {  // D = 128: 16 bytes per lane per row
  uint4 u;
  __device__ static VChunk zero() { VChunk c; c.u = make_uint4(0, 0, 0, 0); return c; }
  __device__ float el(int e) const {
    const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <>
struct VChunk<4> {  // D = 64: 8 bytes per lane per row
  uint2 u;
  __device__ static VChunk zero() { VChunk c; c.u = make_uint2(0, 0); return c; }
  __device__ float el(int e) const {
    const uint32_t w = e < 2 ? u.x : u.y;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};

template <int D>
struct Tile {
  static constexpr int KS = D / 32;
  static constexpr int VE = D / 16;
  uint4 k[KS];
  VChunk<VE> v[4];
};

template <int D>
__device__ __forceinline__ Tile<D> load_tile(const uint16_t* kl, const uint16_t* vl, int64_t stride,
                                             int32_t slot, int r, int c) {
  Tile<D> t;
  constexpr int KS = Tile<D>::KS, VE = Tile<D>::VE;
#pragma unroll
  for (int s = 0; s < KS; ++s) t.k[s] = make_uint4(0, 0, 0, 0);
  if (slot >= 0) {
    const uint16_t* kp = kl + (int64_t)slot * stride + 8 * r;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.k[s] = *reinterpret_cast<const uint4*>(kp + 32 * s);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t sv = __shfl(slot, 4 * r + i, 64);
    t.v[i] = VChunk<VE>::zero();
    if (sv >= 0) {
      const uint16_t* vp = vl + (int64_t)sv * stride + VE * c;
      if constexpr (VE == 8) t.v[i].u = *reinterpret_cast<const uint4*>(vp);
      else t.v[i].u = *reinterpret_cast<const uint2*>(vp);
    }
  }
  return t;
}

__device__ inline void store_empty(const AttnArgs& a, int b, int g, int j, int D) {
  for (int h = 0; h < a.group; ++h) {
    const int64_t row = ((int64_t)b * a.n_heads + g * a.group + h) * a.max_splits + j;
    for (int d = threadIdx.x; d < D; d += kThreads) a.o_part[row * D + d] = 0.0f;
    if (threadIdx.x == 0) {
      a.ml_part[row * 2 + 0] = -INFINITY;
      a.ml_part[row * 2 + 1] = -INFINITY;
    }
  }
}

template <int D, int GP>
__global__ void __launch_bounds__(kThreads)
split_attn_mfma_kernel(AttnArgs a) {
  constexpr int KS = Tile<D>::KS, VE = Tile<D>::VE;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;

  const int32_t start = a.kv_indptr[b];
  const int32_t L = a.kv_indptr[b + 1] - start;
  const int64_t pmax = a.meta[kMetaMaxPages];
  int64_t cp = (pmax + a.num_splits - 1) / a.num_splits;
  cp = cp < 1 ? 1 : cp;
  const int64_t lo64 = (int64_t)j * cp * a.page_size;
  const int64_t hi64 = lo64 + cp * a.page_size;
  const int32_t lo = (int32_t)(lo64 < L ? lo64 : L);
  const int32_t hi = (int32_t)(hi64 < L ? hi64 : L);
  if (lo >= hi) { store_empty(a, b, g, j, D); return; }

  // Q^T operand: column c holds head c % GP (zeros past the group).
  bf16x8_t qop[KS];
  {
    const int hq = c % GP;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (hq < a.group)
        v = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.n_heads + g * a.group + hq) * D +
                                            8 * r + 32 * s);
      qop[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lsum = 0.f, mtrue = -INFINITY;

  const int64_t stride = (int64_t)a.n_kv_heads * D;
  const uint16_t* kl = a.k_layer + (int64_t)g * D;
  const uint16_t* vl = a.v_layer + (int64_t)g * D;
  const int32_t* idx = a.kv_indices + start;
  const int ntiles = (hi - lo + 15) >> 4;

  auto slot_of = [&](int tile) -> int32_t {
    const int32_t t = lo + tile * 16 + c;
    return (tile < ntiles && t < hi) ? idx[t] : -1;
  };

  auto compute = [&](const Tile<D>& T, int tile) {
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, T.k[s]), qop[s], sc, 0, 0, 0);
    const int ntok = hi - (lo + tile * 16);
    float t[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[i] = (4 * r + i < ntok) ? sc[i] * a.scale_log2 : -INFINITY;
      need |= t[i] > mref + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
      float cm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float mnew = fmaxf(mref, cm);
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
      lsum *= alpha;
      mref = mnew;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float ar = __shfl(alpha, 4 * r + jj, 64);  // row 4r+jj is head column 4r+jj
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e][jj] *= ar;
      }
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mtrue = fmaxf(mtrue, t[i]);
      p[i] = __builtin_amdgcn_exp2f(t[i] - mref);
      lsum += p[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < VE; ++e)
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[i], T.v[i].el(e), acc[e], 0, 0, 0);
    }
  };

  // Tiles of this wave: wave, wave + 4, ...  Two buffers, each refilled right
  // after it is consumed, so a load is always in flight during compute.
  int tile = wave;
  int32_t slot_a = slot_of(tile), slot_b = slot_of(tile + kWaves);
  Tile<D> A = load_tile<D>(kl, vl, stride, slot_a, r, c);
  Tile<D> Bt = load_tile<D>(kl, vl, stride, slot_b, r, c);
  slot_a = slot_of(tile + 2 * kWaves);
  slot_b = slot_of(tile + 3 * kWaves);
  while (tile < ntiles) {
    compute(A, tile);
    A = load_tile<D>(kl, vl, stride, slot_a, r, c);
    slot_a = slot_of(tile + 4 * kWaves);
    tile += kWaves;
    if (tile >= ntiles) break;
    compute(Bt, tile);
    Bt = load_tile<D>(kl, vl, stride, slot_b, r, c);
    slot_b = slot_of(tile + 4 * kWaves);
    tile += kWaves;
  }

  // Reduce the wave's row groups (tokens) for the per-column statistics.
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  mtrue = fmaxf(mtrue, __shfl_xor(mtrue, 16, 64));
  mtrue = fmaxf(mtrue, __shfl_xor(mtrue, 32, 64));

  __shared__ float s_o[kWaves][GP][D];
  __shared__ float s_stat[kWaves][GP][3];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int h = 4 * r + jj;  // accumulator row = head
    if (h < GP && h < a.group) {
#pragma unroll
      for (int e = 0; e < VE; ++e) s_o[wave][h][VE * c + e] = acc[e][jj];
    }
  }
  if (r == 0 && c < GP) {
    s_stat[wave][c][0] = mref;
    s_stat[wave][c][1] = lsum;
    s_stat[wave][c][2] = mtrue;
  }
  __syncthreads();

  for (int e = threadIdx.x; e < a.group * D; e += kThreads) {
    const int h = e / D, d = e % D;
    float M = -INFINITY, mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      M = fmaxf(M, s_stat[w][h][0]);
      mt = fmaxf(mt, s_stat[w][h][2]);
    }
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (s_stat[w][h][0] == -INFINITY) continue;  // wave had no tile
      const float f = __builtin_amdgcn_exp2f(s_stat[w][h][0] - M);
      l = fmaf(s_stat[w][h][1], f, l);
      o = fmaf(s_o[w][h][d], f, o);
    }
    const int64_t row = ((int64_t)b * a.n_heads + g * a.group + h) * a.max_splits + j;
    a.o_part[row * D + d] = o / l;
    if (d == 0) {
      a.ml_part[row * 2 + 0] = mt * kLn2;
      a.ml_part[row * 2 + 1] = __logf(l) + (M - mt) * kLn2;
    }
  }
}

template <int D, int GP>
hipError_t launch_dg(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.num_splits, a.n_kv_heads, a.batch);
  hipLaunchKernelGGL((split_attn_mfma_kernel<D, GP>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  if (a.group <= 1) return launch_dg<D, 1>(a, stream);
  if (a.group <= 2) return launch_dg<D, 2>(a, stream);
  if (a.group <= 4) return launch_dg<D, 4>(a, stream);
  if (a.group <= 8) return launch_dg<D, 8>(a, stream);
  return launch_dg<D, 16>(a, stream);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace pd
