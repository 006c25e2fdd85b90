// Split-KV paged decode attention for gfx950, matrix-core path.
//
// Same contract as the VALU path (AstrAI commit 0b661bae, workspace.py view:
// per-split partials into decode_o_part / decode_ml_part); this file is the
// CDNA4 design that moves both contractions onto MFMA so that the VALU only
// does the softmax and packs operands.
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
//   p.V     v_mfma_f32_16x16x16_bf16: the A operand is lane l's four p values
//           rounded to bf16 (A[head l%16][token 4*(l/16)+i]) -- exactly where
//           the score MFMA left them.  V rows are loaded as lane l: token
//           4*(l/16)+i, 16-byte chunk l%16 (whole rows per load instruction),
//           and the B operand of column group e is element e of those four
//           rows, packed with two byte permutes.  D/16 accumulators hold
//           O[head][d = (D/16)*n + e].  The softmax sum uses p in fp32.
// Two tiles of K/V are in flight per wave while the current one is used.
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
#ifndef PD_MFMA_MIN_WAVES_PER_EU
#define PD_MFMA_MIN_WAVES_PER_EU 2
#endif
constexpr float kSlack = 8.0f;  // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

template <int VE>
struct VChunk;
template <>
struct VChunk<8> {  // D = 128: 16 bytes (8 bf16) of one V row per lane
  uint4 u;
  __device__ uint32_t dw(int w) const { return w == 0 ? u.x : w == 1 ? u.y : w == 2 ? u.z : u.w; }
};
template <>
struct VChunk<4> {  // D = 64: 8 bytes (4 bf16) of one V row per lane
  uint2 u;
  __device__ uint32_t dw(int w) const { return w == 0 ? u.x : u.y; }
};

template <int D>
struct Tile {
  static constexpr int KS = D / 32;
  static constexpr int VE = D / 16;
  uint4 k[KS];
  VChunk<VE> v[4];
};

// All loads are unconditional: every lane holds a valid slot (tokens past the
// split's end were redirected to its last token), so the compiler can count
// the loads in flight exactly and never drains the pipeline early.
template <int D>
__device__ __forceinline__ Tile<D> load_tile(const uint16_t* kl, const uint16_t* vl, int64_t stride,
                                             int32_t slot, int r, int c) {
  Tile<D> t;
  constexpr int KS = Tile<D>::KS, VE = Tile<D>::VE;
  const uint16_t* kp = kl + (int64_t)slot * stride + 8 * r;
#pragma unroll
  for (int s = 0; s < KS; ++s) t.k[s] = *reinterpret_cast<const uint4*>(kp + 32 * s);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t sv = __shfl(slot, 4 * r + i, 64);
    const uint16_t* vp = vl + (int64_t)sv * stride + VE * c;
    if constexpr (VE == 8) t.v[i].u = *reinterpret_cast<const uint4*>(vp);
    else t.v[i].u = *reinterpret_cast<const uint2*>(vp);
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
__global__ void __launch_bounds__(kThreads, PD_MFMA_MIN_WAVES_PER_EU)
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
    const bool real = hq < a.group;
    const uint16_t* qp = a.q + ((int64_t)b * a.n_heads + g * a.group + (real ? hq : 0)) * D + 8 * r;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * s);  // unconditional load
      if (!real) v = make_uint4(0, 0, 0, 0);
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

  // Slot of token c of a tile.  Tokens at or past hi (the tail of the last
  // tile, and tiles past the end that are only prefetched) read the split's
  // last token instead: a real row of this request, so finite, and its score
  // is masked to -inf below, giving it weight 0.
  auto slot_of = [&](int tile) -> int32_t {
    const int32_t t = lo + tile * 16 + c;
    return idx[t < hi ? t : hi - 1];
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
    // p in fp32 for the softmax sum (exact lse); rounded to bf16 as the
    // A operand of the p.V product.
    bf16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mtrue = fmaxf(mtrue, t[i]);
      const float p = __builtin_amdgcn_exp2f(t[i] - mref);
      lsum += p;
      pb[i] = (__bf16)p;
    }
    const i16x4_t pa = __builtin_bit_cast(i16x4_t, pb);
    // B operand for column group e: element e of the lane's 4 token rows,
    // packed pairwise with byte permutes (low or high bf16 of a dword).
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2_t bv;
      bv[0] = __builtin_amdgcn_perm(T.v[1].dw(e >> 1), T.v[0].dw(e >> 1), sel);
      bv[1] = __builtin_amdgcn_perm(T.v[3].dw(e >> 1), T.v[2].dw(e >> 1), sel);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(i16x4_t, bv), acc[e], 0, 0, 0);
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
