// Split-KV paged decode attention for gfx950 (VALU path).
//
// AstrAI commit 0b661bae (workspace.py view): the decode attention kernel
// writes per-split partial outputs and (max, log-sum) statistics into the
// preallocated decode_o_part / decode_ml_part buffers; a merge produces
// decode_out.  Everything else here is this kernel's own design for CDNA4.
//
// One workgroup (4 waves) per (request b, kv head g, split j).  The G query
// heads of kv head g share every K/V row the workgroup reads.
//
// Lane layout: a token is handled by LPT = D / DPL lanes, each holding DPL
// elements of the row as 16-byte chunks interleaved so that the LPT lanes of
// one load instruction read LPT*16 contiguous bytes of the row.  A wave covers
// TOK = 64 / LPT tokens per step; the four waves take steps round-robin.
//   * q.k: v_dot2 on bf16 pairs (q is bf16 already, so no conversion), then a
//     DPP butterfly over the LPT lanes of the token.
//   * softmax: online, in log2 units (scale * log2(e) folded into the score),
//     with a wave-uniform reference max per head that is only raised when a
//     score exceeds it by more than kRescaleSlack, so the accumulator rescale
//     is rare; the exact max is tracked separately for the (m, ln l) output.
//   * p.v: fp32 FMAs on the converted V chunk; each lane accumulates its DPL
//     columns for its own tokens, and the token groups are summed once at the
//     end of the split.
// The next step's K/V rows are loaded while the current step is computed.
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleSlack = 8.0f;  // log2 units: p stays <= 256
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Sum over the LPT consecutive lanes of a token (all of them get the total).
template <int LPT>
__device__ inline float token_sum(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "LPT");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if (LPT >= 8) x += dpp<kRowHalfMirror>(x);
  if (LPT >= 16) x += dpp<kRowMirror>(x);
  return x;
}

// Sum over the token groups of a wave (lanes with equal lane % LPT).
template <int LPT>
__device__ inline float group_sum(float x) {
  if (LPT == 4) { x += dpp<kRowRor4>(x); x += dpp<kRowRor8>(x); }
  if (LPT == 8) { x += dpp<kRowRor8>(x); }
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ inline void store_empty(const AttnArgs& a, int b, int g, int j, int D) {
  for (int h = 0; h < a.group; ++h) {
    const int hq = g * a.group + h;
    const int64_t row = ((int64_t)b * a.n_heads + hq) * a.max_splits + j;
    for (int d = threadIdx.x; d < D; d += kThreads) a.o_part[row * D + d] = 0.0f;
    if (threadIdx.x == 0) {
      a.ml_part[row * 2 + 0] = -INFINITY;
      a.ml_part[row * 2 + 1] = -INFINITY;
    }
  }
}

template <int CH>
struct Rows {
  uint4 k[CH];
  uint4 v[CH];
};

// K and V chunks of one slot (this lane's slice).  Unconditional, so the
// compiler can count the loads in flight exactly.
template <int CH, int LPT>
__device__ __forceinline__ Rows<CH> load_rows(const uint4* kbase, const uint4* vbase,
                                              int64_t stride16, int ls, int32_t slot) {
  Rows<CH> r;
  const int64_t off = (int64_t)slot * stride16 + ls;
#pragma unroll
  for (int k = 0; k < CH; ++k) { r.k[k] = kbase[off + LPT * k]; r.v[k] = vbase[off + LPT * k]; }
  return r;
}

template <int D, int GP, int DPL>
struct Cfg {
  static constexpr int LPT = D / DPL;     // lanes per token
  static constexpr int TOK = 64 / LPT;    // tokens per wave step
  static constexpr int CH = DPL / 8;      // 16-byte chunks per lane per row
  static constexpr int W = DPL / 2;       // 32-bit words per lane per row
};

template <int D, int GP, int DPL>
__global__ void __launch_bounds__(kThreads)
split_attn_valu_kernel(AttnArgs a) {
  using C = Cfg<D, GP, DPL>;
  constexpr int LPT = C::LPT, TOK = C::TOK, CH = C::CH, W = C::W;

  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tg = lane / LPT;  // token within the step
  const int ls = lane % LPT;  // slice of the row

  const int32_t start = a.kv_indptr[b];
  const int32_t L = a.kv_indptr[b + 1] - start;
  const int64_t pmax = a.meta[kMetaMaxPages];
  int64_t c = (pmax + a.num_splits - 1) / a.num_splits;
  c = c < 1 ? 1 : c;
  const int64_t lo64 = (int64_t)j * c * a.page_size;
  const int32_t lo = (int32_t)(lo64 < L ? lo64 : L);
  const int32_t hi = (int32_t)(lo64 + c * a.page_size < L ? lo64 + c * a.page_size : L);
  if (lo >= hi) { store_empty(a, b, g, j, D); return; }

  // q of the G heads, this lane's slice, as packed bf16 pairs.
  uint32_t qv[GP][W];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    const bool real = h < a.group;  // loads stay unconditional; padded heads get zeros
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + ((int64_t)b * a.n_heads + g * a.group + (real ? h : 0)) * D);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      uint4 v = qp[ls + LPT * k];
      if (!real) v = make_uint4(0, 0, 0, 0);
      qv[h][4 * k + 0] = v.x; qv[h][4 * k + 1] = v.y;
      qv[h][4 * k + 2] = v.z; qv[h][4 * k + 3] = v.w;
    }
  }

  float acc[GP][DPL];
  float lsum[GP], mref[GP], mtrue[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    lsum[h] = 0.f; mref[h] = -INFINITY; mtrue[h] = -INFINITY;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[h][i] = 0.f;
  }

  const int32_t* idx = a.kv_indices + start;
  const int64_t row_stride = (int64_t)a.n_kv_heads * D;  // elements per slot
  const uint4* kbase = reinterpret_cast<const uint4*>(a.k_layer + (int64_t)g * D);
  const uint4* vbase = reinterpret_cast<const uint4*>(a.v_layer + (int64_t)g * D);
  const int64_t row_stride16 = row_stride / 8;  // in uint4 units

  const int nsteps = (hi - lo + TOK - 1) / TOK;

  // Tokens at or past hi read the split's last token (a real, finite row);
  // their scores are masked to -inf so they carry weight 0.
  auto token_valid = [&](int step) { return lo + step * TOK + tg < hi; };
  auto load_slot = [&](int step) -> int32_t {
    const int32_t t = lo + step * TOK + tg;
    return idx[t < hi ? t : hi - 1];
  };

  int step = wave;
  int32_t slot_cur = load_slot(step);
  int32_t slot_nxt = load_slot(step + kWaves);
  Rows<CH> cur = load_rows<CH, LPT>(kbase, vbase, row_stride16, ls, slot_cur);

  for (; step < nsteps; step += kWaves) {
    // Prefetch: next step's rows and the index two steps ahead.
    const Rows<CH> nxt = load_rows<CH, LPT>(kbase, vbase, row_stride16, ls, slot_nxt);
    const int32_t slot_nn = load_slot(step + 2 * kWaves);
    const bool valid = token_valid(step);

    // Scores (log2 units) for the G heads of this lane's token.
    float t[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        s = dot2_bf16(qv[h][4 * k + 0], cur.k[k].x, s);
        s = dot2_bf16(qv[h][4 * k + 1], cur.k[k].y, s);
        s = dot2_bf16(qv[h][4 * k + 2], cur.k[k].z, s);
        s = dot2_bf16(qv[h][4 * k + 3], cur.k[k].w, s);
      }
      s = token_sum<LPT>(s);
      t[h] = valid ? s * a.scale_log2 : -INFINITY;
    }

    // Raise the wave's reference max only when some score would overflow the
    // slack; rescale the running sums by exp2(old - new) then.
    bool need = false;
#pragma unroll
    for (int h = 0; h < GP; ++h) need |= t[h] > mref[h] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float mnew = fmaxf(mref[h], wave_max(t[h]));
        const float alpha = __builtin_amdgcn_exp2f(mref[h] - mnew);
        lsum[h] *= alpha;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[h][i] *= alpha;
        mref[h] = mnew;
      }
    }

    float vf[DPL];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      vf[8 * k + 0] = bf16_lo(cur.v[k].x); vf[8 * k + 1] = bf16_hi(cur.v[k].x);
      vf[8 * k + 2] = bf16_lo(cur.v[k].y); vf[8 * k + 3] = bf16_hi(cur.v[k].y);
      vf[8 * k + 4] = bf16_lo(cur.v[k].z); vf[8 * k + 5] = bf16_hi(cur.v[k].z);
      vf[8 * k + 6] = bf16_lo(cur.v[k].w); vf[8 * k + 7] = bf16_hi(cur.v[k].w);
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      mtrue[h] = fmaxf(mtrue[h], t[h]);
      const float p = __builtin_amdgcn_exp2f(t[h] - mref[h]);
      lsum[h] += p;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[h][i] = fmaf(p, vf[i], acc[h][i]);
    }

    slot_cur = slot_nxt;
    slot_nxt = slot_nn;
    cur = nxt;
  }

  // Sum the wave's token groups (they share mref), then combine the waves.
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    lsum[h] = group_sum<LPT>(lsum[h]);
    mtrue[h] = wave_max(mtrue[h]);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[h][i] = group_sum<LPT>(acc[h][i]);
  }

  __shared__ float s_acc[kWaves][GP][D];
  __shared__ float s_stat[kWaves][GP][3];
  if (tg == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * (ls + LPT * k) + e] = acc[h][8 * k + e];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      s_stat[wave][h][0] = mref[h];
      s_stat[wave][h][1] = lsum[h];
      s_stat[wave][h][2] = mtrue[h];
    }
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
      const float f = __builtin_amdgcn_exp2f(s_stat[w][h][0] - M);  // 0 for an idle wave
      l = fmaf(s_stat[w][h][1], f, l);
      o = fmaf(s_acc[w][h][d], f, o);
    }
    const int hq = g * a.group + h;
    const int64_t row = ((int64_t)b * a.n_heads + hq) * a.max_splits + j;
    a.o_part[row * D + d] = o / l;
    if (d == 0) {
      // natural-log units: m = mtrue*ln2;  ln l_true = ln l + (M - mtrue)*ln2
      a.ml_part[row * 2 + 0] = mt * kLn2;
      a.ml_part[row * 2 + 1] = __logf(l) + (M - mt) * kLn2;
    }
  }
}

template <int D, int GP>
hipError_t launch_dg(const AttnArgs& a, hipStream_t stream) {
  constexpr int DPL = GP >= 8 ? 8 : 16;
  dim3 grid(a.num_splits, a.n_kv_heads, a.batch);
  hipLaunchKernelGGL((split_attn_valu_kernel<D, GP, DPL>), grid, dim3(kThreads), 0, stream, a);
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

hipError_t launch_attn_valu(const AttnArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace pd
