// Paged prefill / extend attention for gfx950 (CDNA4).
//
// AstrAI commits 0b661bae / cbc58447 (workspace.py and cache.py views): the
// prefill qo_indptr is built once per step in the workspace and reused by
// every layer's prefill, like kv_indptr for decode.  Here request b's last
// n_b cached tokens are new, each with a query row (rows ragged by
// qo_indptr); new token i sits at position p = L_b - n_b + i and attends
// causally to the cached tokens 0 .. p of its request.
//
// Work item = (request b, kv head g, kPrefillRows = 128 query rows).  The
// rows of a request and kv head are its (new token i, query head hh) pairs,
// token major, hh in [0, G): item k holds rows 128k .. 128k + 127, so each
// 16-row MFMA tile covers 16/G new tokens (G <= 16).  A workgroup of four
// waves takes an item; wave wv holds the 32 rows 128k + 32wv .. as two
// 16-row tiles, and all four share the item's K/V, which the workgroup stages
// into LDS 64 tokens at a time.  The launch is persistent: workgroup w takes
// item w first, then items handed out by a counter, longest requests first
// (the extend bind orders them).  Per 64-token stage, with the decode
// kernel's matrix-core scheme:
//   scores  S[token][row] = K[16 x D] . Q^T[D x 16] on v_mfma_f32_16x16x32_bf16,
//           K read from LDS in the A-operand layout and the q of the tile's
//           16 rows held as the B operand for the whole item;
//   p       exp2 with a lazily raised reference max (rescale only when a score
//           passes it by more than 8 in log2 units); tokens past a row's
//           causal limit are -inf;
//   p.V     v_mfma_f32_16x16x32_bf16 over two 16-token units at a time, p
//           (bf16) as the A operand where the score MFMA left it and V staged
//           in LDS already in the B-operand layout.
// The next stage's K/V is fetched into registers while the current one is
// computed.  Outputs are normalised and rounded to bf16.
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWavesTotal = 2048;
constexpr float kSlack = 8.0f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// LDS staging: double buffered (stage s+1 is fetched into registers while
// the four 16-token units of stage s are computed from LDS, and the slots of
// stage s+2 are in flight).  Each K/V row is read from memory once per item,
// and one memory round trip covers four units of compute.
constexpr int kStageTok = 64;

// One token's V values for one lane column group: VE bf16 (16 or 8 bytes).
template <int VE>
struct VPiece;
template <>
struct VPiece<8> {
  uint4 u;
  __device__ uint32_t dw(int w) const { return w == 0 ? u.x : w == 1 ? u.y : w == 2 ? u.z : u.w; }
  __device__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
};
template <>
struct VPiece<4> {
  uint2 u;
  __device__ uint32_t dw(int w) const { return w == 0 ? u.x : u.y; }
  __device__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint2*>(p); }
};

// Load at a 32-bit byte offset from a wave-uniform base (one address register).
template <typename T>
__device__ __forceinline__ T ld_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(static_cast<const char*>(base) + byte_off);
}

template <int D, bool OFF32>
__global__ void __launch_bounds__(kThreads, 2)
prefill_lds_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;  // score MFMA steps (32 bf16 of q.k each)
  constexpr int VE = D / 16;  // p.V accumulators (16 columns each)
  constexpr int NQ = kPrefillTiles;
  constexpr int CPR = D / 8;                          // 16-byte chunks per K or V row
  constexpr int RS = CPR;                             // LDS row stride (uint4), chunks XOR-swizzled by token
  constexpr int kStageChunks = kStageTok * CPR;       // K chunks per stage
  constexpr int kKPer = kStageChunks / kThreads;      // K chunks a thread moves per stage
  constexpr int kPer = kKPer + 4;                     // slots a thread needs per stage (K chunks, 4 V tokens)
  // K: [token][chunk], 16-byte chunk k of token t stored at position k ^ (t % CPR)
  // of the token's row (an XOR swizzle: the score reads, 16 tokens x one chunk
  // per instruction, hit 16 different bank groups; rows padded by 16 bytes
  // instead measured 3x the bank-conflict cycles).  V: transposed for the p.V operand --
  // word (pair p, element e, lane 16r + c) holds element e of lane column
  // group c for tokens 4r..4r+3 of the pair's first unit, then of its second
  // (eight bf16, the B operand of one 16x16x32 MFMA), written at staging.
  __shared__ uint4 sK[2][kStageTok * RS];
  __shared__ uint4 sVt[2][2 * VE * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int B = a.batch, G = a.group, H = a.n_heads, Hkv = a.n_kv_heads;
  const int total_items = a.meta[kMetaTotalItems];
  const int64_t kv_stride = (int64_t)Hkv * D;

  // Schedule: workgroup w first takes item w, then items W + k for k handed out
  // by the counter (the next claim is requested while an item is computed).
  // Every workgroup that had a first item ends with exactly one claim past the
  // end; the one that receives the last index ever handed out resets the
  // counter for the next launch.
  __shared__ int32_t s_claim;
  const int W = gridDim.x;
  const int last_claim = max(total_items - W, 0) + min(total_items, W) - 1;
  for (int item = blockIdx.x; item < total_items;) {
    int32_t kc = 0;
    if (tid == 0) kc = __hip_atomic_fetch_add(a.claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int cnt = 0;
    for (int i0 = 0; i0 <= B; i0 += 64) {
      const int i = i0 + lane;
      const bool le = i <= B && a.item_indptr[i <= B ? i : B] <= item;
      cnt += __popcll(__builtin_amdgcn_ballot_w64(le));
    }
    const int pos = __builtin_amdgcn_readfirstlane(cnt - 1);  // place of the request in the schedule
    const int b = __builtin_amdgcn_readfirstlane(a.req_order[pos]);
    const int i_lo = __builtin_amdgcn_readfirstlane(a.item_indptr[pos]);
    const int i_hi = __builtin_amdgcn_readfirstlane(a.item_indptr[pos + 1]);
    const int groups = (i_hi - i_lo) / Hkv;
    const int k = item - i_lo;  // the request's row groups last-first (longest causal range first)
    const int g = k % Hkv, grp = groups - 1 - k / Hkv;
    const int kv0 = __builtin_amdgcn_readfirstlane(a.kv_indptr[b]);
    const int L = __builtin_amdgcn_readfirstlane(a.kv_indptr[b + 1]) - kv0;
    const int q0 = __builtin_amdgcn_readfirstlane(a.qo_indptr[b]);
    const int n_all = __builtin_amdgcn_readfirstlane(a.qo_indptr[b + 1]) - q0;
    const int n = min(n_all, max(a.q_rows - q0, 0));
    if (n < n_all && tid == 0) atomicOr(a.error_word, PD_ERR_TOTAL_OVER_CAP);
    const int row0_item = kPrefillRows * grp;
    const bool skip = n <= 0 || row0_item >= n * G;  // the whole workgroup skips the item
    if (!skip) {
    // the item's K/V range (all four waves walk it; rows past their own
    // causal limit are masked)
    const int last_item_tok = min(n - 1, (row0_item + kPrefillRows - 1) / G);
    const int kv_end = L - n_all + last_item_tok + 1;
    const int nstages = (kv_end + kStageTok - 1) / kStageTok;
    const int row0 = row0_item + 16 * NQ * wv;  // this wave's rows

    uint4 qv[NQ][KS];
    int pos_c[NQ], pos_lo[NQ];
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      const int rc = row0 + 16 * x + c;
      const int ic = rc / G, hh = rc % G;
      const bool valid = ic < n;
      pos_c[x] = L - n_all + ic;
      pos_lo[x] = __builtin_amdgcn_readfirstlane(L - n_all + (row0 + 16 * x) / G);  // the tile's smallest causal limit
      const uint16_t* qp =
          a.q + ((int64_t)(q0 + (valid ? ic : 0)) * H + (int64_t)g * G + (valid ? hh : 0)) * D + 8 * r;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * s);
        if (!valid) v = make_uint4(0, 0, 0, 0);
        qv[x][s] = v;
      }
    }
    // A thread moves, per stage, K chunks tid + kThreads*m (token index / CPR,
    // chunk index % CPR), and the V values of lane column group vc for the
    // four tokens 16*vu + 4*vr + i of unit vu.  Tokens past kv_end are read as
    // the last token (they are masked).
    const int vu = tid >> 6, vr = (tid >> 4) & 3, vc = tid & 15;
    auto tok_of = [&](int m) { return m < kKPer ? (tid + kThreads * m) / CPR : 16 * vu + 4 * vr + (m - kKPer); };
    auto slots_of = [&](int st, int32_t (&sl)[kPer]) {
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        int t = kStageTok * st + tok_of(m);
        t = t < kv_end ? t : kv_end - 1;
        if constexpr (OFF32) sl[m] = ld_at<int32_t>(a.kv_indices, (uint32_t)(kv0 + t) * 4u);
        else sl[m] = a.kv_indices[kv0 + t];
      }
    };
    struct Staged {
      uint4 k[kKPer];
      VPiece<VE> v[4];
    };
    auto fetch = [&](const int32_t (&sl)[kPer], Staged& d) {
      if constexpr (OFF32) {
        const uint16_t* kb = a.k_layer + g * D;  // wave-uniform bases
        const uint16_t* vb = a.v_layer + g * D;
        const uint32_t row = (uint32_t)kv_stride * 2u;  // bytes per slot
#pragma unroll
        for (int m = 0; m < kKPer; ++m) {
          const int ch = (tid + kThreads * m) % CPR;
          d.k[m] = ld_at<uint4>(kb, (uint32_t)sl[m] * row + 16u * ch);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          d.v[i].load(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(vb) +
                                                        ((uint32_t)sl[kKPer + i] * row + 2u * VE * vc)));
      } else {
#pragma unroll
        for (int m = 0; m < kKPer; ++m) {
          const int ch = (tid + kThreads * m) % CPR;
          d.k[m] = *reinterpret_cast<const uint4*>(a.k_layer + (int64_t)sl[m] * kv_stride + (int64_t)g * D + 8 * ch);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          d.v[i].load(a.v_layer + (int64_t)sl[kKPer + i] * kv_stride + (int64_t)g * D + VE * vc);
      }
    };
    auto stage_to_lds = [&](int buf, const Staged& d) {
#pragma unroll
      for (int m = 0; m < kKPer; ++m) {
        const int idx = tid + kThreads * m;
        sK[buf][(idx / CPR) * RS + ((idx % CPR) ^ ((idx / CPR) & (CPR - 1)))] = d.k[m];
      }
      // element e of tokens (4vr, 4vr+1) and (4vr+2, 4vr+3), paired by byte permutes
      uint2* vt = reinterpret_cast<uint2*>(sVt[buf]);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int dw = e >> 1;
        const uint2 w = make_uint2(__builtin_amdgcn_perm(d.v[1].dw(dw), d.v[0].dw(dw), sel),
                                   __builtin_amdgcn_perm(d.v[3].dw(dw), d.v[2].dw(dw), sel));
        vt[(((vu >> 1) * VE + e) * 64 + 16 * vr + vc) * 2 + (vu & 1)] = w;
      }
    };

    f32x4_t acc[NQ][VE];
    float mref[NQ], lsum[NQ];
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[x][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      mref[x] = -INFINITY;
      lsum[x] = 0.f;
    }

    // One 64-token stage (LDS buffer buf, tokens 64*st ...): the scores of its
    // four 16-token units for both tiles, one wave-uniform check whether a
    // row's reference max must move, then p = exp2(s - mref) and p.V two
    // units at a time.  p.V runs on the 16x16x32 MFMA: lane (r, c) holds p of
    // query row c for tokens 4r..4r+3 of the first unit and of the second in
    // its eight k slots, and the V operand lists the same tokens in the same
    // order, so the k order is a permutation that the sum does not see.  Rows
    // of the stage past kv_end hold copies of the last token (the staging
    // clamps them) and are masked, so a short last stage needs no branch.
    auto compute_stage = [&](int buf, int st) {
      f32x4_t t[4][NQ];  // raw scores (masked ones -inf)
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        uint4 kk[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) kk[s] = sK[buf][(16 * uu + c) * RS + ((r + 4 * s) ^ ((16 * uu + c) & (CPR - 1)))];  // token c of unit uu
#pragma unroll
        for (int x = 0; x < NQ; ++x) t[uu][x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int x = 0; x < NQ; ++x)
            t[uu][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[s]),
                                                               __builtin_bit_cast(bf16x8_t, qv[x][s]), t[uu][x], 0,
                                                               0, 0);
      }
      // A stage wholly inside the item's range and below both tiles' causal
      // diagonals needs no mask (the common case).
      const int last_tok = kStageTok * st + kStageTok - 1;
      bool full = last_tok < kv_end;
#pragma unroll
      for (int x = 0; x < NQ; ++x) full = full && last_tok <= pos_lo[x];
      // (t stays in raw score units: the scale is applied in the max test and
      // folded into the exponent)
      if (!full) {
#pragma unroll
        for (int uu = 0; uu < 4; ++uu)
#pragma unroll
          for (int x = 0; x < NQ; ++x)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tok = kStageTok * st + 16 * uu + 4 * r + i;
              if (!(tok <= pos_c[x] && tok < kv_end)) t[uu][x][i] = -INFINITY;
            }
      }
      bool need[NQ];
#pragma unroll
      for (int x = 0; x < NQ; ++x) {
        float mx = -INFINITY;
#pragma unroll
        for (int uu = 0; uu < 4; ++uu)
          mx = fmaxf(mx, fmaxf(fmaxf(t[uu][x][0], t[uu][x][1]), fmaxf(t[uu][x][2], t[uu][x][3])));
        need[x] = mx * a.scale_log2 > mref[x] + kSlack;
      }
      bool any = false;
#pragma unroll
      for (int x = 0; x < NQ; ++x) any |= need[x];
      if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
        for (int x = 0; x < NQ; ++x) {
          if (!__builtin_amdgcn_ballot_w64(need[x])) continue;
          float cm = -INFINITY;
#pragma unroll
          for (int uu = 0; uu < 4; ++uu)
            cm = fmaxf(cm, fmaxf(fmaxf(t[uu][x][0], t[uu][x][1]), fmaxf(t[uu][x][2], t[uu][x][3])));
          cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
          cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
          const float mnew = fmaxf(mref[x], cm * a.scale_log2);
          const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref[x] - mnew);
          lsum[x] *= alpha;
          mref[x] = mnew;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float ar = __shfl(alpha, 4 * r + jj, 64);
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[x][e][jj] *= ar;
          }
        }
      }
      // p for every unit and tile, packed to bf16 (the scores die here).
      // mref is finite here: token 0 is visible to every row, so the first
      // stage set it, and a masked score gives exp2(-inf) = 0.
      bf16x4_t pk[4][NQ];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)
#pragma unroll
        for (int x = 0; x < NQ; ++x)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(t[uu][x][i], a.scale_log2, -mref[x]));
            lsum[x] += p;
            pk[uu][x][i] = (__bf16)p;
          }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        bf16x8_t pa[NQ];
#pragma unroll
        for (int x = 0; x < NQ; ++x)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pa[x][i] = pk[2 * pr][x][i];
            pa[x][4 + i] = pk[2 * pr + 1][x][i];
          }
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const uint4 b = sVt[buf][(pr * VE + e) * 64 + lane];
#pragma unroll
          for (int x = 0; x < NQ; ++x)
            acc[x][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[x], __builtin_bit_cast(bf16x8_t, b), acc[x][e], 0,
                                                                0, 0);
        }
      }
    };

    // ---- pipeline over 64-token stages ----
    __syncthreads();  // the previous item's last compute is done with the buffers
    int32_t sl_next[kPer];
    {
      int32_t sl0[kPer];
      Staged v0;
      slots_of(0, sl0);
      fetch(sl0, v0);
      stage_to_lds(0, v0);
      slots_of(nstages > 1 ? 1 : 0, sl_next);
    }
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
      int32_t sl_after[kPer];
      slots_of(st + 2 < nstages ? st + 2 : nstages - 1, sl_after);
      Staged vnext;
      fetch(sl_next, vnext);
      compute_stage(st & 1, st);
      if (st + 1 < nstages) stage_to_lds((st + 1) & 1, vnext);
#pragma unroll
      for (int m = 0; m < kPer; ++m) sl_next[m] = sl_after[m];
      __syncthreads();
    }

    // ---- finalize ----
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      float l = lsum[x] + __shfl_xor(lsum[x], 16, 64);
      l += __shfl_xor(l, 32, 64);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = 4 * r + jj;
        const float lc = __shfl(l, col, 64);
        const int rc = row0 + 16 * x + col;
        const int i_tok = rc / G, h_in = rc % G;
        if (i_tok < n) {
          const float inv = 1.0f / lc;
          uint16_t* dst = a.out + ((int64_t)(q0 + i_tok) * H + (int64_t)g * G + h_in) * D + VE * c;
          __bf16 ob[VE];
#pragma unroll
          for (int e = 0; e < VE; ++e) ob[e] = (__bf16)(acc[x][e][jj] * inv);
          if constexpr (VE == 8) *reinterpret_cast<uint4*>(dst) = __builtin_bit_cast(uint4, ob);
          else *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, ob);
        }
      }
    }
    }  // !skip
    // ---- next item ----
    if (tid == 0) s_claim = kc;
    __syncthreads();
    kc = s_claim;
    __syncthreads();  // s_claim is rewritten by the next item
    item = W + kc;
    if (item >= total_items && tid == 0 && kc == last_claim)
      __hip_atomic_store(a.claim, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(kWavesTotal / kWaves), block(kThreads);
  if (head_dim == 64) {
    if (a.off32) hipLaunchKernelGGL((prefill_lds_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((prefill_lds_kernel<64, false>), grid, block, 0, stream, a);
  } else {
    if (a.off32) hipLaunchKernelGGL((prefill_lds_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((prefill_lds_kernel<128, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pd
