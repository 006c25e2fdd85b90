// Split-KV paged decode attention for gfx950 (CDNA4).
//
// AstrAI commit 0b661bae (workspace.py view): the decode attention kernel
// writes per-split partial outputs and (max, log-sum) statistics into the
// preallocated decode_o_part / decode_ml_part buffers, and a merge produces
// decode_out.  The partition and everything below are this kernel's own design.
//
// Work plan.  The kv heads are bundled in teams of T = gcd(n_kv_heads, 4)
// heads, and the launch's 2048 waves in teams of T waves (within one
// workgroup).  The bundle rows (request b, bundle gs) are laid end to end,
// request major, each as its P_b = ceil(L_b / page_size) pages.  With S >= 2
// splits the page sequence is cut into chunks of
//     Qp = max(ceil(TP / C), ceil(P_max / (S - 1)), 1)
// pages (C = 2048 / T chunks, TP = total pages of all bundle rows), and team
// t processes chunk t: a contiguous run of pages that may end one bundle row
// and start the next; wave i of the team reads kv head T*gs + i of those
// pages, so a team reads T contiguous head rows of every token together.
// Split j of a row (b, g) is its bundle row's intersection with the j-th
// chunk touching it, so a row has at most S splits and every wave carries
// the same number of pages: the work is balanced across waves, CUs and XCDs
// whatever the length mix.  With S = 1 rows are not split: team t takes
// bundle rows t, t + C, ...
//
// Per wave (no barriers: the waves of a team share only the plan; each wave
// has its own LDS rows for re-laying out K), the pages are consumed as
// 16-token units (a page, or a 16-token piece of a larger page) in a software
// pipeline that crosses row boundaries: the slots of unit n+4 are requested
// while unit n is computed, and its K and V rows and its row's q two units
// before they are needed, so a new row costs no exposed latency.
//
// Per unit, with lane l = 16*r + c:
//   scores  S[token][head] = K[16 x D] . Q^T[D x 16] on v_mfma_f32_16x16x32_bf16
//           (D/32 steps).  K rows are loaded whole like V (lane l: chunk c of
//           token 4r+i, four whole rows per instruction) and pass through the
//           wave's LDS rows into the A-operand layout (lane l: token c, 16-byte
//           chunks at byte 16*r + 64*s); loading that layout directly reads 64
//           bytes per row per instruction, which gathers slower.  The B operand
//           is q of the G heads of the row, replicated over the 16 columns
//           (column c holds head c % GP), assembled by cross-lane permutes from
//           one copy of the row's q.  Lane l receives tokens 4r+i, head
//           column c.
//   p       exp2(score * scale*log2(e) - mref): a per-head reference max that
//           is only raised when a score passes it by more than kSlack (rare),
//           so the accumulator rescale is off the common path; the exact max
//           is tracked for the (m, ln l) output and l sums p in fp32.
//   p.V     v_mfma_f32_16x16x16_bf16 with A = lane l's four p rounded to bf16
//           (A[head c][token 4r+i], exactly where the score MFMA left them)
//           and B = element e of the four V rows the lane loaded (lane l:
//           token 4r+i, 16-byte chunk c, whole rows per instruction), packed
//           pairwise with two byte permutes.  D/16 accumulators hold
//           O[head][(D/16)*n + e].
// At the end of a row segment the wave reduces its row groups with
// shuffles, normalises, and writes the split's partial for the G heads.
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kSlack = 8.0f;  // log2 units: p <= 256 before a rescale
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

// One 16-token unit in flight: K (A operand), V rows, and the q of its row
// (loaded per unit so a row change needs no extra step).  The score MFMA's
// B operand repeats the row's GP query heads over its 16 columns, so a
// direct load would move 16/GP copies of each q byte through the vector
// memory pipe with every unit.  Instead the row's distinct q bytes (GP heads
// x D bf16, QCH 16-byte chunks) are read once, chunk 64j + l by lane l in
// load j, and the operand is assembled with cross-lane permutes (QPACK).
// With 16 heads there is no duplication to remove and each lane loads its
// operand directly.
template <int D, int GP>
struct Tile {
  static constexpr int KS = D / 32;
  static constexpr int VE = D / 16;
  static constexpr int CPH = D / 8;               // 16-byte chunks per head row
  static constexpr int QCH = GP * CPH;            // distinct q chunks of a row
  static constexpr int NQL = (QCH + 63) / 64;     // q loads per lane when packed
  static constexpr bool QPACK = NQL < KS;
  VChunk<VE> k[4];  // like v: lane (r, c) holds chunk c of token 4r + i
  VChunk<VE> v[4];
  uint4 q[QPACK ? NQL : KS];
};

// Wave-uniform description of a unit, plus the lane's slot.
struct Unit {
  int valid;   // 0 past the end of the wave's work
  int first;   // first unit of a row segment: reset the running state
  int last;    // last unit of a row segment: write the split
  int row_end; // the segment ends the row: splits after it are empty
  int ntok;    // valid tokens in the unit (lanes c < ntok)
  int newtok;  // index in the unit of the row's newest token (position L - 1), else -1
  int fresh_lo; // tokens 4r+i >= fresh_lo of the unit resolve to position L - 1 (the
                // newest token itself, or padding lanes that read it): 16 = none
  int b, g, j;   // g: the wave's kv head
  int32_t slot;  // per lane: slot of token c (a real row of the request)
};

// Walks this wave's pages in order and describes one unit per call.
struct Producer {
  // launch constants (Hs = bundle rows per request, nch = chunks, w = team)
  int B, Hs, ps, ut, upp, S, w, row_mode, nch, team, member;
  int64_t Qp, p1;
  const int32_t* kv_indptr;
  const int32_t* page_indptr;
  const int32_t* kv_indices;
  // current row segment (g = bundle index)
  int done, b, g, j;
  int32_t start, L, P;
  int64_t G;      // global page index of the row's first page
  int lp, piece;  // next unit: page within the row, 16-token piece of the page
  int lp_end;     // end page (exclusive) of the segment
  int seg_first;

  __device__ int pages_of(int bb) const { return page_indptr[bb + 1] - page_indptr[bb]; }

  __device__ void open_row() {
    start = kv_indptr[b];
    L = kv_indptr[b + 1] - start;
    P = pages_of(b);
  }

  // Row mode (S = 1): bundle rows w, w + nch, ...; chunk mode: rows after (b, g).
  __device__ void next_segment() {
    if (row_mode) {
      int r = b * Hs + g + nch;
      for (;;) {
        if (r >= B * Hs) { done = 1; return; }
        b = r / Hs;
        g = r % Hs;
        if (pages_of(b) > 0) break;
        r += nch;
      }
      open_row();
      lp = 0; piece = 0; lp_end = P; j = 0; seg_first = 1;
      return;
    }
    if (lp_end < P) { done = 1; return; }  // the chunk ended inside this row
    // Candidate next row; b and g only change once it is known to exist, so
    // the (masked) loads issued after the end still address real rows.
    int nb = b, ng = g + 1;
    if (ng == Hs) {
      ng = 0;
      ++nb;
      while (nb < B && pages_of(nb) == 0) ++nb;
      if (nb >= B) { done = 1; return; }
    }
    const int64_t nG = (int64_t)Hs * page_indptr[nb] + (int64_t)ng * pages_of(nb);
    if (nG >= p1) { done = 1; return; }
    b = nb;
    g = ng;
    open_row();
    G = nG;
    lp = 0; piece = 0;
    lp_end = (int)min((int64_t)P, p1 - G);
    j = (int)(w - G / Qp);
    seg_first = 1;
  }

  __device__ Unit next(int c) {
    Unit u;
    u.valid = !done;
    u.b = b; u.g = g * team + member; u.j = j;
    u.first = seg_first;
    const int tok_lo = lp * ps + piece * ut;
    const int tok_hi = min(lp * ps + min((piece + 1) * ut, ps), L);
    u.ntok = done ? 0 : tok_hi - tok_lo;
    // (a trailing 16-token piece of a page past the row's end holds no token)
    u.newtok = (!done && tok_lo <= L - 1 && tok_hi == L) ? L - 1 - tok_lo : -1;
    // Lanes past the unit's tokens (and every lane past the end of the work)
    // read a real token of the row instead; their scores are masked.
    const int t_last = (!done && u.ntok > 0) ? tok_hi - 1 : L - 1;
    // Which lanes end up on position L - 1: from the newest token on in the
    // unit that holds it (the padding lanes after it read it too), and every
    // lane of a trailing piece past the row's end (page_size > 16).
    u.fresh_lo = done ? 16 : u.newtok >= 0 ? u.newtok : u.ntok <= 0 ? 0 : 16;
    const int t = (c < u.ntok) ? tok_lo + c : t_last;
    u.slot = kv_indices[start + t];
    u.last = 0;
    u.row_end = 0;
    if (!done) {
      seg_first = 0;
      if (++piece == upp) { piece = 0; ++lp; }
      if (lp == lp_end && piece == 0) {
        u.last = 1;
        u.row_end = lp_end == P;
        next_segment();  // the following units belong to the next segment
      }
    }
    return u;
  }
};

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

// With APPEND every lane that resolves to the row's newest token reads it from
// the new-row buffer: the store still holds that slot's old contents (possibly
// NaN) until this launch writes them, and a masked lane's p = 0 would still
// turn a NaN V element into a NaN accumulator in the p.V MFMA.
template <int D, int GP, bool APPEND>
__device__ __forceinline__ Tile<D, GP> load_tile(const AttnArgs& a, const Unit& u, int r, int c) {
  using TT = Tile<D, GP>;
  TT t;
  constexpr int KS = TT::KS, VE = TT::VE;
  const int64_t stride = (int64_t)a.n_kv_heads * D;
  // K and V rows are read whole, four tokens per instruction (lane (r, c):
  // chunk c of token 4r + i), and exactly once: streaming (non-temporal)
  // loads keep them from evicting the q rows and the index lists.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t sv = __shfl(u.slot, 4 * r + i, 64);
    const int64_t off = (int64_t)sv * stride + (int64_t)u.g * D + VE * c;
    const uint16_t* kp = a.k_layer + off;
    const uint16_t* vp = a.v_layer + off;
    if constexpr (APPEND) {
      const int64_t noff = ((int64_t)u.b * a.n_kv_heads + u.g) * D + VE * c;
      const bool fresh = 4 * r + i >= u.fresh_lo;
      kp = fresh ? a.k_new + noff : kp;
      vp = fresh ? a.v_new + noff : vp;
    }
    if constexpr (VE == 8) {
      t.k[i].u = ld_stream(reinterpret_cast<const uint4*>(kp));
      t.v[i].u = ld_stream(reinterpret_cast<const uint4*>(vp));
    } else {
      t.k[i].u = ld_stream(reinterpret_cast<const uint2*>(kp));
      t.v[i].u = ld_stream(reinterpret_cast<const uint2*>(vp));
    }
  }
  // q of the row (zeros for heads past the group); the loads are unconditional.
  const uint16_t* qrow = a.q + ((int64_t)u.b * a.n_heads + (int64_t)u.g * a.group) * D;
  if constexpr (TT::QPACK) {
#pragma unroll
    for (int j = 0; j < TT::NQL; ++j) {
      const int idx = 64 * j + 16 * r + c;  // chunk of this lane: head idx / CPH, chunk idx % CPH
      const bool real = idx < TT::QCH && idx / TT::CPH < a.group;
      uint4 v = *reinterpret_cast<const uint4*>(qrow + 8 * (real ? idx : 0));
      if (!real) v = make_uint4(0, 0, 0, 0);
      t.q[j] = v;
    }
  } else {
    // head column c, chunks r + 4s: the operand itself
    const int hq = c % GP;
    const bool real = hq < a.group;
    const uint16_t* qp = qrow + (int64_t)(real ? hq : 0) * D + 8 * r;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * s);
      if (!real) v = make_uint4(0, 0, 0, 0);
      t.q[s] = v;
    }
  }
  return t;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// The score MFMA's B operand for step s: lane (r, c) holds chunk r + 4s of
// head c % GP.  In the packed layout that chunk sits in lane idx % 64 of
// load idx / 64, idx = (c % GP) * CPH + 4s + r.
template <int D, int GP>
__device__ __forceinline__ uint4 q_operand(const Tile<D, GP>& T, int s, int r, int c) {
  using TT = Tile<D, GP>;
  if constexpr (TT::QPACK) {
    const int idx = (c % GP) * TT::CPH + 4 * s + r;
    const int addr = (idx & 63) * 4;  // ds_bpermute takes a byte address
    const int j = idx >> 6;
    uint32_t w4[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t val = 0;
#pragma unroll
      for (int jj = 0; jj < TT::NQL; ++jj) {
        const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)dword_of(T.q[jj], w));
        val = (TT::NQL == 1 || j == jj) ? x : val;
      }
      w4[w] = val;
    }
    return make_uint4(w4[0], w4[1], w4[2], w4[3]);
  } else {
    return T.q[s];
  }
}

template <int D, int GP, bool APPEND>
__global__ void __launch_bounds__(kThreads, 2)
split_attn_kernel(AttnArgs a) {
  using TT = Tile<D, GP>;
  constexpr int KS = TT::KS, VE = TT::VE;
  constexpr int kRowB = 2 * D + 16;  // LDS bytes per K row (16 bytes of padding against bank conflicts)
  __shared__ __attribute__((aligned(16))) char k_lds[kWaves * 16 * kRowB];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  char* const kl = k_lds + wave * 16 * kRowB;
  // Wave index, team (= chunk) index and head within the team: wave-uniform,
  // so the plan lives in SGPRs.
  const int T = a.team;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wave);
  const int tm = __builtin_amdgcn_readfirstlane(blockIdx.x * (kWaves / T) + wave / T);
  const int member = __builtin_amdgcn_readfirstlane(wave % T);
  const int r = lane >> 4, c = lane & 15;
  const int Hkv = a.n_kv_heads, S = a.num_splits, H = a.n_heads;
  const int Bk = a.batch;  // launch batch: bounds the per-lane index loads below
  const int B = active_batch(a.active, a.batch);
  const int Hs = Hkv / T, nch = kSplitChunks / T;

  // ---- this wave's first row segment ----
  // All plan inputs are fetched in one round trip: the max-pages meta word,
  // and (for the first 64 requests) page_indptr and kv_indptr, held one per
  // lane.  The total page count is page_indptr[B] itself, so the chunks never
  // reach past the requests this launch walks.
  Producer pr;
  pr.B = B; pr.Hs = Hs; pr.ps = a.page_size; pr.S = S; pr.w = tm;
  pr.nch = nch; pr.team = T; pr.member = member;
  pr.ut = a.page_size < 16 ? a.page_size : 16;
  pr.upp = (a.page_size + pr.ut - 1) / pr.ut;
  pr.kv_indptr = a.kv_indptr; pr.page_indptr = a.page_indptr; pr.kv_indices = a.kv_indices;
  pr.done = 0;
  const bool row_mode = S == 1;
  pr.row_mode = row_mode;
  const int i_lane = lane <= Bk ? lane : Bk;  // entries past B are never used
  const int32_t pi_lane = a.page_indptr[i_lane];
  const int32_t ki_lane = a.kv_indptr[i_lane];
  // page_indptr / kv_indptr of request bb, a wave-uniform index (read from
  // lane bb's register when bb < 64)
  auto pi_of = [&](int bb) { return bb < 64 ? __builtin_amdgcn_readlane(pi_lane, bb) : a.page_indptr[bb]; };
  auto ki_of = [&](int bb) { return bb < 64 ? __builtin_amdgcn_readlane(ki_lane, bb) : a.kv_indptr[bb]; };
  const int32_t total_pages = __builtin_amdgcn_readfirstlane(pi_of(B));
  const int32_t max_pages = a.meta[kMetaMaxPages];
  const int64_t TP = (int64_t)Hs * total_pages;
  bool active = true;
  if (row_mode) {
    pr.Qp = 1; pr.p1 = 0;
    int rr = tm;  // first non-empty bundle row among tm, tm + nch, ...
    for (;;) {
      if (rr >= B * Hs) { active = false; break; }
      const int bb = rr / Hs;
      if (pi_of(bb + 1) - pi_of(bb) > 0) break;
      rr += nch;
    }
    if (active) {
      pr.b = __builtin_amdgcn_readfirstlane(rr / Hs);
      pr.g = __builtin_amdgcn_readfirstlane(rr % Hs);
      pr.start = __builtin_amdgcn_readfirstlane(ki_of(pr.b));
      pr.L = __builtin_amdgcn_readfirstlane(ki_of(pr.b + 1)) - pr.start;
      pr.P = __builtin_amdgcn_readfirstlane(pi_of(pr.b + 1) - pi_of(pr.b));
      pr.lp = 0; pr.piece = 0; pr.lp_end = pr.P; pr.j = 0; pr.seg_first = 1;
    }
  } else {
    int64_t qp = (TP + nch - 1) / nch;
    const int64_t qs = (max_pages + S - 2) / (S - 1);
    qp = qp > qs ? qp : qs;
    qp = qp < 1 ? 1 : qp;
    const int64_t p0 = (int64_t)tm * qp;
    if (p0 >= TP) {
      active = false;
    } else {
      pr.Qp = qp;
      pr.p1 = p0 + qp < TP ? p0 + qp : TP;
      // Request holding global page p0: the number of entries of
      // Hs * page_indptr[0..B] that are <= p0, minus one.
      int cnt = __popcll(__builtin_amdgcn_ballot_w64(lane <= B && (int64_t)Hs * pi_lane <= p0));
      for (int i0 = 64; i0 <= B; i0 += 64) {
        const int i = i0 + lane;
        const bool le = i <= B && (int64_t)Hs * a.page_indptr[i] <= p0;
        cnt += __popcll(__builtin_amdgcn_ballot_w64(le));
      }
      pr.b = cnt - 1;
      const int32_t pib = __builtin_amdgcn_readfirstlane(pi_of(pr.b));
      pr.P = __builtin_amdgcn_readfirstlane(pi_of(pr.b + 1)) - pib;
      pr.start = __builtin_amdgcn_readfirstlane(ki_of(pr.b));
      pr.L = __builtin_amdgcn_readfirstlane(ki_of(pr.b + 1)) - pr.start;
      const int64_t off = p0 - (int64_t)Hs * pib;
      pr.g = (int)(off / pr.P);
      pr.G = (int64_t)Hs * pib + (int64_t)pr.g * pr.P;
      pr.lp = (int)(off % pr.P);
      pr.piece = 0;
      pr.lp_end = (int)min((int64_t)pr.P, pr.p1 - pr.G);
      pr.j = (int)(tm - pr.G / qp);
      pr.seg_first = 1;
    }
  }

  // Requests with no tokens: every split of every head is empty (done after
  // the plan's loads are in flight; independent of them).
  auto mark_empty_requests = [&]() {
    for (int b = w; b < B; b += kSplitChunks) {
      if (ki_of(b + 1) == ki_of(b)) {
        for (int e = lane; e < H * S; e += 64) {
          const int64_t row = ((int64_t)b * H + e / S) * a.max_splits + e % S;
          a.ml_part[row * 2 + 0] = -INFINITY;
          a.ml_part[row * 2 + 1] = -INFINITY;
        }
      }
    }
  };
  if (!active) {
    mark_empty_requests();
    return;
  }

  // ---- running state of the current segment ----
  f32x4_t acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lsum = 0.f, mtrue = -INFINITY;

  auto reset = [&]() {
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mref = -INFINITY; lsum = 0.f; mtrue = -INFINITY;
  };

  auto finalize = [&](const Unit& u) {
    if (u.j >= S) return;  // cannot happen: the plan keeps j < S
    // Per head column: sum / max over the four row groups (tokens).
    float l = lsum + __shfl_xor(lsum, 16, 64);
    l += __shfl_xor(l, 32, 64);
    float mt = fmaxf(mtrue, __shfl_xor(mtrue, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const int64_t head0 = (int64_t)u.b * H + (int64_t)u.g * a.group;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int h = 4 * r + jj;  // accumulator row = head column h
      const float lh = __shfl(l, h, 64);
      if (h < GP && h < a.group) {
        const float inv = 1.0f / lh;
        float* dst = a.o_part + ((head0 + h) * a.max_splits + u.j) * D + VE * c;
        if constexpr (VE == 8) {
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc[0][jj] * inv, acc[1][jj] * inv, acc[2][jj] * inv, acc[3][jj] * inv);
          *reinterpret_cast<float4*>(dst + 4) =
              make_float4(acc[4][jj] * inv, acc[5][jj] * inv, acc[6][jj] * inv, acc[7][jj] * inv);
        } else {
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc[0][jj] * inv, acc[1][jj] * inv, acc[2][jj] * inv, acc[3][jj] * inv);
        }
      }
    }
    if (r == 0 && c < GP && c < a.group) {
      // natural-log units: m = mt * ln2;  ln l_true = ln l + (mref - mt) * ln2
      float* ml = a.ml_part + ((head0 + c) * a.max_splits + u.j) * 2;
      ml[0] = mt * kLn2;
      ml[1] = __logf(l) + (mref - mt) * kLn2;
    }
    if (u.row_end) {
      // Splits after the row's last one are empty.
      const int n_empty = S - 1 - u.j;
      for (int e = lane; e < a.group * n_empty; e += 64) {
        float* ml = a.ml_part + ((head0 + e / n_empty) * a.max_splits + u.j + 1 + e % n_empty) * 2;
        ml[0] = -INFINITY;
        ml[1] = -INFINITY;
      }
    }
  };

  auto compute = [&](const TT& T, const Unit& u) {
    if (u.first) reset();
    if (APPEND && u.newtok >= 0) {
      // Fused KV append: this unit holds the row's newest token, which the
      // tile took from the new-row buffer (nobody reads its slot in the store
      // during this launch).  The lanes that hold its K and V chunks store
      // them at that slot, straight from the tile's registers.
      const int64_t row = (__shfl(u.slot, u.newtok, 64) * (int64_t)a.n_kv_heads + u.g) * D;
      if (r == (u.newtok >> 2)) {  // row group of token 4r + i: K and V chunk VE*c
        const int i = u.newtok & 3;
        auto pick = [&](uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
          return i == 0 ? x0 : i == 1 ? x1 : i == 2 ? x2 : x3;
        };
        auto put = [&](uint16_t* d, const VChunk<VE> (&x)[4]) {
          if constexpr (VE == 8) {
            *reinterpret_cast<uint4*>(d) = make_uint4(
                pick(x[0].u.x, x[1].u.x, x[2].u.x, x[3].u.x), pick(x[0].u.y, x[1].u.y, x[2].u.y, x[3].u.y),
                pick(x[0].u.z, x[1].u.z, x[2].u.z, x[3].u.z), pick(x[0].u.w, x[1].u.w, x[2].u.w, x[3].u.w));
          } else {
            *reinterpret_cast<uint2*>(d) = make_uint2(pick(x[0].u.x, x[1].u.x, x[2].u.x, x[3].u.x),
                                                      pick(x[0].u.y, x[1].u.y, x[2].u.y, x[3].u.y));
          }
        };
        put(a.k_dst + row + VE * c, T.k);
        put(a.v_dst + row + VE * c, T.v);
      }
    }
    // K rows through this wave's LDS rows: written as loaded (lane (r, c):
    // token 4r + i, chunk c), read back as the score MFMA's A operand (lane
    // (r, c): token c, 16-byte chunks r + 4s).  LDS operations of one wave
    // complete in order; the wave barrier keeps the compiler from moving the
    // reads above the writes.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      char* dst = kl + (4 * r + i) * kRowB + c * (VE * 2);
      if constexpr (VE == 8) *reinterpret_cast<uint4*>(dst) = T.k[i].u;
      else *reinterpret_cast<uint2*>(dst) = T.k[i].u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint4 kk[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) kk[s] = *reinterpret_cast<const uint4*>(kl + c * kRowB + (r + 4 * s) * 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[s]),
                                                   __builtin_bit_cast(bf16x8_t, q_operand(T, s, r, c)), sc, 0, 0,
                                                   0);
    float t[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[i] = (4 * r + i < u.ntok) ? sc[i] * a.scale_log2 : -INFINITY;
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
    bf16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mtrue = fmaxf(mtrue, t[i]);
      const float p = __builtin_amdgcn_exp2f(t[i] - mref);
      lsum += p;
      pb[i] = (__bf16)p;
    }
    const i16x4_t pa = __builtin_bit_cast(i16x4_t, pb);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2_t bv;
      bv[0] = __builtin_amdgcn_perm(T.v[1].dw(e >> 1), T.v[0].dw(e >> 1), sel);
      bv[1] = __builtin_amdgcn_perm(T.v[3].dw(e >> 1), T.v[2].dw(e >> 1), sel);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(i16x4_t, bv), acc[e], 0, 0, 0);
    }
    if (u.last) finalize(u);
  };

  // ---- pipeline: units A, B computed alternately; C, D have slots in flight ----
  Unit uA = pr.next(c);
  Unit uB = pr.next(c);
  Unit uC = pr.next(c);
  Unit uD = pr.next(c);
  TT TA = load_tile<D, GP, APPEND>(a, uA, r, c);
  TT TB = load_tile<D, GP, APPEND>(a, uB, r, c);
  int nunits = 0;
  // The two workgroups sharing a CU: the wave arbiter favours the older one,
  // which then finishes ~20% earlier.  The later-dispatched workgroup (second
  // half of the grid) raises its priority for the first half of its units and
  // the earlier one for the second half, so each is favoured for half its
  // life.  Priority only changes timing, never results.
  const bool young = blockIdx.x >= gridDim.x / 2;
  const int half = (int)((row_mode ? 1 : pr.Qp) * pr.upp / 2);
  if (young) __builtin_amdgcn_s_setprio(1);
  while (uA.valid) {
    compute(TA, uA);
    if (nunits == half) {
      if (young) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(1);
    }
    ++nunits;
    TA = load_tile<D, GP, APPEND>(a, uC, r, c);
    uA = uC;
    uC = pr.next(c);
    if (!uB.valid) break;
    compute(TB, uB);
    ++nunits;
    TB = load_tile<D, GP, APPEND>(a, uD, r, c);
    uB = uD;
    uD = pr.next(c);
  }
  mark_empty_requests();
}

template <int D, int GP>
hipError_t launch_dg(const AttnArgs& a, hipStream_t stream) {
  if (a.k_new != nullptr)
    hipLaunchKernelGGL((split_attn_kernel<D, GP, true>), dim3(kSplitChunks / kWaves), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((split_attn_kernel<D, GP, false>), dim3(kSplitChunks / kWaves), dim3(kThreads), 0, stream, a);
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

hipError_t launch_attn(const AttnArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace pd
