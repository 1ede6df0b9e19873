// Chunkwise-parallel mLSTM / retention forward for gfx950.
//
// Method (mLSTM recurrence with exponential input gate and log-space max
// stabiliser; block-diagonal memory of the "Edifice.Recurrent.XLSTMv2" page,
// "Key Improvements" items 1-2; retention of the "Edifice.Attention.RetNet"
// page, "Key Innovation" and "Multi-Scale Retention"; chunked scan with dense
// intra-chunk products as in the "Chunk" mode doc of burn-gdn2's Gdn2Mode).
//
// Per chunk of L tokens (local index j) with stabiliser m_prev at its start,
// all logarithms in base 2 inside the kernels:
//   b_j = sum_{l<=j} log sigmoid(f_l);  a_l = i_l - b_l
//   M_j = max(m_prev, max_{l<=j} a_l);  m_j = b_j + M_j
//   num_j = 2^{m_prev-M_j} S~^T q_j + sum_{l<=j} 2^{a_l-M_j} (q_j.k_l) v_l
//   den_j = 2^{m_prev-M_j} n~.q_j   + sum_{l<=j} 2^{a_l-M_j} (q_j.k_l)
//   h_j   = o_j num_j / max(|den_j + bias 2^{-m_j}|, 2^{-m_j})
//   S~   <- 2^{m_prev-M_L} S~ + sum_l 2^{a_l-M_L} k_l v_l^T;  m <- b_L + M_L
// Retention is the same with i = 1, f = gamma_h and no normaliser.
//
// Three launches on the caller's stream:
//   pass 1  every superchunk of G chunks but the last runs the state update
//           from a zero state (m = -inf): its local end state dS, dn, its log
//           scale mu and its total log decay A go to the workspace.
//   pass 2  per state element, a scan over superchunks
//           m' = max(A + m, mu); S' = 2^{A+m-m'} S + 2^{mu-m'} dS
//           leaves the start state of every superchunk in the workspace.
//   pass 3  every (batch*head, superchunk, d_v slice) work-group runs its
//           chunks sequentially from its start state: readout, intra-chunk
//           product, output, state update.
//
// Work-group: 4 waves of 64.  A work-group owns W = 4*WC columns of d_v; wave
// w owns WC of them and all d_qk/NB rows of the memory block they lie in.  The
// fp32 state slice lives in registers as MFMA accumulator tiles for the whole
// superchunk.  Its rows are stored in a permuted order (perm_row) so that the
// accumulator registers are directly the A operand of the readout MFMA.
#include "common.h"
#include "kernels.h"

namespace mlstm {

// Storage row rho (0..15) of state tile nt -> feature index within the block.
// bf16: a pair of tiles covers 32 features, lane group g gets 8g..8g+7.
// fp32: a tile covers 16 features, the i-th MFMA of a tile covers 4i..4i+3.
template <typename T>
__device__ __forceinline__ int perm_row(int nt, int rho);
template <>
__device__ __forceinline__ int perm_row<__bf16>(int nt, int rho) {
  return (nt >> 1) * 32 + (rho >> 2) * 8 + (nt & 1) * 4 + (rho & 3);
}
template <>
__device__ __forceinline__ int perm_row<float>(int nt, int rho) {
  return nt * 16 + (rho & 3) * 4 + (rho >> 2);
}

// perm_row(nt, 4*lg + i) split into a lane part (depends on lg only) and a
// wave-uniform part, so that state addresses need one lane offset.
template <typename T>
__device__ __forceinline__ int perm_row_lane(int lg) { return sizeof(T) == 2 ? lg * 8 : lg; }
template <typename T>
__device__ __forceinline__ constexpr int perm_row_uni(int nt, int i) {
  return sizeof(T) == 2 ? (nt >> 1) * 32 + (nt & 1) * 4 + i : nt * 16 + i * 4;
}

// Readout A operand (rows = columns of d_v, k = features kk*K .. +K-1 of the
// block) taken from the accumulator tiles of the state.
template <typename T, int NT, int CT>
struct StateFrag;
template <int NT, int CT>
struct StateFrag<__bf16, NT, CT> {
  __device__ __forceinline__ static bf16x8 get(const f32x4 (&st)[NT][CT], int kk, int ct) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (__bf16)st[2 * kk][ct][i];
      r[4 + i] = (__bf16)st[2 * kk + 1][ct][i];
    }
    return r;
  }
};
template <int NT, int CT>
struct StateFrag<float, NT, CT> {
  __device__ __forceinline__ static float get(const f32x4 (&st)[NT][CT], int kk, int ct) {
    return st[kk >> 2][ct][kk & 3];
  }
};

// fragment scaled by per-k weights (weights for k = base .. base+KL-1)
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 x, const float* w) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)((float)x[e] * w[e]);
  return r;
}
__device__ __forceinline__ float scale_frag(float x, const float* w) { return x * w[0]; }

template <typename T, int DQK, int NB, int WC, int NRG, int L>
struct ChunkCfg {
  static constexpr int K = Mma<T>::K;
  static constexpr int KL = Mma<T>::KL;
  static constexpr int NW = 4 * NRG;              // waves per work-group
  static constexpr int NTH = 64 * NW;             // threads per work-group
  static constexpr int DQKB = DQK / NB;           // rows of a memory block
  static constexpr int RPW = DQKB / NRG;          // state rows per wave
  static constexpr int NT = RPW / 16;             // state row tiles per wave
  static constexpr int CT = WC / 16;              // state column tiles per wave
  static constexpr int W = 4 * WC;                // d_v columns per work-group
  static constexpr int NJT = L / 16;              // 16-token tiles per chunk
  static constexpr int JPW = NJT / NRG;           // token tiles finished per wave
  static constexpr int NKL = L / K;               // token k-blocks per chunk
  static constexpr int NKQ = DQK / K;             // feature k-blocks of a head
  static constexpr int NKQB = DQKB / K;           // feature k-blocks of a block
  static constexpr int NKQR = RPW / K;            // feature k-blocks of a wave's rows
  static constexpr int NTQK = NJT * (NJT + 1) / 2;  // causal score tiles
  static constexpr int VE = 16 / (int)sizeof(T);  // elements per 16 bytes
  // Row strides (elements) of the token-major tiles: the smallest padding
  // that makes a row step move the bank by one of the given residues (mod 64
  // dwords).  Q/K (16-byte fragment reads, 16 rows) use 8 + 16i; V (only
  // transposing reads, 4 rows x 32 bytes per 16 lanes) uses 12, 28, 36, 52.
  // Both choices were the fastest in a sweep on MI355X.
  static constexpr int pad_for(int row_elems, bool v) {
    const int dw = row_elems * (int)sizeof(T) / 4;
    int best = 64;
    const int rq[4] = {8, 24, 40, 56}, rv[4] = {12, 28, 36, 52};
    for (int i = 0; i < 4; ++i) {
      const int r = v ? rv[i] : rq[i];
      const int pad = ((r - dw % 64) % 64 + 64) % 64;
      if (pad < best) best = pad;
    }
    return best * 4 / (int)sizeof(T);
  }
  static constexpr int QS = DQK + pad_for(DQK, false);  // sQ, sK
  static constexpr int VS = W + pad_for(W, true);       // sV
  static constexpr int PS = L + 16 / (int)sizeof(T);  // sP
  // staging units (16-byte loads) per chunk
  static constexpr int NQU = L * DQK / VE;
  static constexpr int NVU = L * W / VE;
  static constexpr int QIT = (NQU + NTH - 1) / NTH;
  static constexpr int VIT = (NVU + NTH - 1) / NTH;
  static_assert(DQK % NB == 0, "d_qk % nb");
  static_assert(RPW % (sizeof(T) == 2 ? 32 : 16) == 0, "state rows per wave");
  static_assert(L % K == 0 && L % 16 == 0 && L <= 64, "chunk length");
  static_assert(NJT % NRG == 0, "token tiles per row group");
  static_assert(WC % 16 == 0, "wave columns");
  static constexpr size_t lds_bytes(bool full, bool ret) {
    size_t b = 0;
    b += (size_t)L * QS * sizeof(T);             // sK
    b += (size_t)L * VS * sizeof(T);             // sV
    b += 6 * L * 4 + 16;                         // gate vectors
    if (!ret) b += DQK * 4 + (full ? 16 * DQK * sizeof(T) : 0);  // n~
    if (full) {
      b += (size_t)L * QS * sizeof(T);           // sQ
      b += (size_t)NB * L * PS * sizeof(T);      // sP
      b += (size_t)(NJT + 1) * L * 4;            // den partials
      if (NRG > 1) b += (size_t)4 * NJT * CT * 64 * 16;  // readout exchange
    }
    return b;
  }
};

// MFMA fragment along the rows of a token-major tile: lane (lr, lg) gets rows
// r0 + KL*lg + e (e < KL) of one column.
//   bf16: two transposing reads; source lane lr addresses column csrc(lr),
//         chosen by the caller so that output lane lr sees its column.
//   fp32: one element, column ccol(lr).
__device__ __forceinline__ bf16x8 frag_rows(const __bf16* tile, int RS, int r0, int lr, int csrc) {
  const __bf16* p = tile + (r0 + (lr >> 2)) * RS + csrc;
  const bf16x4 a = ds_read_tr16(p);
  const bf16x4 b = ds_read_tr16(p + 4 * RS);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = a[e];
    r[4 + e] = b[e];
  }
  return r;
}
__device__ __forceinline__ float frag_rows(const float* tile, int RS, int r0, int lr, int ccol) {
  (void)lr;
  return tile[r0 * RS + ccol];
}

// Main kernel.  FULL = true: pass 3 (readout, outputs, update).  FULL = false:
// pass 1 (update only, from a zero state).
//
// Work-group = 4 column groups x NRG row groups of waves.  Wave (cg, rg) owns
// columns [cg*WC, cg*WC+WC) of the work-group's d_v slice and state rows
// [rg*RPW, rg*RPW+RPW) of their memory block.  With NRG = 2 the readout of a
// column group is split over its two waves by rows; each wave finishes half of
// the token tiles and the two partial sums meet in LDS (sX).
// Q, K and V are staged token-major with plain 16-byte copies; the operands
// that run along tokens (K^T and V^T) are read with transposing LDS reads.
template <typename T, int DQK, int NB, int WC, int NRG, int L, bool RET, bool FULL>
__global__ __launch_bounds__(256 * NRG) void chunk_kernel(ChunkParams p) {
  using C = ChunkCfg<T, DQK, NB, WC, NRG, L>;
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int K = C::K, KL = C::KL, DQKB = C::DQKB, NT = C::NT, CT = C::CT, NW = C::NW;
  constexpr int NTH = C::NTH, RPW = C::RPW, JPW = C::JPW;
  constexpr int W = C::W, NJT = C::NJT, NKL = C::NKL, NKQ = C::NKQ, NKQB = C::NKQB, NKQR = C::NKQR;
  constexpr int VE = C::VE, QS = C::QS, VS = C::VS, PS = C::PS;
  constexpr unsigned ES = sizeof(T);
  constexpr bool XCH = FULL && NRG > 1;
  constexpr bool BF = sizeof(T) == 2;

  __shared__ __attribute__((aligned(16))) T sK[L * QS];   // K, token-major
  __shared__ __attribute__((aligned(16))) T sV[L * VS];   // V slice, token-major
  __shared__ __attribute__((aligned(16))) T sQ[FULL ? L * QS : 8];   // Q, token-major
  __shared__ __attribute__((aligned(16))) T sP[FULL ? NB * L * PS : 8];
  __shared__ __attribute__((aligned(16))) f32x4 sX[XCH ? 4 * NJT * CT * 64 : 1];
  // n~ as a 16-row A-operand tile: row 0 = bf16 hi part, row 1 = lo part,
  // rows 2..15 zero (fp32: row 0 = n~, row 1 zero)
  __shared__ __attribute__((aligned(16))) T sNh[RET || !FULL ? 8 : 16 * DQK];
  __shared__ float sNf[RET ? 4 : DQK];
  __shared__ float sA2[L], sM2[L], sRS[L], sCL[L], sBT[L], sW[L];
  __shared__ float sDenPart[FULL ? NJT * L : 4];
  __shared__ float sDenInter[FULL ? L : 4];
  __shared__ float sAlpha;

  const int tid = threadIdx.x;
  // The wave index must be known to be wave-uniform: branches on it guard
  // MFMA instructions, which do not honour a partial EXEC mask.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = w & 3, rg = w >> 2;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // Work-group coordinates.  Integer division by runtime values runs on the
  // VALU; readfirstlane keeps the results (and the buffer descriptors built
  // from them) in scalar registers, otherwise every buffer load would be
  // wrapped in a waterfall loop.
  const int BH = p.B * p.H;
  const int idx = blockIdx.x;
  const int bh = __builtin_amdgcn_readfirstlane(idx % BH);
  const int slice = __builtin_amdgcn_readfirstlane((idx / BH) % p.nslices);
  const int sc = __builtin_amdgcn_readfirstlane((idx / BH) / p.nslices);
  const int hd = __builtin_amdgcn_readfirstlane(bh % p.H);
  const int T_ = p.T, DV = p.DV, DVB = DV / NB;
  const size_t CS = (size_t)DQK * DV / NB;
  const size_t NSTATE = CS + (RET ? 0 : DQK);

  const int wcol0 = slice * W + cg * WC;  // first global d_v column of this wave
  const int blk = __builtin_amdgcn_readfirstlane(wcol0 / DVB);  // memory block of this wave
  const int wcl0 = wcol0 - blk * DVB;     // first column inside the block
  const int rrow0 = rg * RPW;             // first state row of this wave inside the block
  const int rb0 = blk * DQKB + rrow0;     // ... as a feature index of the head
  const int jt0 = rg * JPW;               // first token tile finished by this wave

  // buffer resources over this (batch, head): reads past T return zero
  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * T_ * DV, (unsigned)T_ * DV * ES);
  const auto ri = make_rsrc(RET ? nullptr : static_cast<const T*>(p.i_pre) + (size_t)bh * T_,
                            RET ? 0u : (unsigned)T_ * ES);
  const auto rf = make_rsrc(RET ? nullptr : static_cast<const T*>(p.f_pre) + (size_t)bh * T_,
                            RET ? 0u : (unsigned)T_ * ES);
  const bool has_o = FULL && p.o_pre != nullptr;
  const auto ro = make_rsrc(has_o ? static_cast<const T*>(p.o_pre) + (size_t)bh * T_ * DV : nullptr,
                            has_o ? (unsigned)T_ * DV * ES : 0u);
  T* __restrict__ gh = FULL ? static_cast<T*>(p.h) + (size_t)bh * T_ * DV : nullptr;
  const float bias = (!RET && p.bias) ? p.bias[hd] : 0.f;
  float ret_lg2 = 0.f;
  if constexpr (RET) ret_lg2 = log2f(p.ret_gamma ? p.ret_gamma[hd] : 1.f - exp2f(-5.f - (float)hd));

  const int c_begin = sc * p.G;
  const int c_end = FULL ? min(c_begin + p.G, p.NC) : c_begin + p.G;

  // Source columns of the transposing reads.  K^T (update A operand): output
  // lane lr must see feature rb0 + perm_row(nt, lr).  V^T (PV A operand and
  // update B operand): output lane lr sees column cg*WC + ct*16 + lr.
  const int kcol = BF ? rb0 + 8 * (lr & 3) : rb0;  // + perm part added per tile
  const int vcol = BF ? cg * WC + 4 * (lr & 3) : cg * WC + lr;

  // ---------------------------------------------------------------- state in
  f32x4 st[NT][CT];
  const float* Sin = nullptr;
  if (FULL && (sc > 0 || p.has_init)) Sin = p.ws_state + ((size_t)bh * p.NS + sc) * NSTATE;
  // state element (nt, ct, i) of this lane sits at soff + (uni(nt,i)*DVB + ct*16)
  const int soff = blk * DQKB * DVB + (rrow0 + perm_row_lane<T>(lg)) * DVB + wcl0 + lr;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st[nt][ct][i] = Sin ? Sin[soff + perm_row_uni<T>(nt, i) * DVB + ct * 16] : 0.f;
  // n~ in fp32 and as the hi/lo rows of the den tile
  auto put_n = [&](int r, float x) __attribute__((always_inline)) {
    sNf[r] = x;
    if constexpr (FULL) {
      const T hi = from_f32<T>(x);
      sNh[r] = hi;
      sNh[DQK + r] = from_f32<T>(x - to_f32(hi));
    }
  };
  if constexpr (!RET) {
    if constexpr (FULL)
      for (int e = tid; e < 16 * DQK; e += NTH) sNh[e] = from_f32<T>(0.f);
    __syncthreads();
    for (int r = tid; r < DQK; r += NTH) put_n(r, Sin ? Sin[CS + r] : 0.f);
  }
  if constexpr (FULL) {
    // masked (l > j) tiles of P and their den partials are never written
    for (int e = tid; e < NB * L * PS; e += NTH) sP[e] = from_f32<T>(0.f);
    for (int e = tid; e < NJT * L; e += NTH) sDenPart[e] = 0.f;
  }
  // The registers hold S^ = S~ / 2^{sig}: the per-chunk decay of the state is
  // folded into sig (a wave-uniform scalar) instead of multiplying every
  // state element; new contributions are weighted by 2^{-sig}, the readout by
  // 2^{sig}.  When sig drops below -64 the registers are rescaled once.
  float sig = 0.f;
  // stabiliser carried by wave 0 (log2 units)
  float m_prev = FULL ? p.ws_min[(size_t)bh * p.NS + sc] : -INFINITY;
  float a_total = 0.f;

  // ------------------------------------------------------ staging registers
  // All global loads are unconditional buffer loads (units past the end of a
  // staging loop reload a valid unit and are not stored).  The next chunk's
  // loads are issued during the current chunk and written to LDS at its end,
  // so no staging register lives across a loop iteration.
  Vec16<T> rgq[FULL ? C::QIT : 1];
  Vec16<T> rgk[C::QIT];
  Vec16<T> rgv[C::VIT];
  float rgi = 0.f, rgf = 0.f;

  auto load_q = [&](int c) __attribute__((always_inline)) {
    const unsigned t0 = (unsigned)c * L;
    if constexpr (FULL) {
#pragma unroll
      for (int it = 0; it < C::QIT; ++it) {
        const int u = (tid + it * NTH) % C::NQU;
        const unsigned j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
        rgq[it] = bload16<T>(rq, ((t0 + j) * DQK + col) * ES);
      }
    }
  };

  auto load_kv = [&](int c) __attribute__((always_inline)) {
    const unsigned t0 = (unsigned)c * L;
#pragma unroll
    for (int it = 0; it < C::QIT; ++it) {
      const int u = (tid + it * NTH) % C::NQU;
      const unsigned j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
      rgk[it] = bload16<T>(rk, ((t0 + j) * DQK + col) * ES);
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int u = (tid + it * NTH) % C::NVU;
      const unsigned j = u / (W / VE), col = (u % (W / VE)) * VE;
      rgv[it] = bload16<T>(rv, ((t0 + j) * DV + slice * W + col) * ES);
    }
    if constexpr (!RET) {
      rgi = bload1<T>(ri, (t0 + (lane & (L - 1))) * ES);
      rgf = bload1<T>(rf, (t0 + (lane & (L - 1))) * ES);
    }
  };

  auto store_stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::QIT; ++it) {
      const int u = tid + it * NTH;
      if (u < C::NQU) {
        const int j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
        if constexpr (FULL)
          *reinterpret_cast<uint4*>(&sQ[j * QS + col]) = *reinterpret_cast<const uint4*>(rgq[it].v);
        *reinterpret_cast<uint4*>(&sK[j * QS + col]) = *reinterpret_cast<const uint4*>(rgk[it].v);
      }
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int u = tid + it * NTH;
      if (u < C::NVU) {
        const int j = u / (W / VE), col = (u % (W / VE)) * VE;
        *reinterpret_cast<uint4*>(&sV[j * VS + col]) = *reinterpret_cast<const uint4*>(rgv[it].v);
      }
    }
  };

  // Gate scan for one chunk on wave 0 (one lane per token).
  auto gates = [&](int c) __attribute__((always_inline)) {
    const int t0 = c * L;
    const bool valid = lane < L && t0 + lane < T_;
    float lf2, li2;
    if constexpr (RET) {
      lf2 = valid ? ret_lg2 : 0.f;
      li2 = valid ? 0.f : -INFINITY;
    } else {
      lf2 = valid ? log2_sigmoid(rgf) : 0.f;
      li2 = valid ? rgi * kLog2e : -INFINITY;
    }
    float b = lf2;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(b, d, 64);
      if (lane >= d) b += y;
    }
    const float a = li2 - b;
    float g = a;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(g, d, 64);
      if (lane >= d) g = fmaxf(g, y);
    }
    const float Mj = fmaxf(m_prev, g);
    const float ML = __shfl(Mj, L - 1, 64);
    const float bL = __shfl(b, L - 1, 64);
    if (lane < L) {
      const float mj = b + Mj;
      const float cl = exp2_fast(-mj);
      sA2[lane] = a;
      sM2[lane] = Mj;
      sRS[lane] = exp2_fast(m_prev - Mj);
      sCL[lane] = cl;
      sBT[lane] = bias * cl;
      sW[lane] = exp2_fast(a - ML);
    }
    if (lane == 0) sAlpha = m_prev - ML;  // log2 of the state decay over the chunk
    m_prev = bL + ML;
    a_total += bL;
  };

  // Prime the first chunk.
  load_q(c_begin);
  load_kv(c_begin);
  store_stage();
  if (w == 0) gates(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * L;
    __syncthreads();  // B1: chunk staged, gate factors ready
    const bool more = c + 1 < c_end;
    // pass 1 prefetches at the top; pass 3 after its second barrier, so that
    // the readout (its register peak) holds no staging registers
    if (!FULL && more) {
      load_q(c + 1);
      load_kv(c + 1);
    }

    // update of the state is needed unless this is the last chunk of a
    // superchunk whose end state nobody reads
    const bool need_update = !FULL || more || (sc == p.NS - 1);

    frag vf[CT][NKL];  // V^T fragments of this wave's columns
    auto load_vf = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) vf[ct][kb] = frag_rows(sV, VS, kb * K + KL * lg, lr, vcol + ct * 16);
    };
    if constexpr (!FULL) load_vf();

    if constexpr (FULL) {
      // ---------------------------------------------------------- phase B
      // causal score tiles (key tile lt, query tile jt), spread over the waves
#pragma unroll
      for (int ti = 0; ti < C::NTQK; ++ti) {
        if (w == ti % NW) {
          int lt = 0, jt = ti, rem = NJT;
          while (jt >= rem) {  // tile index -> (lt, jt) with lt <= jt
            jt -= rem;
            ++lt;
            --rem;
          }
          jt += lt;
          f32x4 pt[NB];
#pragma unroll
          for (int be = 0; be < NB; ++be) {
            pt[be] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKQB; ++kk) {
              const int kb = be * NKQB + kk;
              const frag kf = M::load(&sK[(lt * 16 + lr) * QS + kb * K + KL * lg]);
              const frag qj = M::load(&sQ[(jt * 16 + lr) * QS + kb * K + KL * lg]);
              pt[be] = M::mma(kf, qj, pt[be]);
              if (kk & 1) __builtin_amdgcn_sched_barrier(0);
            }
          }
          // decay factors, P to LDS, den partial sums
          const int j = jt * 16 + lr;
          const float m2 = sM2[j];
          float fac[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int l = lt * 16 + 4 * lg + i;
            fac[i] = (l <= j) ? exp2_fast(sA2[l] - m2) : 0.f;
          }
          float dsum = 0.f;
#pragma unroll
          for (int be = 0; be < NB; ++be) {
            T pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = pt[be][i] * fac[i];
              dsum += x;
              pv[i] = from_f32<T>(x);
            }
            store4(&sP[(be * L + j) * PS + lt * 16 + 4 * lg], pv[0], pv[1], pv[2], pv[3]);
          }
          dsum += __shfl_xor(dsum, 16, 64);
          dsum += __shfl_xor(dsum, 32, 64);
          if (lg == 0) sDenPart[lt * L + j] = dsum;
        }
      }
      // n~ . q_j per query tile, n~ split in hi + lo parts (last waves)
      if constexpr (!RET) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          if (w == NW - 1 - (jt % NW)) {
            f32x4 pn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKQ; ++kb) {
              const frag nf = M::load(&sNh[lr * DQK + kb * K + KL * lg]);
              pn = M::mma(nf, M::load(&sQ[(jt * 16 + lr) * QS + kb * K + KL * lg]), pn);
              if (kb & 1) __builtin_amdgcn_sched_barrier(0);
            }
            if (lg == 0) sDenInter[jt * 16 + lr] = pn[0] + pn[1];
          }
        }
      }
      // readout of the state at the chunk start over this wave's rows:
      // acc[jt][ct] = S~[rows, c]^T q_j
      f32x4 acc[NJT][CT];
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[jt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int kq0 = rb0 / K;  // first feature k-block of this wave's rows
#pragma unroll
      for (int kk = 0; kk < NKQR; ++kk) {
        frag qf[NJT];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
          qf[jt] = M::load(&sQ[(jt * 16 + lr) * QS + (kq0 + kk) * K + KL * lg]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const frag sf = StateFrag<T, NT, CT>::get(st, kk, ct);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) acc[jt][ct] = M::mma(sf, qf[jt], acc[jt][ct]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // hand the readout partials of the other row group's token tiles over
      if constexpr (XCH) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
          if (jt / JPW != rg)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) sX[((cg * NJT + jt) * CT + ct) * 64 + lane] = acc[jt][ct];
      }
      __syncthreads();  // B2: P, den partials and readout partials ready
      if (more) {
        load_kv(c + 1);
        load_q(c + 1);
      }
      load_vf();

      // ---------------------------------------------------------- phase C
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int jt = jt0 + jj;  // runtime, wave-uniform
        f32x4 o_acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          // select acc[jt][ct] with a compile-time index
          f32x4 a = acc[0][ct];
#pragma unroll
          for (int t = 1; t < NJT; ++t)
            if (jt == t) a = acc[t][ct];
          if constexpr (XCH) a += sX[((cg * NJT + jt) * CT + ct) * 64 + lane];
          o_acc[ct] = a;
        }
        const int j = jt * 16 + lr;
        const float rs = sRS[j];
        const float rs_state = rs * exp2_fast(sig);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o_acc[ct] *= rs_state;
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) {
          if (kb * K <= jt * 16 + 15) {
            const frag pf = M::load(&sP[(blk * L + jt * 16 + lr) * PS + kb * K + KL * lg]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) o_acc[ct] = M::mma(vf[ct][kb], pf, o_acc[ct]);
          }
        }
        float inv;
        if constexpr (RET) {
          inv = 1.f;
        } else {
          float den = rs * sDenInter[j] + sBT[j];
#pragma unroll
          for (int t = 0; t < NJT; ++t) den += sDenPart[t * L + j];
          inv = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), sCL[j]));
        }
        if (t0 + j < T_) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int col = wcol0 + ct * 16 + 4 * lg;
            float o[4] = {1.f, 1.f, 1.f, 1.f};
            if (has_o) {
              bload4<T>(ro, ((unsigned)(t0 + j) * DV + col) * ES, o);
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = sigmoidf_(o[i]);
            }
            T hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = from_f32<T>(o[i] * o_acc[ct][i] * inv);
            store4(gh + (size_t)(t0 + j) * DV + col, hv[0], hv[1], hv[2], hv[3]);
          }
        }
      }
    }

    // ------------------------------------------------------- state update
    if (need_update) {
      const float la = sAlpha;
      const float alpha = exp2_fast(la);
      sig += la;
      if (sig < -64.f) {  // wave-uniform: rescale the registers, rarely
        const float f = exp2_fast(sig);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st[nt][ct] *= f;
        sig = 0.f;
      }
      const float wscale = exp2_fast(-sig);
      // n~ gets sum_l w_l k_l.  With one memory block the K^T fragments of the
      // update carry every feature of k: each is summed by one wave (tile nt
      // goes to column group nt % 4).  With several blocks a work-group's waves
      // need not cover all blocks, so a plain loop over sK does it.
      constexpr bool NFRAG = !RET && NB == 1;
      float dn[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) dn[nt] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb) {
        float wl[KL];
#pragma unroll
        for (int e = 0; e < KL; ++e) wl[e] = sW[kb * K + KL * lg + e];
        float wls[KL];
#pragma unroll
        for (int e = 0; e < KL; ++e) wls[e] = wl[e] * wscale;
        frag wv[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) wv[ct] = scale_frag(vf[ct][kb], wls);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int kc = BF ? kcol + (nt >> 1) * 32 + (nt & 1) * 4 : kcol + perm_row<T>(nt, lr);
          const frag ka = frag_rows(sK, QS, kb * K + KL * lg, lr, kc);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st[nt][ct] = M::mma(ka, wv[ct], st[nt][ct]);
          if constexpr (NFRAG) {
            if ((nt & 3) == cg) {
#pragma unroll
              for (int e = 0; e < KL; ++e) {
                if constexpr (BF) dn[nt] += wl[e] * (float)ka[e];
                else dn[nt] += wl[e] * ka;
              }
            }
          }
          if ((nt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!RET && !NFRAG) {
        for (int r = tid; r < DQK; r += NTH) {
          float x = alpha * sNf[r];
          for (int l = 0; l < L; ++l) x += sW[l] * to_f32(sK[l * QS + r]);
          put_n(r, x);
        }
      }
      if constexpr (NFRAG) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if ((nt & 3) == cg) {
            float d = dn[nt];
            d += __shfl_xor(d, 16, 64);
            d += __shfl_xor(d, 32, 64);
            if (lg == 0) {
              const int r = rb0 + perm_row<T>(nt, lr);
              put_n(r, alpha * sNf[r] + d);
            }
          }
        }
      }
    }
    __syncthreads();  // B3: LDS free for the next chunk
    if (more) {
      store_stage();
      if (w == 0) gates(c + 1);
    }
  }

  // ---------------------------------------------------------------- outputs
  float* Sdst = nullptr;
  if (!FULL) Sdst = p.ws_state + ((size_t)bh * p.NS + sc + 1) * NSTATE;
  else if (sc == p.NS - 1 && p.C_out) Sdst = p.C_out + (size_t)bh * CS;  // [B,H,NB,DQKB,DVB]
  if (Sdst) {
    const float f = exp2_fast(sig);
    int so = soff;
    asm volatile("" : "+v"(so));  // recompute addresses here, do not keep the prologue's
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sdst[so + perm_row_uni<T>(nt, i) * DVB + ct * 16] = st[nt][ct][i] * f;
  }
  if (slice == 0) {
    if (!FULL) {
      float* nd = p.ws_state + ((size_t)bh * p.NS + sc + 1) * NSTATE + CS;
      if constexpr (!RET)
        for (int r = tid; r < DQK; r += NTH) nd[r] = sNf[r];
      if (tid == 0) {
        p.ws_scal[((size_t)bh * p.NS + sc) * 2 + 0] = a_total;
        p.ws_scal[((size_t)bh * p.NS + sc) * 2 + 1] = m_prev;
      }
    } else if (sc == p.NS - 1) {
      if constexpr (!RET) {
        if (p.n_out)
          for (int r = tid; r < DQK; r += NTH) p.n_out[(size_t)bh * DQK + r] = sNf[r];
      }
      if (tid == 0 && p.m_out) p.m_out[bh] = m_prev * kLn2;
    }
  }
}

// Pass 2: start state of every superchunk.  One thread per 4 state elements
// of one (batch*head); sequential over superchunks.
template <bool RET>
__global__ __launch_bounds__(256) void superchunk_scan_kernel(ScanParams p) {
  const int bh = blockIdx.y;
  const size_t NSTATE = p.CS + (RET ? 0 : p.DQK);
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const float m0 = (!RET && p.m0) ? p.m0[bh] * kLog2e : 0.f;
  const bool writer = blockIdx.x == 0 && threadIdx.x == 0;
  if (writer) p.ws_min[(size_t)bh * p.NS] = m0;
  float* base = p.ws_state + (size_t)bh * p.NS * NSTATE;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  const bool active = e0 < NSTATE;
  if (active && p.has_init) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t e = e0 + i;
      if (e < p.CS) x[i] = p.C0 ? p.C0[(size_t)bh * p.CS + e] : 0.f;
      else x[i] = p.n0 ? p.n0[(size_t)bh * p.DQK + (e - p.CS)] : 0.f;
    }
    S = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(base + e0) = S;
  }
  float m = m0;
  for (int sc = 1; sc < p.NS; ++sc) {
    const float A = p.ws_scal[((size_t)bh * p.NS + sc - 1) * 2 + 0];
    const float mu = p.ws_scal[((size_t)bh * p.NS + sc - 1) * 2 + 1];
    const float mn = fmaxf(A + m, mu);
    const float fa = exp2_fast(A + m - mn), fb = exp2_fast(mu - mn);
    if (active) {
      float4* ptr = reinterpret_cast<float4*>(base + (size_t)sc * NSTATE + e0);
      const float4 d = *ptr;
      S.x = fa * S.x + fb * d.x;
      S.y = fa * S.y + fb * d.y;
      S.z = fa * S.z + fb * d.z;
      S.w = fa * S.w + fb * d.w;
      *ptr = S;
    }
    m = mn;
    if (writer) p.ws_min[(size_t)bh * p.NS + sc] = mn;
  }
}

template <typename T, int DQK, int NB, int WC, int NRG, int L, bool RET>
size_t chunk_lds_bytes() {
  return ChunkCfg<T, DQK, NB, WC, NRG, L>::lds_bytes(true, RET);
}

template <typename T, int DQK, int NB, int WC, int NRG, int L, bool RET>
hipError_t launch_chunkwise(ChunkParams p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int NTH = 256 * NRG;
  const int BH = p.B * p.H;
  const size_t CS = (size_t)DQK * p.DV / NB;
  if (p.NS > 1) {
    dim3 g1((unsigned)(BH * p.nslices * (p.NS - 1)));
    hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, NRG, L, RET, false>), g1, dim3(NTH), 0, stream, p);
  }
  ScanParams s;
  s.NS = p.NS;
  s.CS = CS;
  s.DQK = DQK;
  s.ws_state = p.ws_state;
  s.ws_scal = p.ws_scal;
  s.ws_min = p.ws_min;
  s.has_init = p.has_init;
  s.C0 = p.C0;
  s.n0 = p.n0;
  s.m0 = p.m0;
  const size_t nstate = CS + (RET ? 0 : DQK);
  dim3 g2((unsigned)((nstate / 4 + 255) / 256), (unsigned)BH);
  hipLaunchKernelGGL((superchunk_scan_kernel<RET>), g2, dim3(256), 0, stream, s);
  dim3 g3((unsigned)(BH * p.nslices * p.NS));
  if (ev0) (void)hipEventRecord(ev0, stream);
  hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, NRG, L, RET, true>), g3, dim3(NTH), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (ev1) (void)hipEventRecord(ev1, stream);
  return e;
}

// ------------------------------------------------------------ dispatch table
// (dtype, d_qk, num_blocks, columns per wave, row groups, chunk, retention)
#define MLSTM_CHUNK_VARIANTS(X)            \
  X(__bf16, 64, 1, 16, 1, 64, false)       \
  X(__bf16, 64, 2, 16, 1, 64, false)       \
  X(__bf16, 64, 1, 16, 1, 32, false)       \
  X(__bf16, 128, 1, 32, 2, 64, false)      \
  X(__bf16, 256, 1, 32, 2, 64, false)      \
  X(__bf16, 256, 2, 16, 2, 64, false)      \
  X(float, 64, 1, 16, 1, 64, false)        \
  X(float, 64, 1, 16, 1, 32, false)        \
  X(float, 64, 1, 16, 1, 16, false)        \
  X(float, 64, 2, 16, 1, 64, false)        \
  X(__bf16, 64, 1, 16, 1, 64, true)        \
  X(__bf16, 64, 1, 16, 1, 32, true)        \
  X(__bf16, 128, 1, 32, 2, 64, true)       \
  X(float, 64, 1, 16, 1, 64, true)

bool find_chunk_variant(int dtype, int dqk, int nb, int wc, int L, bool ret, ChunkVariant* out) {
#define X(T_, DQK_, NB_, WC_, NRG_, L_, RET_)                                                    \
  if (dtype == (sizeof(T_) == 2 ? 1 : 0) && dqk == DQK_ && nb == NB_ && wc == WC_ && L == L_ && \
      ret == RET_) {                                                                             \
    out->launch = &launch_chunkwise<T_, DQK_, NB_, WC_, NRG_, L_, RET_>;                         \
    out->lds_bytes = chunk_lds_bytes<T_, DQK_, NB_, WC_, NRG_, L_, RET_>();                      \
    out->wc = WC_;                                                                               \
    return true;                                                                                 \
  }
  MLSTM_CHUNK_VARIANTS(X)
#undef X
  return false;
}

}  // namespace mlstm
