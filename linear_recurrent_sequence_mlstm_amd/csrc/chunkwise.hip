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
//   pass 1  the gate logs of every superchunk of G chunks (extra work-groups)
//           and, for every superchunk but the last, its local end state dS,
//           dn from a zero state (m = -inf) as one dense product; dS, dn, the
//           log scale mu and the total log decay A go to the workspace.  With
//           a single superchunk a small gate kernel replaces it.
//   pass 2  per state element, a scan over superchunks
//           m' = max(A + m, mu); S' = 2^{A+m-m'} S + 2^{mu-m'} dS
//           leaves the start state of every superchunk in the workspace.
//   pass 3  every (batch*head, superchunk, d_v slice) work-group runs its
//           chunks sequentially from its start state: readout, intra-chunk
//           product, output, state update.
//
// Pass 3 work-group: 4 column groups x NRG row groups of waves.  It owns
// W = 4*WC columns of d_v; wave (cg, rg) owns WC of them and d_qk/NB/NRG rows
// of the memory block they lie in.  The fp32 state slice lives in registers
// as MFMA accumulator tiles for the whole superchunk.  Its rows are stored in
// a permuted order (perm_row) so that the accumulator registers are directly
// the A operand of the readout MFMA.
#include <type_traits>

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

// Superchunk start states of the 7B head shape (bf16, d_qk = 256, d_v a
// multiple of 128, one memory block) are kept in the order the pass-3 state
// waves hold them: for each group of 32 columns (one state wave of one
// slice), each of its 32 (row tile, column tile) pairs, each lane, the four
// rows of that lane's accumulator.  Pass 1 then stores a lane's 4 rows as
// one 16-byte store, and pass 3 reads each lane's 128 values as 32 16-byte
// loads that cover 1 KB per wave.  Index of the float4 holding rows
// r0 .. r0 + 3 (r0 a multiple of 4) of column c:
__device__ __forceinline__ unsigned ws_perm4(int r0, int c) {
  const int nt = 2 * (r0 >> 5) + ((r0 >> 2) & 1);  // inverse of perm_row<bf16>
  const int lg = (r0 >> 3) & 3;
  return (unsigned)((((c >> 5) * 32 + nt * 2 + ((c >> 4) & 1)) * 64 + (c & 15) + 16 * lg) * 4);
}

// Readout A operand (rows = columns of d_v, k = features kk*K .. +K-1 of the
// block) taken from the accumulator tiles of the state.
template <typename T, int NT, int CT>
struct StateFrag;
template <int NT, int CT>
struct StateFrag<__bf16, NT, CT> {
  __device__ __forceinline__ static bf16x8 get(const f32x4 (&st)[NT][CT], int kk, int ct) {
    const f32x4 a = st[2 * kk][ct], b = st[2 * kk + 1][ct];
    const u32x4 r = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                     pack_bf16x2(b[2], b[3])};
    return __builtin_bit_cast(bf16x8, r);
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
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2((float)x[2 * q] * w[2 * q], (float)x[2 * q + 1] * w[2 * q + 1]);
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ float scale_frag(float x, const float* w) { return x * w[0]; }

// Row padding (elements) of a token-major LDS tile: the smallest padding that
// makes a row step move the bank by 8 + 16i dwords (mod 64).  In a sweep on
// MI355X these residues were the fastest both for 16-byte fragment loads
// over 16 rows and for transposing reads in the frag_rows layout (16 lanes
// over 16 consecutive rows, 32 contiguous bytes per row).
constexpr int lds_row_pad(int row_elems, int esize) {
  const int dw = row_elems * esize / 4;
  int best = 64;
  const int rq[4] = {8, 24, 40, 56};
  for (int i = 0; i < 4; ++i) {
    const int pad = ((rq[i] - dw % 64) % 64 + 64) % 64;
    if (pad < best) best = pad;
  }
  return best * 4 / esize;
}

// Row padding (elements) that makes a row step move the bank by `res` dwords
// (mod 64).
constexpr int lds_pad_res(int row_elems, int esize, int res) {
  const int dw = row_elems * esize / 4;
  return (((res - dw % 64) % 64 + 64) % 64) * 4 / esize;
}
#ifndef MLSTM_P1_ROWS
#define MLSTM_P1_ROWS 256  // most state rows of a bf16 pass-1 tile
#endif
#ifndef MLSTM_P1_STAGES
#define MLSTM_P1_STAGES 4  // LDS ring stages of pass 1 (3 to 6; loads run stages-1 k-steps ahead)
#endif
#ifndef MLSTM_P3_QRES
#define MLSTM_P3_QRES 8
#endif
#ifndef MLSTM_P3_KRES
#define MLSTM_P3_KRES 24
#endif
#ifndef MLSTM_P3_UPD
#define MLSTM_P3_UPD 1  // K^T fragment groups read ahead in the 7B pass-3 state update
#endif
#ifndef MLSTM_P3_SCD
#define MLSTM_P3_SCD 1  // k-blocks of score fragments read ahead in the 7B pass-3 helpers
#endif
#ifndef MLSTM_P3_PRIO
// wave priorities in the 7B pass 3: 0 none; 1 helpers raised while they form
// the score tiles (the longer role before barrier B: their MFMAs then issue
// ahead of the readout's); 2 that, and the state waves raised above the
// helpers' staging after barrier B; 3 state waves raised only
#define MLSTM_P3_PRIO 1
#endif

template <typename T, int DQK, int NB, int WC, int NRG, int NCG, int L, bool GN = false, bool PB = false>
struct ChunkCfg {
  static constexpr int K = Mma<T>::K;
  static constexpr int KL = Mma<T>::KL;
  static constexpr int NW = NCG * NRG;            // waves per work-group
  static constexpr int NTH = 64 * NW;             // threads per work-group
  static constexpr int DQKB = DQK / NB;           // rows of a memory block
  static constexpr int RPW = DQKB / NRG;          // state rows per wave
  static constexpr int NT = RPW / 16;             // state row tiles per wave
  static constexpr int CT = WC / 16;              // state column tiles per wave
  static constexpr int W = NCG * WC;              // d_v columns per work-group
  static constexpr int NJT = L / 16;              // 16-token tiles per chunk
  static constexpr int JPW = NJT / NRG;           // token tiles finished per wave
  // jj-th token tile finished by row group g (snake order) and its owner
  static constexpr int jt_of(int g, int jj) { return jj * NRG + ((jj & 1) ? NRG - 1 - g : g); }
  static constexpr int owner_of(int jt) { return ((jt / NRG) & 1) ? NRG - 1 - jt % NRG : jt % NRG; }
  static constexpr int NKL = L / K;               // token k-blocks per chunk
  static constexpr int NKQ = DQK / K;             // feature k-blocks of a head
  static constexpr int NKQB = DQKB / K;           // feature k-blocks of a block
  static constexpr int NKQR = RPW / K;            // feature k-blocks of a wave's rows
  static constexpr int NTQK = NJT * (NJT + 1) / 2;  // causal score tiles
  static constexpr int NUMAX = (NTQK + NCG * NRG - 1) / (NCG * NRG);  // score tiles per wave
  static_assert(NUMAX <= 3, "at most three score tiles per wave");
  // With one memory block, n~.q_j for query tile j is summed by wave j
  // together with its first score tile (0, j), which reads the same Q rows;
  // else in a loop of its own.
  static constexpr bool FUSED_NQ = NB == 1;
  static_assert(NJT <= NCG * NRG, "a wave per query tile");
  static constexpr int VE = 16 / (int)sizeof(T);  // elements per 16 bytes
  // row strides (elements) of the token-major tiles
  // sQ is read with 16-byte row fragments only; sK also with transposing
  // reads (the update's K^T, 16-byte spaced 8-byte runs per row), whose
  // bank spread is best at residue 24
  // (heads narrower than 128 take the smallest padding of the same residue
  // family instead: there the tuned residues would nearly double the row
  // and halve the work-groups that fit on a CU)
  static constexpr int QS = DQK + (DQK >= 128 ? lds_pad_res(DQK, (int)sizeof(T), MLSTM_P3_QRES)
                                              : lds_row_pad(DQK, (int)sizeof(T)));  // sQ
  static constexpr int KST = DQK + (DQK >= 128 ? lds_pad_res(DQK, (int)sizeof(T), MLSTM_P3_KRES)
                                               : lds_row_pad(DQK, (int)sizeof(T)));  // sK
  static constexpr int VS = W + lds_row_pad(W, (int)sizeof(T));  // sV
  static constexpr int PS = L + 16 / (int)sizeof(T);  // sP
  // bf16 outputs are staged in LDS (sH, token-major) and written as whole
  // 16-byte units of the work-group's row segment.  With the fused group
  // norm (GN) every output is staged, in fp32, and normalised per row.
  static constexpr bool HST = sizeof(T) == 2 || GN;
  using HT = typename std::conditional<GN, float, T>::type;  // staging type
  static constexpr int HS = W + 16 / (int)sizeof(HT);
  // staging units (16-byte loads) per chunk
  static constexpr int NQU = L * DQK / VE;
  static constexpr int NVU = L * W / VE;
  static constexpr int QIT = (NQU + NTH - 1) / NTH;
  static constexpr int VIT = (NVU + NTH - 1) / NTH;
  static_assert(DQK % NB == 0, "d_qk % nb");
  static_assert(RPW % (sizeof(T) == 2 ? 32 : 16) == 0, "state rows per wave");
  static_assert(L % K == 0 && L % 16 == 0 && L <= 64, "chunk length");
  static_assert(NJT % NRG == 0 && NRG <= 2, "token tiles per row group");
  static_assert(WC % 16 == 0, "wave columns");
  static constexpr size_t lds_bytes(bool ret) {
    size_t b = 0;
    b += (size_t)L * KST * sizeof(T);            // sK
    b += (size_t)L * VS * sizeof(T);             // sV
    b += 2 * 6 * L * 4 + 16;                     // gate vectors, two sets
    if (!ret) b += DQK * 4 + 2 * DQK * sizeof(T);  // n~
    b += (size_t)L * QS * sizeof(T);             // sQ
    b += (size_t)NB * L * PS * sizeof(T);        // sP
    b += (size_t)(PB ? NB : 1) * (NJT + 1) * L * 4;  // den partials
    if (NRG > 1) b += (size_t)NCG * NJT * CT * 64 * 16;  // readout exchange
    if (HST) b += (size_t)L * HS * sizeof(HT);   // sH
    return b;
  }
};

// Row (token) inside a K-row block of element e of lane group lg, for MFMA
// operands whose k index runs along tokens.  bf16: lane group lg takes rows
// 4lg .. 4lg+3 and 16+4lg .. 16+4lg+3, so that the 16 lanes of one
// transposing read cover 16 consecutive rows (fewer LDS bank conflicts than
// 8 consecutive rows per lane group).  The contraction does not care which k
// is which token as long as both operands agree, so every operand along
// tokens (K^T, V^T, P rows, the weights w) uses this order.  fp32: row lg.
template <typename T>
__device__ __forceinline__ constexpr int krow(int lg, int e) {
  return sizeof(T) == 2 ? 4 * lg + (e & 3) + 16 * (e >> 2) : lg + e;
}
// Position of token t (t % 4 == 0) in a P row stored so that a 16-byte row
// fragment at 8 lg holds the tokens krow(lg, 0..7) of its block.
template <typename T>
__device__ __forceinline__ constexpr int kpos4(int t) {
  return sizeof(T) == 2 ? (t & ~31) + 8 * ((t >> 2) & 3) + 4 * ((t >> 4) & 1) : t;
}

// MFMA fragment along the rows of a token-major tile: lane (lr, lg) gets rows
// kb0 + krow(lg, e) of one column.
//   bf16: two transposing reads; source lane lr addresses column csrc(lr),
//         chosen by the caller so that output lane lr sees its column.
//   fp32: one element, column ccol(lr).
__device__ __forceinline__ bf16x8 frag_rows(const __bf16* tile, int RS, int kb0, int lg, int lr, int csrc) {
  const __bf16* p = tile + (kb0 + 4 * lg + (lr >> 2)) * RS + csrc;
  const bf16x4 a = ds_read_tr16(p);
  const bf16x4 b = ds_read_tr16(p + 16 * RS);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = a[e];
    r[4 + e] = b[e];
  }
  return r;
}
__device__ __forceinline__ float frag_rows(const float* tile, int RS, int kb0, int lg, int lr, int ccol) {
  (void)lr;
  return tile[(kb0 + lg) * RS + ccol];
}

// inclusive scans over lanes in segments of SEG = 16, 32 or 64 lanes: row
// shifts inside rows of 16, then row broadcasts.  update_dpp with bound_ctrl
// off hands lanes without a source (and lanes of rows outside the row mask)
// the `old` operand, here the identity (checked on MI355X).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or(float x, float identity) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float seg_scan_sum(float x, int seg) {
  x += dpp_or<0x111, 0xF>(x, 0.f);                  // row_shr:1
  x += dpp_or<0x112, 0xF>(x, 0.f);                  // row_shr:2
  x += dpp_or<0x114, 0xF>(x, 0.f);                  // row_shr:4
  x += dpp_or<0x118, 0xF>(x, 0.f);                  // row_shr:8
  if (seg >= 32) x += dpp_or<0x142, 0xA>(x, 0.f);  // row_bcast:15 into rows 1, 3
  if (seg >= 64) x += dpp_or<0x143, 0xC>(x, 0.f);  // row_bcast:31 into rows 2, 3
  return x;
}
__device__ __forceinline__ float seg_scan_max(float x, int seg) {
  x = fmaxf(x, dpp_or<0x111, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_or<0x112, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_or<0x114, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_or<0x118, 0xF>(x, -INFINITY));
  if (seg >= 32) x = fmaxf(x, dpp_or<0x142, 0xA>(x, -INFINITY));
  if (seg >= 64) x = fmaxf(x, dpp_or<0x143, 0xC>(x, -INFINITY));
  return x;
}

// Pass 3: per (batch*head, superchunk, d_v slice), the chunks of the
// superchunk in order from its start state: readout, outputs, update.
//
// Work-group = 4 column groups x NRG row groups of waves.  Wave (cg, rg) owns
// columns [cg*WC, cg*WC+WC) of the work-group's d_v slice and state rows
// [rg*RPW, rg*RPW+RPW) of their memory block.  With NRG = 2 the readout of a
// column group is split over its two waves by rows; each wave finishes half of
// the token tiles and the two partial sums meet in LDS (sX).
// Q, K and V are staged token-major with plain 16-byte copies; the operands
// that run along tokens (K^T and V^T) are read with transposing LDS reads.
// SN: the scalar normaliser n~ = f' n~ + i' (kept in n~[0], the other
// entries zero), denominator |n~ + bias 2^{-m}| instead of |n~ . q + ...|.
// PB: one denominator per memory block, |n~_b . q_b + ...| over the block's
// features (NB > 1).
template <typename T, int DQK, int NB, int WC, int NRG, int NCG, int L, bool RET, bool HAS_O, bool GN = false,
          bool SN = false, bool PB = false, bool DIR = false, bool FS = false>
__global__ __launch_bounds__(64 * NCG * NRG) void chunk_kernel(ChunkParams p) {
  using C = ChunkCfg<T, DQK, NB, WC, NRG, NCG, L, GN, PB>;
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int K = C::K, KL = C::KL, DQKB = C::DQKB, NT = C::NT, CT = C::CT, NW = C::NW;
  constexpr int NTH = C::NTH, RPW = C::RPW, JPW = C::JPW;
  constexpr int W = C::W, NJT = C::NJT, NKL = C::NKL, NKQ = C::NKQ, NKQB = C::NKQB, NKQR = C::NKQR;
  constexpr int VE = C::VE, QS = C::QS, KST = C::KST, VS = C::VS, PS = C::PS, HS = C::HS;
  constexpr bool HST = C::HST;
  constexpr unsigned ES = sizeof(T);
  constexpr bool XCH = NRG > 1;
  constexpr bool BF = sizeof(T) == 2;
  constexpr bool VN = !RET && !SN;  // vector normaliser
  static_assert(!PB || (NB > 1 && VN), "per-block denominators need blocks and the vector normaliser");
  constexpr int NDB = PB ? NB : 1;  // denominators per head

  __shared__ __attribute__((aligned(16))) T sK[L * KST];  // K, token-major
  __shared__ __attribute__((aligned(16))) T sV[L * VS];   // V slice, token-major
  __shared__ __attribute__((aligned(16))) T sQ[L * QS];   // Q, token-major
  __shared__ __attribute__((aligned(16))) T sP[NB * L * PS];
  __shared__ __attribute__((aligned(16))) f32x4 sX[XCH ? NCG * NJT * CT * 64 : 1];
  __shared__ __attribute__((aligned(16))) typename C::HT sH[HST ? L * HS : 8];  // outputs of the chunk
  // n~ as rows 0 and 1 of a 16-row A-operand tile (rows 2..15 are zero and
  // not stored): row 0 = bf16 hi part, row 1 = lo part (fp32: row 0 = n~,
  // row 1 zero)
  __shared__ __attribute__((aligned(16))) T sNh[RET ? 8 : 2 * DQK];
  __shared__ float sNf[RET ? 4 : DQK];
  // gate vectors, two sets: wave 0 fills the next chunk's while the other
  // waves still read the current chunk's
  __shared__ __attribute__((aligned(16))) float sA2b[2][L];
  __shared__ float sM2b[2][L], sRSb[2][L], sCLb[2][L], sBTb[2][L], sWb[2][L];
  __shared__ float sDenPart[NDB * NJT * L];
  __shared__ float sDenInter[NDB * L];
  __shared__ float sAlphab[2];

  const int tid = threadIdx.x;
  // The wave index must be known to be wave-uniform: branches on it guard
  // MFMA instructions, which do not honour a partial EXEC mask.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = w % NCG, rg = w / NCG;
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
  // Token tiles finished by the waves of row group g: jj-th = jt_of(g, jj),
  // snake order (0 and 3 for one row group, 1 and 2 for the other with four
  // tiles), so that both groups get the same share of causal P V work.

  // buffer resources over this (batch, head): reads past T return zero
  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * T_ * DV, (unsigned)T_ * DV * ES);
  // chunk-local gate logs of the gate pass, over the padded sequence
  const size_t NCL = (size_t)p.NC * L;
  const auto rga_r = make_rsrc(p.ws_ga + (size_t)bh * NCL, (unsigned)NCL * 4u);
  const auto rgg_r = make_rsrc(p.ws_gg + (size_t)bh * NCL, (unsigned)NCL * 4u);
  const auto rgb_r = make_rsrc(p.ws_gb + (size_t)bh * NCL, (unsigned)NCL * 4u);
  // ... or, in a direct call, the gate preactivations themselves
  constexpr bool dg = DIR && !RET;
  const auto ri_d = make_rsrc(dg ? static_cast<const T*>(p.i_pre) + (size_t)bh * T_ : nullptr, dg ? (unsigned)T_ * ES : 0u);
  const auto rf_d = make_rsrc(dg ? static_cast<const T*>(p.f_pre) + (size_t)bh * T_ : nullptr, dg ? (unsigned)T_ * ES : 0u);
  constexpr bool has_o = HAS_O;  // output gate present (o_pre not null)
  const auto ro = make_rsrc(has_o ? static_cast<const T*>(p.o_pre) + (size_t)bh * T_ * DV : nullptr,
                            has_o ? (unsigned)T_ * DV * ES : 0u);
  const auto rh = make_rsrc(static_cast<T*>(p.h) + (size_t)bh * T_ * DV, (unsigned)T_ * DV * ES);
  const float bias = (!RET && p.bias) ? p.bias[hd] : 0.f;

  const int c_begin = sc * p.G;
  const int c_end = min(c_begin + p.G, p.NC);

  // Source columns of the transposing reads.  K^T (update A operand): output
  // lane lr must see feature rb0 + perm_row(nt, lr).  V^T (PV A operand and
  // update B operand): output lane lr sees column cg*WC + ct*16 + lr.
  const int kcol = BF ? rb0 + 8 * (lr & 3) : rb0;  // + perm part added per tile
  const int vcol = BF ? cg * WC + 4 * (lr & 3) : cg * WC + lr;

  // ---------------------------------------------------------------- state in
  f32x4 st[NT][CT];
  // the start state through a descriptor that is empty when there is none
  // (reads zero): the loads need no branch and go out back to back
  // (a direct call reads the caller's C0 and n0, a planned one its slot of
  // superchunk start states, whose n~ follows the matrix; FS starts from the
  // caller's state too and composes it below)
  constexpr bool CALLER = DIR || FS;
  const bool has_in = CALLER ? p.C0 != nullptr : (sc > 0 || p.has_init);
  const float* sbase = CALLER ? (p.C0 ? p.C0 + (size_t)bh * CS : nullptr) : p.ws_state + ((size_t)bh * p.NS + sc) * NSTATE;
  const auto rSin = make_rsrc(sbase, has_in ? (unsigned)((CALLER ? CS : NSTATE) * 4) : 0u);
  constexpr int NN = SN ? 1 : DQK;  // entries of a caller's n0 per (batch, head)
  const bool has_n = CALLER ? p.n0 != nullptr : has_in;
  const float* nbase = CALLER ? (p.n0 ? p.n0 + (size_t)bh * NN : nullptr) : sbase + CS;
  const auto rNin = make_rsrc(nbase, has_n ? (unsigned)((CALLER ? NN : DQK) * 4) : 0u);
  // state element (nt, ct, i) of this lane sits at soff + (uni(nt,i)*DVB + ct*16)
  const int soff = blk * DQKB * DVB + (rrow0 + perm_row_lane<T>(lg)) * DVB + wcl0 + lr;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st[nt][ct][i] = bload1<float>(rSin, (unsigned)(soff + perm_row_uni<T>(nt, i) * DVB + ct * 16) * 4u);
  // n~ in fp32 and as the hi/lo rows of the den tile
  auto put_n = [&](int r, float x) __attribute__((always_inline)) {
    sNf[r] = x;
    const T hi = from_f32<T>(x);
    sNh[r] = hi;
    sNh[DQK + r] = from_f32<T>(x - to_f32(hi));
  };
  // FS: pass 2 folded in.  This superchunk's start state is the scan of the
  // local states of superchunks 0 .. sc-1 (pass 1's slots 1 .. sc, with
  // their log2 decay A and scale mu) from the caller's state, in pass 2's
  // arithmetic: m' = max(A + m, mu), S = 2^{A+m-m'} S + 2^{mu-m'} dS.  All
  // FS_J slots load first (past sc they repeat slot sc and are not used), so
  // their latencies overlap.
  constexpr int FS_J = FS ? 7 : 1;
  float fs_m = (!RET && p.m0) ? p.m0[bh] * kLog2e : 0.f;
  float fs_fa[FS_J], fs_fb[FS_J];
  if constexpr (FS) {
    const auto rLoc = make_rsrc(p.ws_state + (size_t)bh * p.NS * NSTATE, (unsigned)(p.NS * NSTATE * 4));
    float dl[FS_J][NT][CT][4];
#pragma unroll
    for (int j = 0; j < FS_J; ++j) {
      const unsigned slot = (unsigned)min(j + 1, sc) * (unsigned)NSTATE;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dl[j][nt][ct][i] =
                bload1<float>(rLoc, (slot + (unsigned)(soff + perm_row_uni<T>(nt, i) * DVB + ct * 16)) * 4u);
    }
#pragma unroll
    for (int j = 0; j < FS_J; ++j) {
      fs_fa[j] = 1.f;
      fs_fb[j] = 0.f;
      if (j < sc) {  // work-group-uniform
        const float A = p.ws_scal[((size_t)bh * p.NS + j) * 2 + 0];
        const float mu = p.ws_scal[((size_t)bh * p.NS + j) * 2 + 1];
        const float mn = fmaxf(A + fs_m, mu);
        fs_fa[j] = exp2_fast(A + fs_m - mn);
        fs_fb[j] = exp2_fast(mu - mn);
        fs_m = mn;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[nt][ct][i] = fs_fa[j] * st[nt][ct][i] + fs_fb[j] * dl[j][nt][ct][i];
      }
    }
  }
  if constexpr (!RET) {
    if constexpr (FS) {
      const auto rLoc = make_rsrc(p.ws_state + (size_t)bh * p.NS * NSTATE, (unsigned)(p.NS * NSTATE * 4));
      for (int r = tid; r < DQK; r += NTH) {
        float x = bload1<float>(rNin, (unsigned)r * 4u);
        float dn[FS_J];
#pragma unroll
        for (int j = 0; j < FS_J; ++j)
          dn[j] = bload1<float>(rLoc, ((unsigned)min(j + 1, sc) * (unsigned)NSTATE + (unsigned)(CS + r)) * 4u);
#pragma unroll
        for (int j = 0; j < FS_J; ++j)
          if (j < sc) x = fs_fa[j] * x + fs_fb[j] * dn[j];
        put_n(r, x);
      }
    } else if constexpr (DIR) {
      for (int r = tid; r < DQK; r += NTH) put_n(r, bload1<float>(rNin, (unsigned)r * 4u));
    } else {
      for (int r = tid; r < DQK; r += NTH) put_n(r, bload1<float>(rSin, (unsigned)(CS + r) * 4u));
    }
  }
  // masked (l > j) tiles of P and their den partials are never written
  for (int e = tid; e < NB * L * PS; e += NTH) sP[e] = from_f32<T>(0.f);
  for (int e = tid; e < NDB * NJT * L; e += NTH) sDenPart[e] = 0.f;
  // The registers hold S^ = S~ / 2^{sig}: the per-chunk decay of the state is
  // folded into sig (a wave-uniform scalar) instead of multiplying every
  // state element; new contributions are weighted by 2^{-sig}, the readout by
  // 2^{sig}.  When sig drops below -64 the registers are rescaled once.
  float sig = 0.f;
  // stabiliser carried by wave 0 (log2 units)
  float m_prev = FS ? fs_m : DIR ? ((!RET && p.m0) ? p.m0[bh] * kLog2e : 0.f) : p.ws_min[(size_t)bh * p.NS + sc];
  float ret_lg2 = 0.f;  // retention: log2 gamma_h (direct calls form the gate logs here)
  if constexpr (RET) ret_lg2 = log2f(p.ret_gamma ? p.ret_gamma[hd] : 1.f - exp2f(-5.f - (float)hd));

  // ------------------------------------------------------ staging registers
  // All global loads are unconditional buffer loads (units past the end of a
  // staging loop reload a valid unit and are not stored).  The next chunk's
  // loads are issued during the current chunk and written to LDS at its end,
  // so no staging register lives across a loop iteration.
  Vec16<T> rgq[C::QIT];
  Vec16<T> rgk[C::QIT];
  Vec16<T> rgv[C::VIT];
  unsigned rga = 0, rgg = 0, rgb = 0;  // chunk-local gate logs of the next chunk (raw fp32)
  unsigned rgt = 0;                    // ... and its first token (direct calls: i, f in rga, rgg)

  auto load_q = [&](int c) __attribute__((always_inline)) {
    const unsigned t0 = (unsigned)c * L;
#pragma unroll
    for (int it = 0; it < C::QIT; ++it) {
      const int u = (tid + it * NTH) % C::NQU;
      const unsigned j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
      rgq[it] = bload16<T>(rq, ((t0 + j) * DQK + col) * ES);
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
    rgt = t0;
    if constexpr (DIR) {
      const unsigned t = t0 + (unsigned)(lane & (L - 1));
      rga = __float_as_uint(bload1<T>(ri_d, t * ES));
      rgg = __float_as_uint(bload1<T>(rf_d, t * ES));
    } else {
      const unsigned o = (t0 + (unsigned)(lane & (L - 1))) * 4u;
      rga = bload1_raw<float>(rga_r, o);
      rgg = bload1_raw<float>(rgg_r, o);
      rgb = bload1_raw<float>(rgb_r, o);
    }
  };

  // With the output gate the staging indices are formed at each use:
  // hoisted out of the chunk loop they would stay live across it, and that
  // variant would spill (whose reloads wait for every load in flight).
  // Without it, hoisting them measures faster.
  auto fresh = [](int& u) __attribute__((always_inline)) {
    if constexpr (HAS_O) asm volatile("" : "+v"(u));
  };
  auto store_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::QIT; ++it) {
      int u = tid + it * NTH;
      fresh(u);
      if (u < C::NQU) {
        const int j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
        *reinterpret_cast<uint4*>(&sQ[j * QS + col]) = *reinterpret_cast<const uint4*>(rgq[it].v);
      }
    }
  };
  auto store_kv = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::QIT; ++it) {
      int u = tid + it * NTH;
      fresh(u);
      if (u < C::NQU) {
        const int j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
        *reinterpret_cast<uint4*>(&sK[j * KST + col]) = *reinterpret_cast<const uint4*>(rgk[it].v);
      }
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      int u = tid + it * NTH;
      fresh(u);
      if (u < C::NVU) {
        const int j = u / (W / VE), col = (u % (W / VE)) * VE;
        *reinterpret_cast<uint4*>(&sV[j * VS + col]) = *reinterpret_cast<const uint4*>(rgv[it].v);
      }
    }
  };

  // Gate factors of one chunk on wave 0 (one lane per token) from the
  // chunk-local logs b_j, a_j, g_j of the gate pass: only the chain through
  // m_prev is left here.
  auto gates = [&](int gb) __attribute__((always_inline)) {
    float a = __uint_as_float(rga), g = __uint_as_float(rgg), b = __uint_as_float(rgb);
    if constexpr (DIR) {
      // the gate pass's chunk-local logs, formed here: tokens past T count
      // as f = 1, i = 0
      const bool valid = rgt + (unsigned)(lane & (L - 1)) < (unsigned)T_;
      float lf2, li;
      if constexpr (RET) {
        lf2 = valid ? ret_lg2 : 0.f;
        li = valid ? 0.f : -INFINITY;
      } else {
        lf2 = valid ? log2_sigmoid(__uint_as_float(rgg)) : 0.f;
        li = valid ? __uint_as_float(rga) * kLog2e : -INFINITY;
      }
      b = seg_scan_sum(lf2, L);
      a = li - b;
      g = seg_scan_max(a, L);
    }
    const float Mj = fmaxf(m_prev, g);
    const float gL = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(g), L - 1));
    const float bL = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(b), L - 1));
    const float ML = fmaxf(m_prev, gL);
    if (lane < L) {
      const float mj = b + Mj;
      const float cl = exp2_fast(-mj);
      sA2b[gb][lane] = a;
      sM2b[gb][lane] = Mj;
      sRSb[gb][lane] = exp2_fast(m_prev - Mj);
      sCLb[gb][lane] = cl;
      sBTb[gb][lane] = bias * cl;
      sWb[gb][lane] = exp2_fast(a - ML);
    }
    if (lane == 0) sAlphab[gb] = m_prev - ML;  // log2 of the state decay over the chunk
    m_prev = bL + ML;
  };

  // Prime the first chunk.
  load_q(c_begin);
  load_kv(c_begin);
  store_q();
  store_kv();
  if (w == 0) gates(0);

  // The chunk's outputs from sH, whole 16-byte units per lane (rows past T
  // are dropped by the buffer range).  Issued after the next chunk's B1, where
  // the waves have slack, and once more after the loop.
  // group norm: a thread's units always have the same 4 columns (NTH is a
  // multiple of the units per row), so its affine parameters load once
  float gnw[GN ? 4 : 1], gnb[GN ? 4 : 1];
  if constexpr (GN) {
    const int col = (tid % (W / 4)) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gnw[i] = p.gn_w ? p.gn_w[hd * DV + col + i] : 1.f;
      gnb[i] = p.gn_b ? p.gn_b[hd * DV + col + i] : 0.f;
    }
  }
  auto store_h = [&](int tc) __attribute__((always_inline)) {
    if constexpr (GN) {
      // Group norm of each output row over the head's d_v channels (the
      // work-group holds the whole row, W = d_v): a group of UR consecutive
      // lanes owns a row, 4 fp32 values per lane; mean, then the biased
      // variance of the centred values; y = (x - mean) rsqrt(var + eps) w + b.
      // A head wider than the work-group (gn_ws set) leaves its fp32 rows in
      // gn_ws for the row pass instead.
      constexpr int UR = W / 4;
      static_assert((UR & (UR - 1)) == 0 && UR <= 64 && NTH % UR == 0, "row groups of lanes");
      if (p.gn_ws) {  // work-group-uniform
#pragma unroll
        for (int u0 = 0; u0 < L * UR; u0 += NTH) {
          const int u = u0 + tid;
          const int j = u / UR, cu = u % UR;
          if (tc + j < T_)
            *reinterpret_cast<f32x4*>(&p.gn_ws[((size_t)bh * T_ + tc + j) * DV + slice * W + cu * 4]) =
                *reinterpret_cast<const f32x4*>(&sH[j * HS + cu * 4]);
        }
        return;
      }
#pragma unroll
      for (int u0 = 0; u0 < L * UR; u0 += NTH) {
        const int u = u0 + tid;
        const int j = u / UR, cu = u % UR;
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sH[j * HS + cu * 4]);
        float sm = (x[0] + x[1]) + (x[2] + x[3]);
#pragma unroll
        for (int d = 1; d < UR; d <<= 1) sm += __shfl_xor(sm, d, 64);
        const float mean = sm * (1.f / W);
        float dx[4], sq = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dx[i] = x[i] - mean;
          sq += dx[i] * dx[i];
        }
#pragma unroll
        for (int d = 1; d < UR; d <<= 1) sq += __shfl_xor(sq, d, 64);
        const float rstd = rsqrtf(sq * (1.f / W) + p.gn_eps);
        const int col = cu * 4;
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = dx[i] * rstd * gnw[i] + gnb[i];
        bstore4<T>(rh, ((unsigned)(tc + j) * DV + col) * ES, y[0], y[1], y[2], y[3]);
      }
    } else if constexpr (HST) {
      constexpr int UR = W / VE;  // units per token row
#pragma unroll
      for (int u = tid; u < L * UR; u += NTH) {
        const int j = u / UR, cu = u % UR;
        const u32x4 x = *reinterpret_cast<const u32x4*>(&sH[j * HS + cu * VE]);
        __builtin_amdgcn_raw_buffer_store_b128(x, rh, ((unsigned)(tc + j) * DV + slice * W + cu * VE) * ES, 0, 0);
      }
    }
  };

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * L;
    __syncthreads();  // B1: chunk staged, gate factors ready
    if (c > c_begin) store_h(t0 - L);
    const bool more = c + 1 < c_end;
    const int pb = (c - c_begin) & 1;  // gate vector set of this chunk
    const float* sA2 = sA2b[pb];
    const float* sM2 = sM2b[pb];
    const float* sRS = sRSb[pb];
    const float* sCL = sCLb[pb];
    const float* sBT = sBTb[pb];
    const float* sW = sWb[pb];
    // update of the state is needed unless this is the last chunk of a
    // superchunk whose end state nobody reads
    const bool need_update = more || (sc == p.NS - 1);

    // output-gate values of this wave's outputs, issued at the chunk start
    // so that phase B hides their latency (phase C uses them)
    Raw4<T> oraw[has_o ? JPW : 1][has_o ? CT : 1];
    if constexpr (has_o) {
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          oraw[jj][ct] = bload4_raw<T>(
              ro, ((unsigned)(t0 + (jj * NRG + ((jj & 1) ? NRG - 1 - rg : rg)) * 16 + lr) * DV + wcol0 +
                   ct * 16 + 4 * lg) * ES);
    }

    frag vf[CT][NKL];  // V^T fragments of this wave's columns
    auto load_vf = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) vf[ct][kb] = frag_rows(sV, VS, kb * K, lg, lr, vcol + ct * 16);
    };
    {
      // ---------------------------------------------------------- phase B
      // causal score tiles (key tile lt, query tile jt): the k-th tile of
      // wave w is k NW + w, or k NW + NW - 1 - w for odd k (so that with
      // NTQK < 2 NW the second tiles go to the last waves, not to waves
      // 0 .. NJT-1, which also sum n~.q); a wave's tiles are computed
      // interleaved
      auto tile_of = [](int ti, int& lt, int& jt) __attribute__((always_inline)) {
        lt = 0;
        jt = ti;
        int rem = NJT;
        while (jt >= rem) {  // tile index -> (lt, jt) with lt <= jt
          jt -= rem;
          ++lt;
          --rem;
        }
        jt += lt;
      };
      auto tile_idx = [&](int k) __attribute__((always_inline)) { return k * NW + ((k & 1) ? NW - 1 - w : w); };
      // A rows alternate the hi and lo parts of n~ (only output rows 0 and 1
      // are used, so no select zeroes the others)
      auto n_frag = [&](int kb) __attribute__((always_inline)) {
        return M::load(&sNh[(lr & 1) * DQK + kb * K + KL * lg]);
      };
      auto scores = [&](auto nuc, auto wnc) __attribute__((always_inline)) {
        constexpr int NU = decltype(nuc)::value;
        constexpr bool WN = decltype(wnc)::value;  // also n~ . q of query tile jt[0]
        int lt[NU], jt[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) tile_of(tile_idx(u), lt[u], jt[u]);
        // decay factors of the tiles first: they do not wait for the MFMAs;
        // every read first (unconditional, 16-byte), then the masked exps
        float fac[NU][4];
        {
          float m2[NU];
          float4 a4[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            m2[u] = sM2[jt[u] * 16 + lr];
            a4[u] = *reinterpret_cast<const float4*>(&sA2[lt[u] * 16 + 4 * lg]);
          }
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int j = jt[u] * 16 + lr;
            const float av[4] = {a4[u].x, a4[u].y, a4[u].z, a4[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int l = lt[u] * 16 + 4 * lg + i;
              fac[u][i] = (l <= j) ? exp2_fast(av[i] - m2[u]) : 0.f;
            }
          }
        }
        f32x4 pt[NU][NB];
        f32x4 pn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int be = 0; be < NB; ++be) {
#pragma unroll
          for (int u = 0; u < NU; ++u) pt[u][be] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKQB; ++kk) {
            const int kb = be * NKQB + kk;
            frag kf[NU], qj[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              kf[u] = M::load(&sK[(lt[u] * 16 + lr) * KST + kb * K + KL * lg]);
              qj[u] = M::load(&sQ[(jt[u] * 16 + lr) * QS + kb * K + KL * lg]);
            }
            frag nf;
            if constexpr (WN) nf = n_frag(kb);
#pragma unroll
            for (int u = 0; u < NU; ++u) pt[u][be] = M::mma(kf[u], qj[u], pt[u][be]);
            if constexpr (WN) pn = M::mma(nf, qj[0], pn);
            if (kk & 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (WN) {
          if (lg == 0) sDenInter[jt[0] * 16 + lr] = pn[0] + pn[1];
        }
        // P to LDS, den partial sums (of the fp32 products: summing the
        // bf16-rounded P instead loses too much where the normaliser cancels)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int j = jt[u] * 16 + lr;
          float dsum[NDB];
#pragma unroll
          for (int db = 0; db < NDB; ++db) dsum[db] = 0.f;
#pragma unroll
          for (int be = 0; be < NB; ++be) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[i] = pt[u][be][i] * fac[u][i];
              if constexpr (SN) {
                if (be == 0) dsum[0] += fac[u][i];  // the decay weights alone
              } else {
                dsum[PB ? be : 0] += x[i];
              }
            }
            store4f(&sP[(be * L + j) * PS + kpos4<T>(lt[u] * 16 + 4 * lg)], x[0], x[1], x[2], x[3]);
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const float ds = sum_lane_groups(dsum[db]);
            // the store index is formed here, not hoisted out of the chunk
            // loop (kept live across the loop it would be spilled, and its
            // reload would wait for the h stores in flight)
            int jd = (db * NJT + lt[u]) * L + j;
            asm volatile("" : "+v"(jd));
            if (lg == 0) sDenPart[jd] = ds;
          }
        }
      };
      {
        int nu = 0;  // tiles of this wave (wave-uniform)
#pragma unroll
        for (int k = 0; k < C::NUMAX; ++k) nu += tile_idx(k) < C::NTQK ? 1 : 0;
        auto run = [&](auto wnc) __attribute__((always_inline)) {
          if (nu == 3) {
            if constexpr (C::NUMAX >= 3) scores(std::integral_constant<int, 3>{}, wnc);
          } else if (nu == 2) {
            if constexpr (C::NUMAX >= 2) scores(std::integral_constant<int, 2>{}, wnc);
          } else if (nu == 1) {
            scores(std::integral_constant<int, 1>{}, wnc);
          }
        };
        if constexpr (VN && C::FUSED_NQ) {
          if (w < NJT) run(std::true_type{});  // first tile (0, w): query tile w
          else run(std::false_type{});
        } else {
          run(std::false_type{});
        }
      }
      if constexpr (SN) {  // the inter part of the denominator is n~ itself
        if (w == NW - 1 && lane < L) sDenInter[lane] = sNf[0];
      }
      // n~ . q_j per query tile in a loop of its own (several memory blocks)
      if constexpr (VN && !C::FUSED_NQ) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          if (w == NW - 1 - (jt % NW)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              f32x4 pn = {0.f, 0.f, 0.f, 0.f};
              constexpr int KPB = NKQ / NDB;  // feature k-blocks per denominator
#pragma unroll
              for (int kk = 0; kk < KPB; ++kk) {
                const int kb = db * KPB + kk;
                pn = M::mma(n_frag(kb), M::load(&sQ[(jt * 16 + lr) * QS + kb * K + KL * lg]), pn);
                if (kk & 1) __builtin_amdgcn_sched_barrier(0);
              }
              if (lg == 0) sDenInter[db * L + jt * 16 + lr] = pn[0] + pn[1];
            }
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
      // (the row group is a compile-time constant in each copy of the code)
      if constexpr (XCH) {
        auto exchange = [&](auto rgc) __attribute__((always_inline)) {
          constexpr int RG = decltype(rgc)::value;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
            if (C::owner_of(jt) != RG)
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) sX[((cg * NJT + jt) * CT + ct) * 64 + lane] = acc[jt][ct];
        };
        if (rg == 0) exchange(std::integral_constant<int, 0>{});
        else exchange(std::integral_constant<int, 1>{});
      }
      __syncthreads();  // B2: P, den partials and readout partials ready
      // Q of the next chunk now (sQ is free after B2); its K and V after
      // phase C, so that fewer staging registers are live at once
      if (more) load_q(c + 1);
      load_vf();

      // ---------------------------------------------------------- phase C
      // one copy of the code per row group, so that the token tiles (and the
      // accumulators they select) are compile-time constants
      auto phase_c = [&](auto rgc) __attribute__((always_inline)) {
        constexpr int RG = decltype(rgc)::value;
        // the normaliser of this lane's tokens of every tile, every read first
        const int db = PB ? blk : 0;  // this wave's columns lie in block blk
        float rsv[JPW], invv[JPW];
        {
          float d_in[JPW], d_bt[JPW], d_cl[JPW], d_pt[JPW][NJT];
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) {
            const int j = C::jt_of(RG, jj) * 16 + lr;
            rsv[jj] = sRS[j];
            if constexpr (!RET) {
              d_in[jj] = sDenInter[db * L + j];
              d_bt[jj] = sBT[j];
              d_cl[jj] = sCL[j];
#pragma unroll
              for (int t = 0; t < NJT; ++t) d_pt[jj][t] = sDenPart[(db * NJT + t) * L + j];
            }
          }
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) {
            if constexpr (RET) {
              invv[jj] = 1.f;
            } else {
              float den = rsv[jj] * d_in[jj] + d_bt[jj];
#pragma unroll
              for (int t = 0; t < NJT; ++t) den += d_pt[jj][t];
              invv[jj] = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), d_cl[jj]));
            }
          }
        }
        const float sig_scale = exp2_fast(sig);
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          const int jt = C::jt_of(RG, jj);  // compile-time after unrolling
          // intra-chunk part first, from zero: its MFMAs do not wait for the
          // exchanged readout partials
          f32x4 o_acc[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) o_acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKL; ++kb) {
            if (kb * K <= jt * 16 + 15) {
              const frag pf = M::load(&sP[(blk * L + jt * 16 + lr) * PS + kb * K + KL * lg]);
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) o_acc[ct] = M::mma(vf[ct][kb], pf, o_acc[ct]);
            }
          }
          const int j = jt * 16 + lr;
          const float rs_state = rsv[jj] * sig_scale;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            f32x4 a = acc[jt][ct];
            if constexpr (XCH) a += sX[((cg * NJT + jt) * CT + ct) * 64 + lane];
            o_acc[ct] += rs_state * a;
          }
          const float inv = invv[jj];
          // rows past T fall outside the output buffer and are dropped
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int col = wcol0 + ct * 16 + 4 * lg;
            float o[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (has_o) {
              raw4_to_f32<T>(oraw[jj][ct], o);
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = sigmoidf_(o[i]);
            }
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = o[i] * o_acc[ct][i] * inv;
            if constexpr (HST)
              store4f(&sH[j * HS + cg * WC + ct * 16 + 4 * lg], hv[0], hv[1], hv[2], hv[3]);
            else
              bstore4<T>(rh, ((unsigned)(t0 + j) * DV + col) * ES, hv[0], hv[1], hv[2], hv[3]);
          }
        }
      };
      if constexpr (NRG == 1) phase_c(std::integral_constant<int, 0>{});
      else if (rg == 0) phase_c(std::integral_constant<int, 0>{});
      else phase_c(std::integral_constant<int, 1>{});
    }

    // The update's B operands, w (x) V^T with w scaled by 2^-sig, are formed
    // after the next chunk's staging loads and before the update, so that
    // their LDS reads and VALU work do not sit between the update's K^T reads
    // and its MFMAs.  The register scale sig is decided first: when it would
    // drop below -64 the state is rescaled to sig = 0 before the update.
    const float la = sAlphab[pb];
    const float sig_new = sig + la;
    const bool rescale = sig_new < -64.f;  // wave-uniform, rare
    if (more) {
      store_q();
      load_kv(c + 1);
    }
    frag wv[CT][NKL];
    if (need_update) {
      const float wscale = exp2_fast(rescale ? 0.f : -sig_new);
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb) {
        float wls[KL];
#pragma unroll
        for (int e = 0; e < KL; ++e) wls[e] = sW[kb * K + krow<T>(lg, e)] * wscale;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) wv[ct][kb] = scale_frag(vf[ct][kb], wls);
      }
    }
    // ------------------------------------------------------- state update
    if (need_update) {
      const float alpha = exp2_fast(la);
      if (rescale) {
        const float f = exp2_fast(sig_new);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st[nt][ct] *= f;
        sig = 0.f;
      } else {
        sig = sig_new;
      }
      // n~ gets sum_l w_l k_l.  With one memory block the K^T fragments of the
      // update carry every feature of k: each is summed by one wave (tile nt
      // goes to column group nt % 4).  With several blocks a work-group's waves
      // need not cover all blocks, so a plain loop over sK does it.
      constexpr bool NFRAG = VN && NB == 1;
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int kc = BF ? kcol + (nt >> 1) * 32 + (nt & 1) * 4 : kcol + perm_row<T>(nt, lr);
          const frag ka = frag_rows(sK, KST, kb * K, lg, lr, kc);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st[nt][ct] = M::mma(ka, wv[ct][kb], st[nt][ct]);
          if ((nt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (VN && !NFRAG) {
        // PPF adjacent lanes per feature, each summing L / PPF tokens with its
        // reads issued together; the partial sums meet by xor shuffles
        constexpr int PPF = NTH >= DQK ? (NTH / DQK > 8 ? 8 : NTH / DQK) : 1;
        constexpr int LP = L / PPF;
        static_assert(L % PPF == 0 && (PPF & (PPF - 1)) == 0, "token parts");
        const int part = tid % PPF;
        for (int r = tid / PPF; r < DQK; r += NTH / PPF) {
          float kv[LP], wl[LP];
#pragma unroll
          for (int l = 0; l < LP; ++l) {
            kv[l] = to_f32(sK[(part * LP + l) * KST + r]);
            wl[l] = sW[part * LP + l];
          }
          float x = 0.f;
#pragma unroll
          for (int l = 0; l < LP; ++l) x += wl[l] * kv[l];
#pragma unroll
          for (int d = 1; d < PPF; d <<= 1) x += __shfl_xor(x, d, 64);
          if (part == 0) put_n(r, alpha * sNf[r] + x);
        }
      }
      if constexpr (SN) {  // n~ <- alpha n~ + sum_l w_l, summed by the last wave
        if (w == NW - 1) {
          float x = lane < L ? sW[lane] : 0.f;
#pragma unroll
          for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d, 64);
          if (lane == 0) put_n(0, alpha * sNf[0] + x);
        }
      }
      if constexpr (NFRAG) {
        // rows of tiles nt = cg, cg + NCG, ...: their K^T fragments are read
        // again here, all before the first is used, so that no branch splits
        // the MFMA loop above
        constexpr int NJ = (NT + NCG - 1) / NCG;
        float d[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          d[j] = 0.f;
          const int nt = j * NCG + cg;  // wave-uniform
          if (NT % NCG == 0 || nt < NT) {
#pragma unroll
            for (int kb = 0; kb < NKL; ++kb) {
              const int kc = BF ? kcol + (nt >> 1) * 32 + (nt & 1) * 4 : kcol + perm_row<T>(nt, lr);
              const frag ka = frag_rows(sK, KST, kb * K, lg, lr, kc);
#pragma unroll
              for (int e = 0; e < KL; ++e) {
                const float wl = sW[kb * K + krow<T>(lg, e)];
                if constexpr (BF) d[j] += wl * (float)ka[e];
                else d[j] += wl * ka;
              }
            }
          }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int nt = j * NCG + cg;
          if (NT % NCG == 0 || nt < NT) {
            const float x = sum_lane_groups(d[j]);
            if (lg == 0) {
              const int r = rb0 + perm_row<T>(nt, lr);
              put_n(r, alpha * sNf[r] + x);
            }
          }
        }
      }
    }
    // the next chunk's gate vectors into the other set (its loads were
    // issued before the update)
    if (more && w == 0) gates(pb ^ 1);
    __syncthreads();  // B3: LDS free for the next chunk
    if (more) store_kv();
  }
  store_h((c_end - 1) * L);

  // ---------------------------------------------------------------- outputs
  float* Sdst = nullptr;
  if (sc == p.NS - 1 && p.C_out) Sdst = p.C_out + (size_t)bh * CS;  // [B,H,NB,DQKB,DVB]
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
  if (slice == 0 && sc == p.NS - 1) {
    if constexpr (!RET) {
      if (p.n_out) {
        if constexpr (SN) {
          if (tid == 0) p.n_out[bh] = sNf[0];
        } else {
          for (int r = tid; r < DQK; r += NTH) p.n_out[(size_t)bh * DQK + r] = sNf[r];
        }
      }
    }
    if (tid == 0 && p.m_out) p.m_out[bh] = m_prev * kLn2;
  }
}

// Pass 3, wave-specialised form for the xLSTM-7B head shape (bf16, d_qk = 256,
// one memory block, chunks of 64 tokens, 128 d_v columns per work-group).
// Same arithmetic as chunk_kernel, split by role so that the MFMA pipes of
// every SIMD see one wave that streams products while another wave on the same
// SIMD does the loads, scores, normaliser and gate work:
//   state waves 0..3  own all 256 state rows x 32 columns each (fp32, in MFMA
//                     accumulator registers): readout S~^T q and n~ . q (hi +
//                     lo bf16 rows of n~), P V, outputs, state update, and
//                     the n~ update of 64 features each (by MFMA, w as hi +
//                     lo bf16).  No exchange between waves.
//   helper waves 4..7 stage the next chunk (global loads into registers,
//                     then LDS), compute the chunk's causal score tiles with
//                     their decay factors (P to LDS, fp32 row sums for the
//                     denominator) and the gate vectors of the next chunk
//                     (the m_prev chain).
// K and V are double-buffered in LDS (the next chunk's go into the other
// buffer while the state waves update from the current one), as are the
// gate vectors and n~, so a chunk needs two work-group barriers:
//   A: the chunk's Q, K, V, gate vectors and n~ are in LDS;
//      state waves: readout, n~ . q; helpers: scores, P and den partials.
//   B: P and the denominators are in LDS, Q is free;
//      state waves: P V, outputs, update, n~ of the next chunk; helpers: the
//      next chunk's Q, K, V and gate vectors into LDS, then the loads of the
//      chunk after.
// The wave-uniform choices (which query tile a state wave takes n~ . q for,
// which features it updates) are address offsets, never register selects,
// and no LDS read is waited for inside a product loop.
template <bool HAS_O, bool SN, bool DIR = false>
__global__ __launch_bounds__(512) void chunk_kernel_ws(ChunkParams p) {
  using T = __bf16;
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int DQK = 256, L = 64, W = 128, WC = 32, CT = 2, NT = 16, NJT = 4, NKL = 2;
  constexpr int K = M::K, KL = M::KL;
  constexpr int VE = 8;  // bf16 elements per 16 bytes
  constexpr int QS = DQK + lds_pad_res(DQK, 2, MLSTM_P3_QRES);
  constexpr int KST = DQK + lds_pad_res(DQK, 2, MLSTM_P3_QRES);  // two K buffers: the smaller padding
  constexpr int VS = W + lds_row_pad(W, 2);
  constexpr int PS = L + 8;
  constexpr unsigned ES = 2;
  constexpr int NTQK = NJT * (NJT + 1) / 2;  // causal score tiles

  __shared__ __attribute__((aligned(16))) T sQ[L * QS];
  __shared__ __attribute__((aligned(16))) T sK[2][L * KST];
  __shared__ __attribute__((aligned(16))) T sV[2][L * VS];
  __shared__ __attribute__((aligned(16))) T sP[L * PS];
  __shared__ __attribute__((aligned(16))) T sNh[2][2 * DQK];  // n~ as hi / lo bf16 rows, two sets
  __shared__ __attribute__((aligned(16))) float sNf[2][DQK];
  __shared__ __attribute__((aligned(16))) float sA2b[2][L];
  __shared__ float sM2b[2][L], sRSb[2][L], sCLb[2][L], sBTb[2][L];
  __shared__ __attribute__((aligned(16))) float sWb[2][L];
  __shared__ float sDenPart[NJT * L];
  __shared__ float sDenInter[L];
  __shared__ float sAlphab[2];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool state_wave = w < 4;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int BH = p.B * p.H;
  const int idx = blockIdx.x;
  const int bh = __builtin_amdgcn_readfirstlane(idx % BH);
  const int slice = __builtin_amdgcn_readfirstlane((idx / BH) % p.nslices);
  const int sc = __builtin_amdgcn_readfirstlane((idx / BH) / p.nslices);
  const int hd = __builtin_amdgcn_readfirstlane(bh % p.H);
  const int T_ = p.T, DV = p.DV;
  const size_t CS = (size_t)DQK * DV;
  const size_t NSTATE = CS + DQK;
  const int c_begin = sc * p.G;
  const int c_end = min(c_begin + p.G, p.NC);

  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * T_ * DV, (unsigned)T_ * DV * ES);
  const size_t NCL = (size_t)p.NC * L;
  const auto rga_r = make_rsrc(p.ws_ga + (size_t)bh * NCL, (unsigned)NCL * 4u);
  const auto rgg_r = make_rsrc(p.ws_gg + (size_t)bh * NCL, (unsigned)NCL * 4u);
  const auto rgb_r = make_rsrc(p.ws_gb + (size_t)bh * NCL, (unsigned)NCL * 4u);
  const auto ro = make_rsrc(HAS_O ? static_cast<const T*>(p.o_pre) + (size_t)bh * T_ * DV : nullptr,
                            HAS_O ? (unsigned)T_ * DV * ES : 0u);
  const auto rh = make_rsrc(static_cast<T*>(p.h) + (size_t)bh * T_ * DV, (unsigned)T_ * DV * ES);
  const float bias = p.bias ? p.bias[hd] : 0.f;
  // the start state through a descriptor that is empty when there is none
  // (reads zero): the loads need no branch and go out back to back
  // (a direct call reads the caller's C0 and n0, a planned one its slot of
  // superchunk start states, whose n~ follows the matrix)
  const bool has_in = DIR ? p.C0 != nullptr : (sc > 0 || p.has_init);
  const float* sbase = DIR ? (p.C0 ? p.C0 + (size_t)bh * CS : nullptr) : p.ws_state + ((size_t)bh * p.NS + sc) * NSTATE;
  const auto rSin = make_rsrc(sbase, has_in ? (unsigned)((DIR ? CS : NSTATE) * 4) : 0u);
  constexpr int NN = SN ? 1 : DQK;  // entries of a caller's n0 per (batch, head)
  const bool has_n = DIR ? p.n0 != nullptr : has_in;
  const float* nbase = DIR ? (p.n0 ? p.n0 + (size_t)bh * NN : nullptr) : sbase + CS;
  const auto rNin = make_rsrc(nbase, has_n ? (unsigned)((DIR ? NN : DQK) * 4) : 0u);
  // the gate preactivations, read by a direct call (helper 0)
  const auto ri_d = make_rsrc(DIR ? static_cast<const T*>(p.i_pre) + (size_t)bh * T_ : nullptr,
                              DIR ? (unsigned)T_ * ES : 0u);
  const auto rf_d = make_rsrc(DIR ? static_cast<const T*>(p.f_pre) + (size_t)bh * T_ : nullptr,
                              DIR ? (unsigned)T_ * ES : 0u);

  // n~ into set s: fp32 and as the hi / lo rows of the den tile
  auto put_n = [&](int s, int r, float x) __attribute__((always_inline)) {
    sNf[s][r] = x;
    const T hi = (T)x;
    sNh[s][r] = hi;
    sNh[s][DQK + r] = (T)(x - (float)hi);
  };
  if constexpr (DIR) {
    for (int r = tid; r < DQK; r += 512) put_n(0, r, bload1<float>(rNin, (unsigned)r * 4u));
  } else {
    for (int r = tid; r < DQK; r += 512) put_n(0, r, bload1<float>(rSin, (unsigned)(CS + r) * 4u));
  }
  for (int e = tid; e < L * PS; e += 512) sP[e] = (T)0.f;  // masked tiles are never written
  for (int e = tid; e < NJT * L; e += 512) sDenPart[e] = 0.f;

  // ------------------------------------------------------------ helper waves
  // Staging: helper thread ht of 256 holds 16-byte units ht + 256 it of the
  // next chunk's Q (8), K (8) and V slice (4) between their loads and their
  // LDS stores.
  const int ht = tid - 256;
  const int hw = w - 4;  // helper index
  Vec16<T> gq[8], gk[8], gv[4];
  unsigned rga = 0, rgg = 0, rgb = 0;  // chunk-local gate logs of the next chunk (helper 0)
  // stabiliser chain, kept by helper 0
  float m_prev = DIR ? (p.m0 ? p.m0[bh] * kLog2e : 0.f) : p.ws_min[(size_t)bh * p.NS + sc];
  unsigned rgt = 0;  // first token of the loaded chunk (direct calls: i, f in rga, rgg)

  auto h_load = [&](int c) __attribute__((always_inline)) {
    const unsigned t0 = (unsigned)c * L;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = ht + it * 256;
      const unsigned j = u >> 5, col = (u & 31) * VE;
      gq[it] = bload16<T>(rq, ((t0 + j) * DQK + col) * ES);
      gk[it] = bload16<T>(rk, ((t0 + j) * DQK + col) * ES);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = ht + it * 256;
      const unsigned j = u >> 4, col = (u & 15) * VE;
      gv[it] = bload16<T>(rv, ((t0 + j) * DV + slice * W + col) * ES);
    }
    if (hw == 0) {
      rgt = t0;
      if constexpr (DIR) {
        rga = __float_as_uint(bload1<T>(ri_d, (t0 + (unsigned)lane) * ES));
        rgg = __float_as_uint(bload1<T>(rf_d, (t0 + (unsigned)lane) * ES));
      } else {
        const unsigned o = (t0 + (unsigned)lane) * 4u;
        rga = bload1_raw<float>(rga_r, o);
        rgg = bload1_raw<float>(rgg_r, o);
        rgb = bload1_raw<float>(rgb_r, o);
      }
    }
  };
  auto h_store = [&](int kv) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = ht + it * 256;
      const int j = u >> 5, col = (u & 31) * VE;
      *reinterpret_cast<uint4*>(&sQ[j * QS + col]) = *reinterpret_cast<const uint4*>(gq[it].v);
      *reinterpret_cast<uint4*>(&sK[kv][j * KST + col]) = *reinterpret_cast<const uint4*>(gk[it].v);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = ht + it * 256;
      const int j = u >> 4, col = (u & 15) * VE;
      *reinterpret_cast<uint4*>(&sV[kv][j * VS + col]) = *reinterpret_cast<const uint4*>(gv[it].v);
    }
  };
  // n~ of the next chunk into set pb ^ 1: alpha n~ + sum_l w_l k_l over the
  // 64 features [fw, fw + 64), by MFMA: K^T fragments of buffer pb times an
  // all-columns B operand of w (its hi and lo bf16 parts, wk = w at this
  // lane's fragment tokens krow(lg, 0..7) of each k-block), 4 MFMAs per
  // 16-feature tile.  Two tiles at a time: their reads are issued first,
  // then 8 MFMAs of 2 independent chains; the lanes of column 0 store 4
  // features each.
  auto n_update = [&](int pb, int fw, const float (&wk)[2][KL], float alpha) __attribute__((always_inline)) {
    const T* sKc = sK[pb];
    frag whi[NKL], wlo[NKL];
#pragma unroll
    for (int kb = 0; kb < NKL; ++kb)
#pragma unroll
      for (int e = 0; e < KL; ++e) {
        const T hi = (T)wk[kb][e];
        whi[kb][e] = hi;
        wlo[kb][e] = (T)(wk[kb][e] - (float)hi);
      }
#pragma unroll
    for (int t0 = 0; t0 < 4; t0 += 2) {
      frag ka[2][NKL];
      float4 nold[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb)
          ka[t][kb] = frag_rows(sKc, KST, kb * K, lg, lr, fw + 16 * (t0 + t) + 4 * (lr & 3));
        nold[t] = *reinterpret_cast<const float4*>(&sNf[pb][fw + 16 * (t0 + t) + 4 * lg]);
      }
      f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) d[t] = M::mma(ka[t][kb], whi[kb], d[t]);
#pragma unroll
        for (int t = 0; t < 2; ++t) d[t] = M::mma(ka[t][kb], wlo[kb], d[t]);
      }
      if (lr == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = fw + 16 * (t0 + t) + 4 * lg;  // features r .. r + 3
          const float x[4] = {alpha * nold[t].x + d[t][0], alpha * nold[t].y + d[t][1], alpha * nold[t].z + d[t][2],
                              alpha * nold[t].w + d[t][3]};
          *reinterpret_cast<float4*>(&sNf[pb ^ 1][r]) = make_float4(x[0], x[1], x[2], x[3]);
          T hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hi[i] = (T)x[i];
            lo[i] = (T)(x[i] - (float)hi[i]);
          }
          *reinterpret_cast<uint2*>(&sNh[pb ^ 1][r]) = *reinterpret_cast<const uint2*>(hi);
          *reinterpret_cast<uint2*>(&sNh[pb ^ 1][DQK + r]) = *reinterpret_cast<const uint2*>(lo);
        }
      }
    }
  };
  // gate vectors of the loaded chunk into set gb (helper 0, one lane per token)
  auto h_gates = [&](int gb) __attribute__((always_inline)) {
    float a = __uint_as_float(rga), g = __uint_as_float(rgg), b = __uint_as_float(rgb);
    if constexpr (DIR) {
      // the gate pass's chunk-local logs, formed here: tokens past T count
      // as f = 1, i = 0
      const bool valid = rgt + (unsigned)lane < (unsigned)T_;
      const float lf2 = valid ? log2_sigmoid(__uint_as_float(rgg)) : 0.f;
      const float li = valid ? __uint_as_float(rga) * kLog2e : -INFINITY;
      b = seg_scan_sum(lf2, L);
      a = li - b;
      g = seg_scan_max(a, L);
    }
    const float Mj = fmaxf(m_prev, g);
    const float gL = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(g), L - 1));
    const float bL = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(b), L - 1));
    const float ML = fmaxf(m_prev, gL);
    const float mj = b + Mj;
    const float cl = exp2_fast(-mj);
    sA2b[gb][lane] = a;
    sM2b[gb][lane] = Mj;
    sRSb[gb][lane] = exp2_fast(m_prev - Mj);
    sCLb[gb][lane] = cl;
    sBTb[gb][lane] = bias * cl;
    sWb[gb][lane] = exp2_fast(a - ML);
    if (lane == 0) sAlphab[gb] = m_prev - ML;
    m_prev = bL + ML;
  };

  // ------------------------------------------------------------- state waves
  // Wave s owns columns [32 s, 32 s + 32) of the slice and every state row,
  // rows stored in perm_row order so that the accumulators are the readout's
  // A operand.
  // The two roles run separate loops with the same two barriers per chunk
  // (their registers never live at the same time).
  if (state_wave) {
  if constexpr (MLSTM_P3_PRIO >= 2) __builtin_amdgcn_s_setprio(1);
  const int sw = w;
  const int wcol0 = slice * W + sw * WC;  // first global d_v column of this state wave
  f32x4 st[NT][CT];
  const int soff = perm_row_lane<T>(lg) * DV + wcol0 + lr;
  if constexpr (DIR) {
    // the caller's C0 in its own order
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[nt][ct][i] = bload1<float>(rSin, (unsigned)(soff + perm_row_uni<T>(nt, i) * DV + ct * 16) * 4u);
  } else {
    // a slot of pass 2 in the register order: one 16-byte load per tile
    const unsigned so4 = (unsigned)(((wcol0 >> 5) * 32 * 64 + lane) * 16);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        st[nt][ct] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rSin, so4 + (unsigned)((nt * 2 + ct) * 64 * 16), 0, 0));
  }
  float sig = 0.f;  // the registers hold S~ / 2^sig (lazy decay)
  const int vcol = sw * WC + 4 * (lr & 3);  // transposing-read source column of V^T (+ 16 ct)
  const int kcol = 8 * (lr & 3);            // ... of K^T (+ perm part per tile)
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * L;
    const int pb = (c - c_begin) & 1;  // buffer / set of this chunk
    const bool need_update = c + 1 < c_end || (sc == p.NS - 1);
    __syncthreads();  // A
    {
      // readout of the state at the chunk start: acc[jt][ct] = S~[:, c]^T q_j
      f32x4 acc[NJT][CT];
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[jt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      // n~ . q_j of query tile sw alongside: the A rows alternate the hi and
      // lo bf16 parts of n~ (only output rows 0 and 1 are used), B is this
      // wave's query tile read once more at a wave-uniform offset (no
      // register selects)
      f32x4 pn = {0.f, 0.f, 0.f, 0.f};
      const T* nhl = &sNh[pb][(lr & 1) * DQK + KL * lg];
      const T* qsw = &sQ[(sw * 16 + lr) * QS + KL * lg];
#pragma unroll
      for (int kk = 0; kk < DQK / K; ++kk) {
        frag qf[NJT];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) qf[jt] = M::load(&sQ[(jt * 16 + lr) * QS + kk * K + KL * lg]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const frag sf = StateFrag<T, NT, CT>::get(st, kk, ct);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) acc[jt][ct] = M::mma(sf, qf[jt], acc[jt][ct]);
        }
        if constexpr (!SN) pn = M::mma(M::load(nhl + kk * K), M::load(qsw + kk * K), pn);
      }
      if constexpr (SN) {  // the inter part of the denominator is n~ itself
        if (sw == 0) sDenInter[lane] = sNf[pb][0];
      } else {
        if (lg == 0) sDenInter[sw * 16 + lr] = pn[0] + pn[1];
      }
      // output-gate values of this wave's outputs, issued after the readout
      // (not live across it) so that the wait at barrier B hides their
      // latency: 16 bytes per lane in the column order of the output stores
      // below, swapped back into the MFMA layout where they are used
      u32x4 oq[HAS_O ? NJT : 1];
      if constexpr (HAS_O) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
          oq[jt] = __builtin_amdgcn_raw_buffer_load_b128(
              ro, ((unsigned)(t0 + jt * 16 + lr) * DV + wcol0 + ((lg & 1) << 4) + ((lg >> 1) << 3)) * ES, 0, 0);
      }
      __syncthreads();  // B
      const float* sA2 = sA2b[pb];
      const float* sRS = sRSb[pb];
      const float* sCL = sCLb[pb];
      const float* sBT = sBTb[pb];
      const float* sW = sWb[pb];
      const T* sVc = sV[pb];
      frag vf[CT][NKL];  // V^T fragments of this wave's columns
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) vf[ct][kb] = frag_rows(sVc, VS, kb * K, lg, lr, vcol + ct * 16);
      // the normaliser of this lane's tokens, every read first
      float rsj[NJT], invj[NJT];
      {
        float d_in[NJT], d_bt[NJT], d_cl[NJT], d_pt[NJT][NJT];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          const int j = jt * 16 + lr;
          rsj[jt] = sRS[j];
          d_in[jt] = sDenInter[j];
          d_bt[jt] = sBT[j];
          d_cl[jt] = sCL[j];
#pragma unroll
          for (int t = 0; t < NJT; ++t) d_pt[jt][t] = sDenPart[t * L + j];
        }
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          float den = rsj[jt] * d_in[jt] + d_bt[jt];
#pragma unroll
          for (int t = 0; t < NJT; ++t) den += d_pt[jt][t];
          invj[jt] = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), d_cl[jt]));
        }
      }
      const float sig_scale = exp2_fast(sig);
      // P V, combine, outputs
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        f32x4 o_acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o_acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) {
          if (kb * K <= jt * 16 + 15) {
            const frag pf = M::load(&sP[(jt * 16 + lr) * PS + kb * K + KL * lg]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) o_acc[ct] = M::mma(vf[ct][kb], pf, o_acc[ct]);
          }
        }
        const int j = jt * 16 + lr;
        const float rs_state = rsj[jt] * sig_scale;
        const float inv = invj[jt];
        unsigned pk[CT][2];  // this lane's 4 outputs of each column tile, as bf16 pairs
        Raw4<T> oraw[CT];
        if constexpr (HAS_O) {
          const auto y0 = __builtin_amdgcn_permlane16_swap(oq[jt][0], oq[jt][2], false, false);
          const auto y1 = __builtin_amdgcn_permlane16_swap(oq[jt][1], oq[jt][3], false, false);
          oraw[0].v = u32x2{y0[0], y1[0]};
          oraw[1].v = u32x2{y0[1], y1[1]};
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          float o[4] = {1.f, 1.f, 1.f, 1.f};
          if constexpr (HAS_O) {
            raw4_to_f32<T>(oraw[ct], o);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = sigmoidf_(o[i]);
          }
          float hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = o[i] * (o_acc[ct][i] + rs_state * acc[jt][ct][i]) * inv;
          pk[ct][0] = pack_bf16x2(hv[0], hv[1]);
          pk[ct][1] = pack_bf16x2(hv[2], hv[3]);
        }
        // 16-lane group g holds columns 4g..4g+3 of both tiles; swapping the
        // odd groups' tile 0 with the even groups' tile 1 gives each lane 8
        // adjacent columns (groups 0..3: 0-7, 16-23, 8-15, 24-31), one
        // 16-byte store (rows past T fall outside the buffer and are dropped)
        const auto x0 = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
        const auto x1 = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
        const u32x4 hq = {x0[0], x1[0], x0[1], x1[1]};
        __builtin_amdgcn_raw_buffer_store_b128(
            hq, rh, ((unsigned)(t0 + j) * DV + wcol0 + ((lg & 1) << 4) + ((lg >> 1) << 3)) * ES, 0, 0);
      }
      // state update: S^ <- S^ + 2^{-sig'} (w . K)^T V (the chunk's decay is
      // folded into sig; rescaled once sig drops below -64)
      if (need_update) {
        const float la = sAlphab[pb];
        const float sig_new = sig + la;
        const bool rescale = sig_new < -64.f;  // wave-uniform, rare
        const float wscale = exp2_fast(rescale ? 0.f : -sig_new);
        // w of this lane's fragment rows
        float wk[NKL][KL];
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb)
#pragma unroll
          for (int e = 0; e < KL; ++e) wk[kb][e] = sW[kb * K + krow<T>(lg, e)];
        frag wv[CT][NKL];
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) {
          float wls[KL];
#pragma unroll
          for (int e = 0; e < KL; ++e) wls[e] = wk[kb][e] * wscale;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) wv[ct][kb] = scale_frag(vf[ct][kb], wls);
        }
        if (rescale) {
          const float f = exp2_fast(sig_new);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) st[nt][ct] *= f;
          sig = 0.f;
        } else {
          sig = sig_new;
        }
        const T* sKc = sK[pb];
        // pairs of row tiles; the K^T fragments of the next UD pairs are
        // read while the current pair multiplies
        constexpr int NG = NKL * NT / 2;
        constexpr int UD = MLSTM_P3_UPD, UB = UD + 1;
        frag ka[UB][2];
        auto load_g = [&](int g, int b) __attribute__((always_inline)) {
          const int kb = g / (NT / 2), nt0 = (g % (NT / 2)) * 2;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int nt = nt0 + q;
            ka[b][q] = frag_rows(sKc, KST, kb * K, lg, lr, kcol + (nt >> 1) * 32 + (nt & 1) * 4);
          }
        };
#pragma unroll
        for (int g = 0; g < UD; ++g) load_g(g, g);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g + UD < NG) load_g(g + UD, (g + UD) % UB);
          const int kb = g / (NT / 2), nt0 = (g % (NT / 2)) * 2;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) st[nt0 + q][ct] = M::mma(ka[g % UB][q], wv[ct][kb], st[nt0 + q][ct]);
        }
        // n~ of the next chunk: features [64 sw, 64 sw + 64) from this wave
        const float alpha = exp2_fast(la);
        if constexpr (SN) {
          if (sw == 0) {
            float x = sW[lane];
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d, 64);
            if (lane == 0) put_n(pb ^ 1, 0, alpha * sNf[pb][0] + x);
          }
        } else {
          n_update(pb, 64 * sw, wk, alpha);
        }
      }
      (void)sA2;
    }
  }
  __syncthreads();
  if (sc == p.NS - 1 && p.C_out) {
    float* Sdst = p.C_out + (size_t)bh * CS;
    const float f = exp2_fast(sig);
    int so = soff;
    asm volatile("" : "+v"(so));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sdst[so + perm_row_uni<T>(nt, i) * DV + ct * 16] = st[nt][ct][i] * f;
  }
  } else {
  // ------------------------------------------------------------ helper waves
  // prime: the first chunk in LDS, the second one's loads in flight
  h_load(c_begin);
  h_store(0);
  if (hw == 0) h_gates(0);
  if (c_begin + 1 < c_end) h_load(c_begin + 1);
  for (int c = c_begin; c < c_end; ++c) {
    const int pb = (c - c_begin) & 1;  // buffer / set of this chunk
    const bool more = c + 1 < c_end;
    const bool need_update = more || (sc == p.NS - 1);
    __syncthreads();  // A
    if constexpr (MLSTM_P3_PRIO == 1 || MLSTM_P3_PRIO == 2) __builtin_amdgcn_s_setprio(2);
    {
      const float* sA2 = sA2b[pb];
      const float* sM2 = sM2b[pb];
      const T* sKc = sK[pb];
      // score tiles (key tile lt, query tile jt): the k-th tile of helper hw
      // is k 4 + hw for even k, k 4 + 3 - hw for odd k; the first is (0, hw),
      // which also sums n~ . q_j of query tile hw
      auto tile_of = [](int ti, int& lt, int& jt) __attribute__((always_inline)) {
        lt = 0;
        jt = ti;
        int rem = NJT;
        while (jt >= rem) {
          jt -= rem;
          ++lt;
          --rem;
        }
        jt += lt;
      };
      auto scores = [&](auto nuc) __attribute__((always_inline)) {
        constexpr int NU = decltype(nuc)::value;
        int lt[NU], jt[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) tile_of(u * 4 + ((u & 1) ? 3 - hw : hw), lt[u], jt[u]);
        // decay factors 2^(a_l - M_j) of this lane's 4 tokens l per tile:
        // every read first (unconditional, 16-byte), then the masked exps
        float fac[NU][4];
        {
          float m2[NU];
          float4 a4[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            m2[u] = sM2[jt[u] * 16 + lr];
            a4[u] = *reinterpret_cast<const float4*>(&sA2[lt[u] * 16 + 4 * lg]);
          }
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int j = jt[u] * 16 + lr;
            const float av[4] = {a4[u].x, a4[u].y, a4[u].z, a4[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int l = lt[u] * 16 + 4 * lg + i;
              fac[u][i] = (l <= j) ? exp2_fast(av[i] - m2[u]) : 0.f;
            }
          }
        }
        f32x4 pt[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) pt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        // fragments of k-blocks kb + 1 .. kb + SD are read while those of kb
        // multiply
        constexpr int SD = MLSTM_P3_SCD, SB = SD + 1;
        frag kf[SB][NU], qj[SB][NU];
        auto load_kb = [&](int kb, int b) __attribute__((always_inline)) {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            kf[b][u] = M::load(&sKc[(lt[u] * 16 + lr) * KST + kb * K + KL * lg]);
            qj[b][u] = M::load(&sQ[(jt[u] * 16 + lr) * QS + kb * K + KL * lg]);
          }
        };
#pragma unroll
        for (int kb = 0; kb < SD; ++kb) load_kb(kb, kb);
#pragma unroll
        for (int kb = 0; kb < DQK / K; ++kb) {
          if (kb + SD < DQK / K) load_kb(kb + SD, (kb + SD) % SB);
#pragma unroll
          for (int u = 0; u < NU; ++u) pt[u] = M::mma(kf[kb % SB][u], qj[kb % SB][u], pt[u]);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int j = jt[u] * 16 + lr;
          float x[4], dsum = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = pt[u][i] * fac[u][i];
            dsum += SN ? fac[u][i] : x[i];
          }
          store4f(&sP[j * PS + kpos4<T>(lt[u] * 16 + 4 * lg)], x[0], x[1], x[2], x[3]);
          const float ds = sum_lane_groups(dsum);
          if (lg == 0) sDenPart[lt[u] * L + j] = ds;
        }
      };
      if (hw < 2) scores(std::integral_constant<int, 3>{});
      else scores(std::integral_constant<int, 2>{});
      if constexpr (MLSTM_P3_PRIO == 1 || MLSTM_P3_PRIO == 2) __builtin_amdgcn_s_setprio(0);
      __syncthreads();  // B
      if (more) {
        h_store(pb ^ 1);  // Q, K, V of the next chunk (loaded during the previous one)
        if (hw == 0) h_gates(pb ^ 1);
      }
      if (c + 2 < c_end) h_load(c + 2);  // the chunk after: in flight during the rest
    }
  }
  __syncthreads();
  if (slice == 0 && sc == p.NS - 1) {
    const int s_end = (c_end - c_begin) & 1;  // set holding n~ after the last chunk
    if (p.n_out) {
      if constexpr (SN) {
        if (ht == 0) p.n_out[bh] = sNf[s_end][0];
      } else {
        for (int r = ht; r < DQK; r += 256) p.n_out[(size_t)bh * DQK + r] = sNf[s_end][r];
      }
    }
    if (w == 4 && lane == 0 && p.m_out) p.m_out[bh] = m_prev * kLn2;
  }
  }
}

// Row pass of the group norm for heads wider than a pass-3 work-group: one
// wave per output row (b, h, t) of d_v fp32 values in gn_ws; mean, then the
// biased variance of the centred values, then y = (x - mean) rsqrt(var + eps)
// w + b into h in the output dtype (the arithmetic of the fused form).
template <typename T>
__global__ __launch_bounds__(256) void groupnorm_rows_kernel(const float* __restrict__ x, T* __restrict__ y,
                                                             long long rows, int T_, int H, int DV,
                                                             const float* __restrict__ gw,
                                                             const float* __restrict__ gb, float eps) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int hd = (int)((r / T_) % H);
  const float* xr = x + r * DV;
  float sm = 0.f;
  for (int c = lane; c < DV; c += 64) sm += xr[c];
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) sm += __shfl_xor(sm, d, 64);
  const float mean = sm / (float)DV;
  float sq = 0.f;
  for (int c = lane; c < DV; c += 64) {
    const float dx = xr[c] - mean;
    sq += dx * dx;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) sq += __shfl_xor(sq, d, 64);
  const float rstd = rsqrtf(sq / (float)DV + eps);
  T* yr = y + r * DV;
  for (int c = lane; c < DV; c += 64) {
    const float wv = gw ? gw[(size_t)hd * DV + c] : 1.f;
    const float bv = gb ? gb[(size_t)hd * DV + c] : 0.f;
    yr[c] = (T)((xr[c] - mean) * rstd * wv + bv);
  }
}

// s_waitcnt with only a vmcnt limit (gfx9 encoding, expcnt and lgkmcnt left
// at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// LDS accesses of this wave done, then a work-group barrier; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Gates, per (batch*head, superchunk).  For every token, in base-2 logs:
//   chunk-local, for pass 3 (chunks of L tokens, index j):
//     b_j = sum_{r<=j} log2 sigmoid(f_r),  a_j = log2(i_j) - b_j,
//     g_j = max_{r<=j} a_r
//   superchunk-local, for pass 1 (every superchunk but the last, t = 0 .. G*L-1):
//     w_t = 2^{a'_t - amax} with a'_t = log2(i_t) - sum_{r<=t} log2 sigmoid(f_r)
//     and amax = max_t a'_t; the total log2 decay A = b'_end and the log2
//     scale mu = b'_end + amax of the superchunk's local state (the stabiliser
//     the token recurrence reaches from m = -inf).
// Tokens past T count as f = 1, i = 0.  The waves of a work-group take
// 64-token groups in turn and scan them with DPP; the group totals meet in
// LDS.  With several superchunks this runs inside pass 1: extra work-groups
// write the chunk-local arrays and the scan scalars, and every state tile's
// work-group computes w_t of its own superchunk (a few KB of gate inputs,
// read by each tile) while its first k-steps are in flight.  With one
// superchunk a stand-alone kernel writes the chunk-local arrays.

// Gate inputs of one superchunk for wave w of NWG: 64-token groups w, w + NWG, ...
template <int NWG>
struct GateRegs {
  static constexpr int GPW = 16 / NWG;  // superchunks of at most 1024 tokens
  float gi[GPW], gf[GPW];
};

template <typename T, bool RET, int NWG>
__device__ __forceinline__ void gate_loads(const ChunkParams& p, int L, int bh, int sc, int w, int lane,
                                           GateRegs<NWG>& r) {
  constexpr unsigned ES = sizeof(T);
  const int T_ = p.T, tb = sc * p.G * L;
  const auto ri = make_rsrc(RET ? nullptr : static_cast<const T*>(p.i_pre) + (size_t)bh * T_,
                            RET ? 0u : (unsigned)T_ * ES);
  const auto rf = make_rsrc(RET ? nullptr : static_cast<const T*>(p.f_pre) + (size_t)bh * T_,
                            RET ? 0u : (unsigned)T_ * ES);
#pragma unroll
  for (int k = 0; k < GateRegs<NWG>::GPW; ++k) {
    const unsigned t = (unsigned)(tb + (w + NWG * k) * 64 + lane);
    r.gi[k] = r.gf[k] = 0.f;
    if constexpr (!RET) {
      r.gi[k] = bload1<T>(ri, t * ES);
      r.gf[k] = bload1<T>(rf, t * ES);
    }
  }
}

// From the loaded gates of superchunk sc (all NWG waves of the work-group
// take part; LDS-only barriers inside).  WRITE: store the chunk-local logs
// for pass 3 and, for superchunks but the last, the scan scalars.  WANT_W:
// the superchunk weights w_t into sw (LDS, 1024 floats).  stot: 16 floats,
// smax: NWG floats of LDS.
template <typename T, bool RET, int NWG, bool WRITE, bool WANT_W>
__device__ __forceinline__ void gate_compute(const ChunkParams& p, int L, int bh, int sc, int w, int lane, int tid,
                                             const GateRegs<NWG>& r, float* sw, float* stot, float* smax) {
  constexpr int GPW = GateRegs<NWG>::GPW;
  const int T_ = p.T, hd = bh % p.H;
  const int GL = p.G * L, tb = sc * GL;
  const int NCL = p.NC * L;           // padded token count of a sequence
  const int GLs = min(GL, NCL - tb);  // tokens of this superchunk (last may be short)
  const int NG = (GLs + 63) / 64;
  const bool local = sc < p.NS - 1;   // pass 1 needs this superchunk
  float ret_lg2 = 0.f;
  if constexpr (RET) ret_lg2 = log2f(p.ret_gamma ? p.ret_gamma[hd] : 1.f - exp2f(-5.f - (float)hd));

  float bl[GPW], li[GPW];
  const size_t gbase = (size_t)bh * NCL + tb;
#pragma unroll
  for (int k = 0; k < GPW; ++k) {
    const int g = w + NWG * k;
    const int tl = g * 64 + lane;  // token within the superchunk
    const bool valid = g < NG && tl < GLs && tb + tl < T_;
    float lf2;
    if constexpr (RET) {
      lf2 = valid ? ret_lg2 : 0.f;
      li[k] = valid ? 0.f : -INFINITY;
    } else {
      lf2 = valid ? log2_sigmoid(r.gf[k]) : 0.f;
      li[k] = valid ? r.gi[k] * kLog2e : -INFINITY;
    }
    if constexpr (WRITE) {
      // chunk-local values for pass 3 (a chunk never straddles a 64-token group)
      const float bc = seg_scan_sum(lf2, L);
      const float ac = li[k] - bc;
      const float gc = seg_scan_max(ac, L);
      if (g < NG && tl < GLs) {
        p.ws_ga[gbase + tl] = ac;
        p.ws_gg[gbase + tl] = gc;
        p.ws_gb[gbase + tl] = bc;
      }
    }
    bl[k] = seg_scan_sum(lf2, 64);
    if (g < NG && lane == 63) stot[g] = bl[k];
  }
  if (!local) return;  // work-group-uniform
  lds_barrier();
  float amax = -INFINITY, carry = 0.f;
  int gdone = 0;
#pragma unroll
  for (int k = 0; k < GPW; ++k) {
    const int g = w + NWG * k;
    if (g < NG) {
      for (; gdone < g; ++gdone) carry += stot[gdone];
      const float a = li[k] - (carry + bl[k]);
      amax = fmaxf(amax, a);
      bl[k] = a;
    }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  if (lane == 0) smax[w] = amax;
  lds_barrier();
  amax = smax[0];
#pragma unroll
  for (int i = 1; i < NWG; ++i) amax = fmaxf(amax, smax[i]);
  if constexpr (WANT_W) {
#pragma unroll
    for (int k = 0; k < GPW; ++k) {
      const int g = w + NWG * k;
      const int tl = g * 64 + lane;  // < 1024
      sw[tl] = (g < NG && tl < GL) ? exp2_fast(bl[k] - amax) : 0.f;
    }
  }
  if (WRITE && tid == 0) {
    float b_end = 0.f;
    for (int g = 0; g < NG; ++g) b_end += stot[g];
    p.ws_scal[((size_t)bh * p.NS + sc) * 2 + 0] = b_end;
    p.ws_scal[((size_t)bh * p.NS + sc) * 2 + 1] = b_end + amax;
  }
}

// Stand-alone gate pass for a plan with one superchunk (no pass 1): one
// work-group of 4 waves per (batch*head) writes the chunk-local logs.
template <typename T, bool RET>
__global__ __launch_bounds__(256) void superchunk_gate_kernel(ChunkParams p, int L) {
  __shared__ float stot[16];
  __shared__ float smax[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = p.B * p.H;
  const int bh = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % BH));
  const int sc = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / BH));
  GateRegs<4> r;
  gate_loads<T, RET, 4>(p, L, bh, sc, w, lane, r);
  gate_compute<T, RET, 4, true, false>(p, L, bh, sc, w, lane, tid, r, nullptr, stot, smax);
}

// Pass 1b (local_state_kernel): the local end state of every superchunk but
// the last from the gate factors above:
//   dS = sum_t w_t k_t v_t^T,   dn = sum_t w_t k_t.
// Nothing chains from chunk to chunk, so this is one dense product (w.K)^T V
// per superchunk and state tile.
//
// Work-group = NWP waves (8 for 256-row tiles, else 4) on a TR x TC tile of
// one memory block, WR x WCW waves (NWP x 1 when the tile has 16 NWP or more
// rows: each wave owns TR/NWP rows and all TC columns).  K-steps of KS tokens run through a ring
// of 4 LDS stages filled by direct global-to-LDS buffer loads issued 3 steps
// ahead, so no staging registers hold data in flight.  A stage holds KS token
// rows of K and of V, row-major with padded rows; one load instruction fills
// 1 KB (lane l writes bytes 16l .. 16l+15), so each lane fetches the 16-byte
// unit of the padded tile that lands in its slot, and pad slots read past the
// end of the buffer (zero).  Both MFMA operands come from transposing LDS
// reads; the K^T fragments are multiplied by w_t in registers (w of the whole
// superchunk sits in LDS), and dn comes from the same scaled fragments.
template <typename T, int TR, int TC, int KS, int NWP>
struct LocalCfg {
  static constexpr int NTH = 64 * NWP;  // threads per work-group
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VE = 16 / ES;
  // row strides: residue 8 + 16i dwords (a 128-wide bf16 row pads to
  // 288 bytes, so a 32-row region is exactly 9 KB)
  static constexpr int RK = TR + lds_row_pad(TR, ES);
  static constexpr int RV = TC + lds_row_pad(TC, ES);
  static constexpr int UK = RK * ES / 16;  // 16-byte units per padded K row
  static constexpr int UV = RV * ES / 16;
  static constexpr int NIK = (KS * RK * ES + 1023) / 1024;  // load instructions per K region
  static constexpr int NIV = (KS * RV * ES + 1023) / 1024;
  static constexpr int NI = NIK + NIV;
  static constexpr int JA = (NI + NWP - 1) / NWP;  // instructions per wave (every wave issues JA)
  static constexpr int STAGE = NI * 1024;  // bytes per stage: K region, then V region
  static constexpr int WR = TR >= 16 * NWP ? NWP : TR / 16;  // waves along rows
  static constexpr int WCW = NWP / WR;                         // waves along columns
  static constexpr int MT = TR / WR / 16;             // 16-row tiles per wave
  static constexpr int NTc = TC / WCW / 16;           // 16-column tiles per wave
  static constexpr int GLMAX = 1024;                  // superchunk tokens (w in LDS)
  static_assert(TR % (16 * WR) == 0 && TC % (16 * WCW) == 0 && WR * WCW == NWP, "tile");
  static_assert(GLMAX % NTH == 0, "w staging");
  static_assert((RK * ES) % 16 == 0 && (RV * ES) % 16 == 0, "rows of whole 16-byte units");
};

// fragment times per-k weights, rounded back to bf16 in pairs
__device__ __forceinline__ bf16x8 scale_frag8(bf16x8 x, const float (&w)[8]) { return scale_frag(x, w); }

// NBS: memory blocks of the stored state.  NBS = NB tiles each block; with
// NB = 1 < NBS (blocks narrower than 64 rows) a tile spans the whole head,
// its product covers every block pair, and only the diagonal blocks are
// stored (the off-diagonal MFMA work is cheaper than tiles of 32 rows).
// SN: scalar normaliser, dn = sum_t w_t in dn[0] (the other entries zero).
template <typename T, int DQK, int NB, int TR, int TC, int L, bool RET, int NWP, int NBS = NB, bool SN = false>
__global__ __launch_bounds__(64 * NWP) void local_state_kernel(ChunkParams p) {
  static_assert(NBS == NB || NB == 1, "whole-head tiles store several blocks");
  constexpr int KS = sizeof(T) == 2 ? 32 : 16;
  using C = LocalCfg<T, TR, TC, KS, NWP>;
  constexpr int NTH = C::NTH;
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int K = M::K, KL = M::KL, RK = C::RK, RV = C::RV, VE = C::VE;
  constexpr int MT = C::MT, NTc = C::NTc, NKL = KS / K, JA = C::JA, WR = C::WR, WCW = C::WCW;
  constexpr int DQKB = DQK / NB, NRT = DQKB / TR;
  constexpr unsigned ES = sizeof(T);
  constexpr bool BF = sizeof(T) == 2;
  static_assert(L % KS == 0, "superchunks of whole k-steps");

  // ring of NSTG stages (separate arrays, so that the compiler's own wait
  // tracking tells their loads apart) and w of the superchunk
  constexpr int NSTG = MLSTM_P1_STAGES;
  static_assert(NSTG >= 3 && NSTG <= 6, "ring stages");
  __shared__ __attribute__((aligned(1024))) unsigned char ring0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring3[NSTG > 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char ring4[NSTG > 4 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char ring5[NSTG > 5 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) float sw[C::GLMAX];
  __shared__ float stot[16];
  __shared__ float smax[NWP];
  auto stage_ptr = [&](auto bidx) -> unsigned char* {
    constexpr int b = decltype(bidx)::value;
    if constexpr (b == 0) return ring0;
    else if constexpr (b == 1) return ring1;
    else if constexpr (b == 2) return ring2;
    else if constexpr (b == 3) return ring3;
    else if constexpr (b == 4) return ring4;
    else return ring5;
  };

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w % WR, wcw = w / WR;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int BH = p.B * p.H, DV = p.DV, DVB = DV / NB, T_ = p.T;
  const int nct = DVB / TC;
  const int ntile = NB * NRT * nct;
  const int idx = blockIdx.x;
  const int ncomp = BH * (p.NS - 1) * ntile;
  if (idx >= ncomp) {
    // gate work-groups, one per (batch*head, superchunk): the chunk-local
    // logs of pass 3 and the scan scalars of pass 2
    const int j = idx - ncomp;
    const int gbh = __builtin_amdgcn_readfirstlane(j % BH);
    const int gsc = __builtin_amdgcn_readfirstlane(j / BH);
    GateRegs<NWP> r;
    gate_loads<T, RET, NWP>(p, L, gbh, gsc, w, lane, r);
    gate_compute<T, RET, NWP, true, false>(p, L, gbh, gsc, w, lane, tid, r, nullptr, stot, smax);
    return;
  }
  const int bh = __builtin_amdgcn_readfirstlane(idx % BH);
  const int tile = __builtin_amdgcn_readfirstlane((idx / BH) % ntile);
  const int sc = __builtin_amdgcn_readfirstlane((idx / BH) / ntile);
  const int blk = tile / (NRT * nct), rt = (tile / nct) % NRT, ctl = tile % nct;
  const int f0 = blk * DQKB + rt * TR;  // first feature (of the head) of the tile
  const int c0 = blk * DVB + ctl * TC;  // first d_v column of the tile
  const size_t CS = (size_t)DQK * (DV / NBS);
  const size_t NSTATE = CS + (RET ? 0 : DQK);

  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * T_ * DQK, (unsigned)T_ * DQK * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * T_ * DV, (unsigned)T_ * DV * ES);

  const int GL = p.G * L;
  const int tb = sc * GL;            // first token of the superchunk
  const int NSTEP = p.G * (L / KS);  // k-steps of the superchunk

  // per-lane byte offsets of the loaded units relative to the step's first
  // token (the token part goes into the scalar offset); pad slots point past
  // any buffer end.  The NI load instructions of a stage are dealt to the
  // waves in turn: waves w < NI mod NWP issue JA of them, the others JA - 1
  // (when NWP does not divide NI).  Every wave issues its loads of a step on
  // every path, also past the last step (clamped to it; those stages are
  // never read), so that its vm counter advances the same way on all paths
  // and its waits name exact counts.
  unsigned voff[JA];
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int i = w + NWP * j;
    voff[j] = 0xFFFFFFF0u;
    if (i < C::NIK) {
      const int unit = i * 64 + lane, row = unit / C::UK, cu = unit % C::UK;
      if (row < KS && cu < TR / VE) voff[j] = (unsigned)(row * DQK + f0 + cu * VE) * ES;
    } else if (i < C::NI) {
      const int unit = (i - C::NIK) * 64 + lane, row = unit / C::UV, cu = unit % C::UV;
      if (row < KS && cu < TC / VE) voff[j] = (unsigned)(row * DV + c0 + cu * VE) * ES;
    }
  }
  // whether this wave issues JA loads per step (else JA - 1)
  const bool full_ja = (C::NI % NWP) == 0 || w < C::NI % NWP;
  auto issue = [&](int s_, auto bidx) __attribute__((always_inline)) {
    unsigned char* st = stage_ptr(bidx);
    const int s = min(s_, NSTEP - 1);
    const unsigned t0 = (unsigned)(tb + s * KS);
    const int sk = __builtin_amdgcn_readfirstlane((int)(t0 * DQK * ES));
    const int sv = __builtin_amdgcn_readfirstlane((int)(t0 * DV * ES));
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int i = w + NWP * j;  // wave-uniform
      const bool isk = i < C::NIK;
      if (j < JA - 1 || full_ja) dma16_to_lds(isk ? rk : rv, st + i * 1024, voff[j], isk ? sk : sv);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // s_waitcnt until at most N steps of this wave's loads are in flight
  auto wait_steps = [&](auto nc) __attribute__((always_inline)) {
    constexpr int N = decltype(nc)::value;
    if (full_ja) wait_vmcnt<N * JA>();
    else wait_vmcnt<N * (JA - 1)>();
  };

  // gate inputs, then the first NSTG steps in flight, then w of the
  // superchunk into LDS (the gate loads are issued first, so waiting for
  // them does not wait for the ring)
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  {
    GateRegs<NWP> r;
    gate_loads<T, RET, NWP>(p, L, bh, sc, w, lane, r);
    issue(0, I0{});
    issue(1, I1{});
    issue(2, I2{});
    if constexpr (NSTG > 3) issue(3, I3{});
    if constexpr (NSTG > 4) issue(4, I4{});
    if constexpr (NSTG > 5) issue(5, I5{});
    gate_compute<T, RET, NWP, false, true>(p, L, bh, sc, w, lane, tid, r, sw, stot, smax);
  }

  // dn = sum_t w_t k_t by MFMA: the scaled K^T fragments times an all-ones B
  // operand put the row sums into every column of dacc (rows 4 lg + i).  All
  // waves compute it (no branch in the k-loop); one column tile and wave per
  // row stores it.
  const bool do_dn = !RET && ctl == 0 && wcw == 0;
  f32x4 dacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) dacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const frag ones = M::ones();
  f32x4 acc[MT][NTc];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTc; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transposing-read source columns: output lane lr sees column base + lr
  const int acol = BF ? wr * (TR / WR) + 4 * (lr & 3) : wr * (TR / WR) + lr;
  const int bcol = BF ? wcw * (TC / WCW) + 4 * (lr & 3) : wcw * (TC / WCW) + lr;
  // fragments of one k-step: A = K^T (scaled by w in registers), B = V^T
  struct StepFrags {
    frag af[NKL][MT];
    frag bf[NKL][NTc];
  };
  auto load_step = [&](auto bidx, StepFrags& f) __attribute__((always_inline)) {
    const unsigned char* st = stage_ptr(bidx);
    const T* sk = reinterpret_cast<const T*>(st);
    const T* sv = reinterpret_cast<const T*>(st + C::NIK * 1024);
#pragma unroll
    for (int kb = 0; kb < NKL; ++kb) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) f.af[kb][mt] = frag_rows(sk, RK, kb * K, lg, lr, acol + mt * 16);
#pragma unroll
      for (int nt = 0; nt < NTc; ++nt) f.bf[kb][nt] = frag_rows(sv, RV, kb * K, lg, lr, bcol + nt * 16);
    }
  };
  auto scale_step = [&](int c, StepFrags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKL; ++kb) {
      float wk[KL];
#pragma unroll
      for (int e = 0; e < KL; ++e) wk[e] = sw[c * KS + kb * K + krow<T>(lg, e)];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (BF) f.af[kb][mt] = scale_frag8(f.af[kb][mt], wk);
        else f.af[kb][mt] *= wk[0];
      }
    }
  };
  auto mma_step = [&](const StepFrags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKL; ++kb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTc; ++nt) acc[mt][nt] = M::mma(f.af[kb][mt], f.bf[kb][nt], acc[mt][nt]);
    if constexpr (!RET && !SN) {
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dacc[mt] = M::mma(f.af[kb][mt], ones, dacc[mt]);
    }
  };

  // ---- Software pipeline over k-steps, stage of step c = c % NSTG.  Step
  // 0's fragments are in registers before the loop.  Iteration c: once this
  // wave's loads of step c + 1 have landed, a barrier publishes that stage
  // (and guarantees every wave has read step c's stage into registers, so
  // step c + NSTG can go into it), then step c + 1's fragments are read
  // while the MFMAs of step c run, and scaled by w after them.  Steps past
  // the end (the loop runs in groups of NSTG) only issue and wait.
  StepFrags F0, F1;
  wait_steps(std::integral_constant<int, NSTG - 1>{});  // step 0 landed
  lds_barrier();
  load_step(I0{}, F0);
  scale_step(0, F0);
  // body<true>: steps c and c + 1 both exist (no branch, so the next step's
  // fragment reads can overlap this step's MFMAs); body<false>: the last
  // group of NSTG, where either may be past the end.
  auto body = [&](auto fullc, int c, auto bidx, StepFrags& cur, StepFrags& nxt) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(fullc)::value;
    constexpr int b = decltype(bidx)::value;
    using B1 = std::integral_constant<int, (b + 1) % NSTG>;
    wait_steps(std::integral_constant<int, NSTG - 2>{});
    lds_barrier();
    issue(c + NSTG, bidx);
    if (FULL || c + 1 < NSTEP) load_step(B1{}, nxt);
    if (FULL || c < NSTEP) mma_step(cur);
    if (FULL || c + 1 < NSTEP) scale_step(c + 1, nxt);
  };
  // one group of NSTG steps; the fragment sets alternate, so a group of odd
  // size starts on the set the previous group did not
  auto group = [&](auto fullc, int c, auto odd) __attribute__((always_inline)) {
    constexpr bool O = decltype(odd)::value;
    StepFrags& A = O ? F1 : F0;
    StepFrags& B = O ? F0 : F1;
    body(fullc, c, I0{}, A, B);
    body(fullc, c + 1, I1{}, B, A);
    body(fullc, c + 2, I2{}, A, B);
    if constexpr (NSTG > 3) body(fullc, c + 3, I3{}, B, A);
    if constexpr (NSTG > 4) body(fullc, c + 4, I4{}, A, B);
    if constexpr (NSTG > 5) body(fullc, c + 5, I5{}, B, A);
  };
  using Full = std::true_type;
  using Tail = std::false_type;
  int c = 0;
  if constexpr (NSTG % 2 == 0) {
    for (; c + NSTG < NSTEP; c += NSTG) group(Full{}, c, std::false_type{});
    group(Tail{}, c, std::false_type{});
  } else {
    // odd ring: two groups per loop trip keep the fragment sets in step
    for (; c + 2 * NSTG < NSTEP; c += 2 * NSTG) {
      group(Full{}, c, std::false_type{});
      group(Full{}, c + NSTG, std::true_type{});
    }
    if (c + NSTG < NSTEP) {
      group(Full{}, c, std::false_type{});
      group(Tail{}, c + NSTG, std::true_type{});
    } else {
      group(Tail{}, c, std::false_type{});
    }
  }
  wait_vmcnt<0>();  // no load into the ring in flight past this point

  // ---- outputs: slot sc + 1 of the workspace holds superchunk sc's local state
  float* dst = p.ws_state + ((size_t)bh * p.NS + sc + 1) * NSTATE;
  constexpr bool PERM_OK = sizeof(T) == 2 && DQK == 256 && NB == 1 && NBS == 1;
  if (PERM_OK && p.perm_state) {
    // the register order of pass 3: a lane's 4 rows are one float4
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTc; ++nt) {
        const int r0 = rt * TR + wr * (TR / WR) + mt * 16 + 4 * lg;
        const int cl = ctl * TC + wcw * (TC / WCW) + nt * 16 + lr;
        *reinterpret_cast<f32x4*>(dst + ws_perm4(r0, cl)) = acc[mt][nt];
      }
  } else
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTc; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * TR + wr * (TR / WR) + mt * 16 + 4 * lg + i;  // row within the block
        const int cl = ctl * TC + wcw * (TC / WCW) + nt * 16 + lr;     // column within the block
        if constexpr (NBS == NB) {
          dst[(size_t)blk * DQKB * DVB + (size_t)r * DVB + cl] = acc[mt][nt][i];
        } else {
          // whole-head tile: row r and column cl of the head; keep the
          // diagonal blocks
          constexpr int RB = DQK / NBS;
          const int DVS = DV / NBS;
          const int bs = r / RB;
          if (bs == cl / DVS)
            dst[(size_t)bs * RB * DVS + (size_t)(r - bs * RB) * DVS + (cl - bs * DVS)] = acc[mt][nt][i];
        }
      }
  if constexpr (!RET && !SN) {
    if (do_dn && lr == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[CS + f0 + wr * (TR / WR) + mt * 16 + 4 * lg + i] = dacc[mt][i];
    }
  }
  if constexpr (SN) {
    // the scalar sum_t w_t (w of the whole superchunk sits in LDS, zero past
    // its end) into dn[0], zeros in this tile's other dn rows
    float ws = 0.f;
    if (do_dn && f0 == 0 && wr == 0) {
      for (int t = lane; t < C::GLMAX; t += 64) ws += sw[t];
#pragma unroll
      for (int d = 32; d > 0; d >>= 1) ws += __shfl_xor(ws, d, 64);
    }
    if (do_dn && lr == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = f0 + wr * (TR / WR) + mt * 16 + 4 * lg + i;
          dst[CS + r] = r == 0 ? ws : 0.f;
        }
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
      if (p.perm && e < p.CS) {
        // gather rows r0 + i of column c (inverse of ws_perm4)
        const int DV = (int)(p.CS / p.DQK);
        const int lane = (int)((e0 >> 2) & 63), q = (int)((e0 >> 8) & 31), nt = q >> 1;
        const int c = (int)(e0 >> 13) * 32 + (q & 1) * 16 + (lane & 15);
        const int r = 32 * (nt >> 1) + 8 * (lane >> 4) + 4 * (nt & 1) + i;
        x[i] = p.C0 ? p.C0[(size_t)bh * p.CS + (size_t)r * DV + c] : 0.f;
      } else if (e < p.CS) x[i] = p.C0 ? p.C0[(size_t)bh * p.CS + e] : 0.f;
      else if (p.scalar_n) x[i] = (p.n0 && e == p.CS) ? p.n0[bh] : 0.f;  // n0 [B,H]
      else x[i] = p.n0 ? p.n0[(size_t)bh * p.DQK + (e - p.CS)] : 0.f;
    }
    S = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(base + e0) = S;
  }
  // Superchunks go in windows of SW: all local states and scalars of a
  // window are loaded before any of its start states is stored (each into
  // the slot its local state was read from), so the loads' latencies
  // overlap instead of queueing behind the stores.
  constexpr int SW = 8;
  float m = m0;
  for (int s0 = 1; s0 < p.NS; s0 += SW) {
    float A[SW], mu[SW];
    float4 d[SW];
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      const int sc = s0 + j;
      A[j] = mu[j] = 0.f;
      d[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (sc < p.NS) {
        A[j] = p.ws_scal[((size_t)bh * p.NS + sc - 1) * 2 + 0];
        mu[j] = p.ws_scal[((size_t)bh * p.NS + sc - 1) * 2 + 1];
        if (active) d[j] = *reinterpret_cast<const float4*>(base + (size_t)sc * NSTATE + e0);
      }
    }
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      const int sc = s0 + j;
      if (sc < p.NS) {
        const float mn = fmaxf(A[j] + m, mu[j]);
        const float fa = exp2_fast(A[j] + m - mn), fb = exp2_fast(mu[j] - mn);
        S.x = fa * S.x + fb * d[j].x;
        S.y = fa * S.y + fb * d[j].y;
        S.z = fa * S.z + fb * d[j].z;
        S.w = fa * S.w + fb * d[j].w;
        if (active) *reinterpret_cast<float4*>(base + (size_t)sc * NSTATE + e0) = S;
        m = mn;
        if (writer) p.ws_min[(size_t)bh * p.NS + sc] = mn;
      }
    }
  }
}

template <typename T, int DQK, int NB, int WC, int NRG, int NCG, int L, bool RET, bool GN>
size_t chunk_lds_bytes() {
  return ChunkCfg<T, DQK, NB, WC, NRG, NCG, L, GN>::lds_bytes(RET);
}

template <typename T, int DQK, int NB, int WC, int NRG, int NCG, int L, bool RET, bool GN, bool SN = false,
          bool PB = false>
hipError_t launch_chunkwise(ChunkParams p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int NTH = 64 * NCG * NRG;
  const int BH = p.B * p.H;
  const size_t CS = (size_t)DQK * p.DV / NB;
  // the xLSTM-7B head shape (d_qk 256, one memory block, 128-column slices):
  // the wave-specialised form of pass 3
  constexpr bool WSK = std::is_same<T, __bf16>::value && DQK == 256 && NB == 1 && WC * NCG == 128 && L == 64 &&
                       !RET && !GN && !PB;
  // the planned 7B-shape pass 3 reads the superchunk slots in its register
  // order (not a state-passes-only call: the backward reads them in order)
  p.perm_state = (WSK && p.h && !p.direct) ? 1 : 0;
  if (p.direct) {
    // one superchunk, run as pass 3 alone (it reads C0 / n0 / m0 and forms
    // the gate logs itself)
  } else if (p.NS == 1)
    hipLaunchKernelGGL((superchunk_gate_kernel<T, RET>), dim3((unsigned)BH), dim3(256), 0, stream, p, L);
  else {
    // pass 1 tiles: TR rows x TC columns of one memory block.  bf16 tiles
    // take up to 256 rows (8 waves, one work-group per CU): every k-step's
    // V rows then serve twice the MFMA work of a 128-row tile, which halves
    // the redundant L2-to-LDS traffic that bounds this pass.  The gate
    // work-groups (one per batch*head and superchunk) follow the tiles.
    // Blocks narrower than 64 rows: whole-head tiles (NBC = 1), diagonal
    // blocks stored.
    constexpr int NBC = (NB > 1 && DQK / NB < 64) ? 1 : NB;  // blocks of the tiling
    constexpr int DQKB = DQK / NBC;
    constexpr int RCAP = sizeof(T) == 2 ? MLSTM_P1_ROWS : 64;
    constexpr int TR = DQKB < RCAP ? DQKB : RCAP;
    constexpr int NWP = TR >= 256 ? 8 : 4;
    constexpr int TCAP = sizeof(T) == 2 ? 128 : 64;
    const int DVB = p.DV / NBC;
    const int TC = DVB % TCAP == 0 ? TCAP : DVB % 64 == 0 ? 64 : 32;
    const dim3 g1((unsigned)(BH * (p.NS - 1) * NBC * (DQKB / TR) * (DVB / TC) + BH * p.NS));
    const dim3 b1(64 * NWP);
    if (TC == TCAP)
      hipLaunchKernelGGL((local_state_kernel<T, DQK, NBC, TR, TCAP, L, RET, NWP, NB, SN>), g1, b1, 0, stream, p);
    else if (TC == 64)
      hipLaunchKernelGGL((local_state_kernel<T, DQK, NBC, TR, 64, L, RET, NWP, NB, SN>), g1, b1, 0, stream, p);
    else
      hipLaunchKernelGGL((local_state_kernel<T, DQK, NBC, TR, 32, L, RET, NWP, NB, SN>), g1, b1, 0, stream, p);
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
  s.scalar_n = SN ? 1 : 0;
  s.perm = p.perm_state;
  const size_t nstate = CS + (RET ? 0 : DQK);
  dim3 g2((unsigned)((nstate / 4 + 255) / 256), (unsigned)BH);
  // fuse_scan: pass 3 composes the start states (a forward call only; the
  // backward's recompute, h = NULL, needs pass 2's slots)
  // (heads of 64 features only: a wider one's state exceeds the fused limit)
  constexpr bool FSK = !WSK && DQK == 64;
  const bool fs = FSK && p.fuse_scan && p.h;
  if (!p.direct && !fs) hipLaunchKernelGGL((superchunk_scan_kernel<RET>), g2, dim3(256), 0, stream, s);
  if (!p.h) return hipGetLastError();  // state passes only (the backward's recompute)
  dim3 g3((unsigned)(BH * p.nslices * p.NS));
  if (ev0) (void)hipEventRecord(ev0, stream);
  constexpr bool WS = WSK;
  // DIR: a direct call (one superchunk, no gate pass or pass 2), a separate
  // instantiation so that the planned kernels carry no branch on it
  auto pass3 = [&](auto dir, auto fsc) {
    constexpr bool DIR = decltype(dir)::value;
    constexpr bool FS = decltype(fsc)::value && FSK;  // generic kernel, 64-wide heads
    if constexpr (WS) {
      if (p.o_pre)
        hipLaunchKernelGGL((chunk_kernel_ws<true, SN, DIR>), g3, dim3(512), 0, stream, p);
      else
        hipLaunchKernelGGL((chunk_kernel_ws<false, SN, DIR>), g3, dim3(512), 0, stream, p);
    } else if constexpr (GN) {
      hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, NRG, NCG, L, RET, false, true, false, false, DIR, FS>), g3,
                         dim3(NTH), 0, stream, p);
      if (p.gn_ws) {
        const long long rows = (long long)BH * p.T;
        hipLaunchKernelGGL((groupnorm_rows_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                           p.gn_ws, static_cast<T*>(p.h), rows, p.T, p.H, p.DV, p.gn_w, p.gn_b, p.gn_eps);
      }
    } else if (!RET && p.o_pre)
      hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, NRG, NCG, L, RET, !RET, false, SN, PB, DIR, FS>), g3,
                         dim3(NTH), 0, stream, p);
    else
      hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, NRG, NCG, L, RET, false, false, SN, PB, DIR, FS>), g3,
                         dim3(NTH), 0, stream, p);
  };
  if (p.direct)
    pass3(std::true_type{}, std::false_type{});
  else if (fs)
    pass3(std::false_type{}, std::integral_constant<bool, FSK>{});
  else
    pass3(std::false_type{}, std::false_type{});
  const hipError_t e = hipGetLastError();
  if (ev1) (void)hipEventRecord(ev1, stream);
  return e;
}

// ------------------------------------------------------------ dispatch table
// (dtype, d_qk, num_blocks, columns per wave, row groups, column groups,
//  chunk, retention); one variant per (dtype, d_qk, num_blocks, chunk,
//  retention)
#define MLSTM_CHUNK_VARIANTS(X)             \
  X(__bf16, 64, 1, 16, 1, 4, 64, false)     \
  X(__bf16, 64, 2, 16, 1, 4, 64, false)     \
  X(__bf16, 64, 1, 16, 1, 4, 32, false)     \
  X(__bf16, 128, 1, 32, 2, 4, 64, false)    \
  X(__bf16, 256, 1, 32, 2, 4, 64, false)    \
  X(__bf16, 256, 2, 16, 2, 4, 64, false)    \
  X(float, 64, 1, 16, 1, 4, 64, false)      \
  X(float, 64, 1, 16, 1, 4, 32, false)      \
  X(float, 64, 1, 16, 1, 4, 16, false)      \
  X(float, 64, 2, 16, 1, 4, 64, false)      \
  X(__bf16, 64, 1, 16, 1, 4, 64, true)      \
  X(__bf16, 64, 1, 16, 1, 4, 32, true)      \
  X(__bf16, 128, 1, 32, 2, 4, 64, true)     \
  X(float, 64, 1, 16, 1, 4, 64, true)

// the scalar-normaliser launcher of an mLSTM variant (none for retention)
template <typename T, int DQK, int NB, int WC, int NRG, int NCG, int L, bool RET>
constexpr ChunkLaunchFn scalar_norm_launcher() {
  if constexpr (RET) return nullptr;
  else return &launch_chunkwise<T, DQK, NB, WC, NRG, NCG, L, RET, false, true>;
}
// the per-block-normaliser launcher of a block-diagonal mLSTM variant
template <typename T, int DQK, int NB, int WC, int NRG, int NCG, int L, bool RET>
constexpr ChunkLaunchFn block_norm_launcher() {
  if constexpr (RET || NB == 1) return nullptr;
  else return &launch_chunkwise<T, DQK, NB, WC, NRG, NCG, L, RET, false, false, true>;
}

bool find_chunk_variant(int dtype, int dqk, int nb, int L, bool ret, ChunkVariant* out) {
#define X(T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_)                                              \
  if (dtype == (sizeof(T_) == 2 ? 1 : 0) && dqk == DQK_ && nb == NB_ && L == L_ && ret == RET_) { \
    out->launch = &launch_chunkwise<T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_, false>;            \
    out->launch_scalar_norm = scalar_norm_launcher<T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_>();  \
    out->launch_block_norm = block_norm_launcher<T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_>();    \
    out->lds_bytes = chunk_lds_bytes<T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_, false>();         \
    out->wc = WC_;                                                                               \
    out->w = NCG_ * WC_;                                                                         \
    return true;                                                                                 \
  }
  MLSTM_CHUNK_VARIANTS(X)
#undef X
  return false;
}

// Retention with the per-head group norm fused into the output store (the
// "Multi-Scale Retention (MSR)" section of the "Edifice.Attention.RetNet"
// page normalises each head's output with a group norm): the retention
// variants above, with d_v equal to their slice width.
bool find_retention_groupnorm_variant(int dtype, int dqk, int L, ChunkVariant* out) {
#define X(T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_)                                              \
  if (RET_ && dtype == (sizeof(T_) == 2 ? 1 : 0) && dqk == DQK_ && NB_ == 1 && L == L_) {        \
    out->launch = &launch_chunkwise<T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_, RET_>;             \
    out->launch_scalar_norm = nullptr;                                                           \
    out->launch_block_norm = nullptr;                                                            \
    out->lds_bytes = chunk_lds_bytes<T_, DQK_, NB_, WC_, NRG_, NCG_, L_, RET_, RET_>();          \
    out->wc = WC_;                                                                               \
    out->w = NCG_ * WC_;                                                                         \
    return true;                                                                                 \
  }
  MLSTM_CHUNK_VARIANTS(X)
#undef X
  return false;
}

}  // namespace mlstm
