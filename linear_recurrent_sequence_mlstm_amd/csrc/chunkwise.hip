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

template <typename T, int DQK, int NB, int WC, int L>
struct ChunkCfg {
  static constexpr int K = Mma<T>::K;
  static constexpr int KL = Mma<T>::KL;
  static constexpr int DQKB = DQK / NB;
  static constexpr int NT = DQKB / 16;
  static constexpr int CT = WC / 16;
  static constexpr int W = 4 * WC;
  static constexpr int NJT = L / 16;
  static constexpr int NKL = L / K;
  static constexpr int NKQ = DQK / K;
  static constexpr int NKQB = DQKB / K;
  static constexpr int VE = 16 / (int)sizeof(T);  // elements per 16 bytes
  static constexpr int PAD = VE;
  static constexpr int QS = DQK + PAD;            // row stride of sQ
  static constexpr int TS = L + PAD;              // row stride of sKt, sVt, sP
  // staging units (16-byte loads) per chunk
  static constexpr int NQU = L * DQK / VE;
  static constexpr int NKU = (L / 4) * (DQK / VE);
  static constexpr int NVU = (L / 4) * (W / VE);
  static constexpr int QIT = (NQU + 255) / 256;
  static constexpr int KIT = (NKU + 255) / 256;
  static constexpr int VIT = (NVU + 255) / 256;
  static_assert(DQK % NB == 0, "d_qk % nb");
  static_assert(DQKB % (2 * 16) == 0 || sizeof(T) == 4, "bf16 path needs 32-row blocks");
  static_assert(DQKB % 16 == 0, "block rows multiple of 16");
  static_assert(L % K == 0 && L % 16 == 0 && L <= 64, "chunk length");
  static_assert(WC % 16 == 0, "wave columns");
  static constexpr size_t lds_bytes(bool full, bool ret) {
    size_t b = 0;
    b += (size_t)DQK * TS * sizeof(T);           // sKt
    b += (size_t)W * TS * sizeof(T);             // sVt
    b += 6 * L * 4 + 16;                         // gate vectors
    if (!ret) b += DQK * 4 + 2 * DQK * sizeof(T);  // n~
    if (full) {
      b += (size_t)L * QS * sizeof(T);           // sQ
      b += (size_t)NB * L * TS * sizeof(T);      // sP
      b += 5 * L * 4;                            // den partials
    }
    return b;
  }
};

template <typename T, int DQK, int NB, int WC, int L, bool RET, bool FULL>
__global__ __launch_bounds__(256) void chunk_kernel(ChunkParams p) {
  using C = ChunkCfg<T, DQK, NB, WC, L>;
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int K = C::K, KL = C::KL, DQKB = C::DQKB, NT = C::NT, CT = C::CT;
  constexpr int W = C::W, NJT = C::NJT, NKL = C::NKL, NKQ = C::NKQ, NKQB = C::NKQB;
  constexpr int VE = C::VE, QS = C::QS, TS = C::TS;

  __shared__ __attribute__((aligned(16))) T sKt[DQK * TS];
  __shared__ __attribute__((aligned(16))) T sVt[W * TS];
  __shared__ __attribute__((aligned(16))) T sQ[FULL ? L * QS : 8];
  __shared__ __attribute__((aligned(16))) T sP[FULL ? NB * L * TS : 8];
  __shared__ __attribute__((aligned(16))) T sNh[RET ? 8 : 2 * DQK];
  __shared__ float sNf[RET ? 4 : DQK];
  __shared__ float sA2[L], sM2[L], sRS[L], sCL[L], sBT[L], sW[L];
  __shared__ float sDenPart[FULL ? 4 * L : 4];
  __shared__ float sDenInter[FULL ? L : 4];
  __shared__ float sAlpha;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int BH = p.B * p.H;
  int idx = blockIdx.x;
  const int bh = idx % BH;
  idx /= BH;
  const int slice = idx % p.nslices;
  const int sc = idx / p.nslices;
  const int hd = bh % p.H;
  const int T_ = p.T, DV = p.DV, DVB = DV / NB;
  const size_t CS = (size_t)DQK * DV / NB;
  const size_t NSTATE = CS + (RET ? 0 : DQK);

  const int wcol0 = slice * W + w * WC;  // first global d_v column of this wave
  const int blk = wcol0 / DVB;           // memory block of this wave
  const int wcl0 = wcol0 - blk * DVB;    // first column inside the block
  const int rb0 = blk * DQKB;            // first feature row of the block

  const T* __restrict__ gq = static_cast<const T*>(p.q) + (size_t)bh * T_ * DQK;
  const T* __restrict__ gk = static_cast<const T*>(p.k) + (size_t)bh * T_ * DQK;
  const T* __restrict__ gv = static_cast<const T*>(p.v) + (size_t)bh * T_ * DV;
  const T* __restrict__ gi = RET ? nullptr : static_cast<const T*>(p.i_pre) + (size_t)bh * T_;
  const T* __restrict__ gf = RET ? nullptr : static_cast<const T*>(p.f_pre) + (size_t)bh * T_;
  const T* __restrict__ go = (FULL && p.o_pre) ? static_cast<const T*>(p.o_pre) + (size_t)bh * T_ * DV : nullptr;
  T* __restrict__ gh = FULL ? static_cast<T*>(p.h) + (size_t)bh * T_ * DV : nullptr;
  const float bias = (!RET && p.bias) ? p.bias[hd] : 0.f;
  float ret_lg2 = 0.f;
  if constexpr (RET) ret_lg2 = log2f(p.ret_gamma ? p.ret_gamma[hd] : 1.f - exp2f(-5.f - (float)hd));

  const int c_begin = sc * p.G;
  const int c_end = FULL ? min(c_begin + p.G, p.NC) : c_begin + p.G;

  // ---------------------------------------------------------------- state in
  f32x4 st[NT][CT];
  const float* Sin = nullptr;
  if (FULL && (sc > 0 || p.has_init)) Sin = p.ws_state + ((size_t)bh * p.NS + sc) * NSTATE;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = perm_row<T>(nt, 4 * lg + i);
        const int col = wcl0 + ct * 16 + lr;
        st[nt][ct][i] = Sin ? Sin[(size_t)blk * DQKB * DVB + (size_t)row * DVB + col] : 0.f;
      }
  if constexpr (!RET) {
    for (int r = tid; r < DQK; r += 256) {
      const float x = Sin ? Sin[CS + r] : 0.f;
      sNf[r] = x;
      const T hi = from_f32<T>(x);
      sNh[r] = hi;
      sNh[DQK + r] = from_f32<T>(x - to_f32(hi));
    }
  }
  if constexpr (FULL) {
    // masked (l > j) tiles of P and their den partials are never written
    for (int e = tid; e < NB * L * TS; e += 256) sP[e] = from_f32<T>(0.f);
    for (int e = tid; e < 4 * L; e += 256) sDenPart[e] = 0.f;
  }
  // stabiliser carried by wave 0 (log2 units)
  float m_prev = FULL ? p.ws_min[(size_t)bh * p.NS + sc] : -INFINITY;
  float a_total = 0.f;

  // ------------------------------------------------------ staging registers
  Vec16<T> rq[FULL ? C::QIT : 1];
  Vec16<T> rk[C::KIT][4];
  Vec16<T> rv[C::VIT][4];
  float rgi = 0.f, rgf = 0.f;

  auto load_stage = [&](int c) {
    const int t0 = c * L;
    if constexpr (FULL) {
#pragma unroll
      for (int it = 0; it < C::QIT; ++it) {
        const int u = tid + it * 256;
        if (u < C::NQU) {
          const int j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
          rq[it] = (t0 + j < T_) ? load16(gq + (size_t)(t0 + j) * DQK + col) : zero16<T>();
        }
      }
    }
#pragma unroll
    for (int it = 0; it < C::KIT; ++it) {
      const int u = tid + it * 256;
      if (u < C::NKU) {
        const int tg = u % (L / 4), fg = u / (L / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 4 * tg + r;
          rk[it][r] = (t < T_) ? load16(gk + (size_t)t * DQK + fg * VE) : zero16<T>();
        }
      }
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int u = tid + it * 256;
      if (u < C::NVU) {
        const int tg = u % (L / 4), fg = u / (L / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 4 * tg + r;
          rv[it][r] = (t < T_) ? load16(gv + (size_t)t * DV + slice * W + fg * VE) : zero16<T>();
        }
      }
    }
    if constexpr (!RET) {
      if (w == 0 && lane < L && t0 + lane < T_) {
        rgi = to_f32(gi[t0 + lane]);
        rgf = to_f32(gf[t0 + lane]);
      }
    }
  };

  auto store_stage = [&]() {
    if constexpr (FULL) {
#pragma unroll
      for (int it = 0; it < C::QIT; ++it) {
        const int u = tid + it * 256;
        if (u < C::NQU) {
          const int j = u / (DQK / VE), col = (u % (DQK / VE)) * VE;
          *reinterpret_cast<uint4*>(&sQ[j * QS + col]) = *reinterpret_cast<const uint4*>(rq[it].v);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < C::KIT; ++it) {
      const int u = tid + it * 256;
      if (u < C::NKU) {
        const int tg = u % (L / 4), fg = u / (L / 4);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          store4(&sKt[(fg * VE + e) * TS + 4 * tg], rk[it][0].v[e], rk[it][1].v[e], rk[it][2].v[e],
                 rk[it][3].v[e]);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int u = tid + it * 256;
      if (u < C::NVU) {
        const int tg = u % (L / 4), fg = u / (L / 4);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          store4(&sVt[(fg * VE + e) * TS + 4 * tg], rv[it][0].v[e], rv[it][1].v[e], rv[it][2].v[e],
                 rv[it][3].v[e]);
        }
      }
    }
  };

  // Gate scan for one chunk on wave 0 (one lane per token).
  auto gates = [&](int c) {
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
    if (lane == 0) sAlpha = exp2_fast(m_prev - ML);
    m_prev = bL + ML;
    a_total += bL;
  };

  load_stage(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * L;
    store_stage();
    if (w == 0) gates(c);
    __syncthreads();  // B1: chunk staged, gate factors ready
    if (c + 1 < c_end) load_stage(c + 1);

    // update of the state is needed unless this is the last chunk of a
    // superchunk whose end state nobody reads
    const bool need_update = !FULL || (c + 1 < c_end) || (sc == p.NS - 1);

    frag vf[CT][NKL];  // V^T fragments of this wave's columns
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb)
        vf[ct][kb] = M::load(&sVt[(w * WC + ct * 16 + lr) * TS + kb * K + KL * lg]);

    if constexpr (FULL) {
      // ---------------------------------------------------------- phase B
      f32x4 acc[NJT][CT];
      f32x4 pt[NB][NJT];
      f32x4 pn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[jt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int be = 0; be < NB; ++be) pt[be][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const bool do_qk = w < NJT;
      frag kf[NKQ];
      if (do_qk) {
        const int t = t0 + w * 16 + lr;
#pragma unroll
        for (int kb = 0; kb < NKQ; ++kb)
          kf[kb] = (t < T_) ? M::load(gk + (size_t)t * DQK + kb * K + KL * lg) : M::zero();
      }
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        frag qf[NKQ];
#pragma unroll
        for (int kb = 0; kb < NKQ; ++kb) qf[kb] = M::load(&sQ[(jt * 16 + lr) * QS + kb * K + KL * lg]);
        // readout of the state at the chunk start: D[c][j] += S~[:, c] . q_j
#pragma unroll
        for (int be = 0; be < NB; ++be) {
          if (be == blk) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
              for (int kk = 0; kk < NKQB; ++kk)
                acc[jt][ct] = M::mma(StateFrag<T, NT, CT>::get(st, kk, ct), qf[be * NKQB + kk], acc[jt][ct]);
          }
        }
        // scores of key tile w against query tile jt, per memory block
        if (do_qk && jt >= w) {
#pragma unroll
          for (int be = 0; be < NB; ++be)
#pragma unroll
            for (int kk = 0; kk < NKQB; ++kk)
              pt[be][jt] = M::mma(kf[be * NKQB + kk], qf[be * NKQB + kk], pt[be][jt]);
        }
        // n~ . q_j for query tile jt == w, n~ split in hi + lo parts
        if constexpr (!RET) {
          if (jt == w) {
#pragma unroll
            for (int kb = 0; kb < NKQ; ++kb) {
              frag nf = M::load(&sNh[(lr & 1) * DQK + kb * K + KL * lg]);
              if (lr > 1) nf = M::zero();
              pn = M::mma(nf, qf[kb], pn);
            }
          }
        }
      }
      // decay mask and factors, P to LDS, den partial sums
      if (do_qk) {
        float a2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a2[i] = sA2[w * 16 + 4 * lg + i];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          if (jt >= w) {
            const int j = jt * 16 + lr;
            const float m2 = sM2[j];
            float fac[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int l = w * 16 + 4 * lg + i;
              fac[i] = (l <= j) ? exp2_fast(a2[i] - m2) : 0.f;
            }
            float dsum = 0.f;
#pragma unroll
            for (int be = 0; be < NB; ++be) {
              T pv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float x = pt[be][jt][i] * fac[i];
                dsum += x;
                pv[i] = from_f32<T>(x);
              }
              store4(&sP[(be * L + j) * TS + w * 16 + 4 * lg], pv[0], pv[1], pv[2], pv[3]);
            }
            dsum += __shfl_xor(dsum, 16, 64);
            dsum += __shfl_xor(dsum, 32, 64);
            if (lg == 0) sDenPart[w * L + j] = dsum;
          }
        }
        if constexpr (!RET) {
          if (lg == 0) sDenInter[w * 16 + lr] = pn[0] + pn[1];
        }
      }
      __syncthreads();  // B2: P and den partials ready

      // ---------------------------------------------------------- phase C
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const int j = jt * 16 + lr;
        const float rs = sRS[j];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[jt][ct] *= rs;
#pragma unroll
        for (int kb = 0; kb < NKL; ++kb) {
          if (kb * K <= jt * 16 + 15) {
            const frag pf = M::load(&sP[(blk * L + jt * 16 + lr) * TS + kb * K + KL * lg]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[jt][ct] = M::mma(vf[ct][kb], pf, acc[jt][ct]);
          }
        }
        if (t0 + j < T_) {
          float inv;
          if constexpr (RET) {
            inv = 1.f;
          } else {
            const float den = rs * sDenInter[j] + sDenPart[j] + sDenPart[L + j] + sDenPart[2 * L + j] +
                              sDenPart[3 * L + j] + sBT[j];
            inv = 1.f / fmaxf(fabsf(den), sCL[j]);
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int col = wcol0 + ct * 16 + 4 * lg;
            const size_t off = (size_t)(t0 + j) * DV + col;
            float o[4] = {1.f, 1.f, 1.f, 1.f};
            if (go) {
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = sigmoidf_(to_f32(go[off + i]));
            }
            T hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = from_f32<T>(o[i] * acc[jt][ct][i] * inv);
            if constexpr (sizeof(T) == 2) {
              *reinterpret_cast<uint2*>(gh + off) = *reinterpret_cast<const uint2*>(hv);
            } else {
              *reinterpret_cast<uint4*>(gh + off) = *reinterpret_cast<const uint4*>(hv);
            }
          }
        }
      }
    }

    // ------------------------------------------------------- state update
    if (need_update) {
      const float alpha = sAlpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) st[nt][ct] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKL; ++kb) {
        float wl[KL];
#pragma unroll
        for (int e = 0; e < KL; ++e) wl[e] = sW[kb * K + KL * lg + e];
        frag wv[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) wv[ct] = scale_frag(vf[ct][kb], wl);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const frag ka = M::load(&sKt[(rb0 + perm_row<T>(nt, lr)) * TS + kb * K + KL * lg]);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st[nt][ct] = M::mma(ka, wv[ct], st[nt][ct]);
        }
      }
      if constexpr (!RET) {
        for (int r = tid; r < DQK; r += 256) {
          float x = alpha * sNf[r];
#pragma unroll
          for (int l = 0; l < L; l += VE) {
            const Vec16<T> kv = load16(&sKt[r * TS + l]);
#pragma unroll
            for (int e = 0; e < VE; ++e) x += sW[l + e] * to_f32(kv.v[e]);
          }
          sNf[r] = x;
          const T hi = from_f32<T>(x);
          sNh[r] = hi;
          sNh[DQK + r] = from_f32<T>(x - to_f32(hi));
        }
      }
    }
    __syncthreads();  // B3: LDS free for the next chunk
  }

  // ---------------------------------------------------------------- outputs
  float* Sdst = nullptr;
  if (!FULL) Sdst = p.ws_state + ((size_t)bh * p.NS + sc + 1) * NSTATE;
  else if (sc == p.NS - 1) Sdst = p.C_out;  // [B,H,NB,DQKB,DVB]
  if (FULL && Sdst) Sdst += (size_t)bh * CS;
  if (Sdst) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = perm_row<T>(nt, 4 * lg + i);
          const int col = wcl0 + ct * 16 + lr;
          Sdst[(size_t)blk * DQKB * DVB + (size_t)row * DVB + col] = st[nt][ct][i];
        }
  }
  if (slice == 0) {
    if (!FULL) {
      float* nd = p.ws_state + ((size_t)bh * p.NS + sc + 1) * NSTATE + CS;
      if constexpr (!RET)
        for (int r = tid; r < DQK; r += 256) nd[r] = sNf[r];
      if (tid == 0) {
        p.ws_scal[((size_t)bh * p.NS + sc) * 2 + 0] = a_total;
        p.ws_scal[((size_t)bh * p.NS + sc) * 2 + 1] = m_prev;
      }
    } else if (sc == p.NS - 1) {
      if constexpr (!RET) {
        if (p.n_out)
          for (int r = tid; r < DQK; r += 256) p.n_out[(size_t)bh * DQK + r] = sNf[r];
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

template <typename T, int DQK, int NB, int WC, int L, bool RET>
size_t chunk_lds_bytes() {
  return ChunkCfg<T, DQK, NB, WC, L>::lds_bytes(true, RET);
}

template <typename T, int DQK, int NB, int WC, int L, bool RET>
hipError_t launch_chunkwise(ChunkParams p, hipStream_t stream) {
  const int BH = p.B * p.H;
  const size_t CS = (size_t)DQK * p.DV / NB;
  if (p.NS > 1) {
    dim3 g1((unsigned)(BH * p.nslices * (p.NS - 1)));
    hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, L, RET, false>), g1, dim3(256), 0, stream, p);
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
  hipLaunchKernelGGL((chunk_kernel<T, DQK, NB, WC, L, RET, true>), g3, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ------------------------------------------------------------ dispatch table
#define MLSTM_CHUNK_VARIANTS(X)            \
  X(__bf16, 64, 1, 16, 64, false)          \
  X(__bf16, 64, 2, 16, 64, false)          \
  X(__bf16, 64, 1, 16, 32, false)          \
  X(__bf16, 128, 1, 32, 64, false)         \
  X(__bf16, 256, 1, 32, 64, false)         \
  X(__bf16, 256, 1, 16, 64, false)         \
  X(__bf16, 256, 2, 16, 64, false)         \
  X(float, 64, 1, 16, 64, false)           \
  X(float, 64, 1, 16, 32, false)           \
  X(float, 64, 1, 16, 16, false)           \
  X(float, 64, 2, 16, 64, false)           \
  X(__bf16, 64, 1, 16, 64, true)           \
  X(__bf16, 64, 1, 16, 32, true)           \
  X(__bf16, 128, 1, 32, 64, true)          \
  X(float, 64, 1, 16, 64, true)

bool find_chunk_variant(int dtype, int dqk, int nb, int wc, int L, bool ret, ChunkVariant* out) {
#define X(T_, DQK_, NB_, WC_, L_, RET_)                                                          \
  if (dtype == (sizeof(T_) == 2 ? 1 : 0) && dqk == DQK_ && nb == NB_ && wc == WC_ && L == L_ && \
      ret == RET_) {                                                                             \
    out->launch = &launch_chunkwise<T_, DQK_, NB_, WC_, L_, RET_>;                               \
    out->lds_bytes = chunk_lds_bytes<T_, DQK_, NB_, WC_, L_, RET_>();                            \
    out->wc = WC_;                                                                               \
    return true;                                                                                 \
  }
  MLSTM_CHUNK_VARIANTS(X)
#undef X
  return false;
}

}  // namespace mlstm
