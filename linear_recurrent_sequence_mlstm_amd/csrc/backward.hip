// Chunkwise backward pass of the mLSTM recurrence (vector normaliser, one
// memory block, chunks of 64 tokens): gradients of sum(dh * h) with respect to
// q, k, v, the gate preactivations, the output gate, the normaliser bias and
// the initial state.  Retention runs through the same kernels (p.ret): gates
// i = 1, f = gamma_h make the stabiliser exactly 0 and the weights below
// powers of gamma; with no normaliser dz~ = 0 and den~ = 1.
//
// The forward's state passes (gates, pass 1, pass 2) leave in the workspace
// the superchunk start states and the chunk-local gate logs a_j, g_j, b_j (log2
// units); bwd_chunk_states_kernel expands them into the stabilised start state
// (S~, n~) and stabiliser m of every chunk.  From these, per chunk with M_j = max(m_prev, g_j) and M_L its
// chunk-end value (the forward's own weights):
//   E_jl = 2^{a_l - M_j} (l <= j),  alpha_j = 2^{m_prev - M_j},
//   w_j = 2^{a_j - M_L},  e^{-m_j} = 2^{-(b_j + M_j)},
//   dn~_j = o_j dh_j / den~_j,  dz~_j = -(dh_j . h_j) sign(z~_j) / den~_j when
//     |z~_j| > e^{-m_j} (else 0),  D'_jl = E_jl (dn~_j . v_l + dz~_j),
//   dq_j = sum_l D'_jl k_l + alpha_j (S~_prev dn~_j + n~_prev dz~_j),
//   dk_j = sum_l D'_lj q_l + w_j (G_c v_j + g_c),
//   dv_j = sum_l E_lj (q_l . k_j) dn~_l + w_j G_c^T k_j,
// with (G_c, g_c) the backward state at the end of chunk c from the reverse
// chunk scan  G_{c-1} = 2^{m_prev - M_L} G_c + sum_j alpha_j q_j [dn~_j, dz~_j]^T,
// which starts from the gradient arriving at the final state (dC_T, dn_T;
// zero without one).
// q and k enter h and the final state only through e^{F_t} q_t, e^{i_t - F_t} k_t
// and the factor e^{F_T} of the final state (F the cumulative log forget
// gate), so d i_pre_t = k_t . dk_t and d log f_t is the reverse cumulative
// sum of q_s . dq_s - k_s . dk_s over s >= t plus the constant
// <dC_T, S~_T> + <dn_T, n~_T>.
//
// Kernels (all on the caller's stream, after the forward's state passes):
//   bwd_chunk_states_kernel  per (batch*head, superchunk, 64 x 64 state tile):
//                      every chunk's start state (and, with a final-state
//                      gradient, the final state's share of <dC_T, S~_T>).
//   bwd_scores_kernel  per (batch*head, chunk): Q K^T, the denominators, the
//                      readout (recomputed), dN V^T; writes P = E.(Q K^T) and
//                      D' (and transposes), 1/den~, dz~, d o_pre and a bias
//                      partial.
//   bwd_dq_kernel      per (batch*head, chunk, 64 features): dq and the chunk's
//                      local backward state sum_j alpha_j q_j [dn~_j, dz~_j]^T.
//   bwd_scan_kernel    reverse scan of the local backward states over chunks
//                      (in place: slot c ends up holding G_c), initial-state
//                      gradients.
//   bwd_dkv_kernel     per (batch*head, chunk, 64 features of dk or 64 columns
//                      of dv): dk, dv.
//   bwd_gate_total_kernel, bwd_gate_kernel  per (batch*head, chunk): d i_pre,
//                      d f_pre (reverse cumulative sum: chunk totals, then
//                      suffix sums with the later chunks' totals).
//   bwd_bias_kernel    d bias summed over the batch and the chunks.
//
// Tiles: 4 waves of 64 lanes own 16 rows each of a 64 x 64 output tile.
// Every operand is staged in LDS as it lies in memory (16-byte row stores);
// one whose contraction index runs along its rows is read with transposing
// LDS reads (mma64x).
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace mlstm {

namespace {

constexpr int BL = 64;  // chunk length of the backward pass

template <typename T>
struct BT {
  static constexpr int LD = 64 + 16 / (int)sizeof(T);  // LDS row stride (elements)
};

// MFMA operand fragments with the contraction index k in the order
// krow(lg, e) = 4 lg + (e & 3) + 16 (e >> 2) within each 32-wide k block (bf16;
// fp32: k = lg), so that an operand stored with k along its columns (row-major,
// k contiguous: two 8-byte reads) and one stored with k along its rows (two
// transposing ds_read_b64_tr_b16) agree on which k is which.
__device__ __forceinline__ bf16x8 frag_kcols(const __bf16* t, int ld, int row, int k0, int lg, int lr) {
  (void)lr;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(t + row * ld + k0 + 4 * lg);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(t + row * ld + k0 + 16 + 4 * lg);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = a[e];
    r[4 + e] = b[e];
  }
  return r;
}
// rows k of column col0 + lr: source lane lr addresses row k0 + 4 lg + lr/4,
// columns col0 + 4 (lr & 3) .. +3, so that output lane lr receives column col0 + lr
__device__ __forceinline__ bf16x8 frag_krows(const __bf16* t, int ld, int col0, int k0, int lg, int lr) {
  const __bf16* p = t + (k0 + 4 * lg + (lr >> 2)) * ld + col0 + 4 * (lr & 3);
  const bf16x4 a = ds_read_tr16(p);
  const bf16x4 b = ds_read_tr16(p + 16 * ld);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = a[e];
    r[4 + e] = b[e];
  }
  return r;
}
__device__ __forceinline__ float frag_kcols(const float* t, int ld, int row, int k0, int lg, int lr) {
  (void)lr;
  return t[row * ld + k0 + lg];
}
__device__ __forceinline__ float frag_krows(const float* t, int ld, int col0, int k0, int lg, int lr) {
  return t[(k0 + lg) * ld + col0 + lr];
}

// acc[n] += A B over k in [0, 64) for the wave's rows 16 w .. +15 and all 64
// columns.  A (rows m, contraction k): AR ? stored [k][m] : stored [m][k];
// B (contraction k, columns n): BR ? stored [k][n] : stored [n][k].
// acc[n][i] is row 16 w + 4 lg + i, column 16 n + lr.
template <typename T, bool AR, bool BR, int KB = 0, int KE = 64>
__device__ __forceinline__ void mma64x(f32x4 (&acc)[4], const T* A, int lda, const T* B, int ldb, int w, int lane) {
  constexpr int K = Mma<T>::K;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int k0 = KB; k0 < KE; k0 += K) {
    const typename Mma<T>::frag a =
        AR ? frag_krows(A, lda, 16 * w, k0, lg, lr) : frag_kcols(A, lda, 16 * w + lr, k0, lg, lr);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const typename Mma<T>::frag b =
          BR ? frag_krows(B, ldb, 16 * n, k0, lg, lr) : frag_kcols(B, ldb, 16 * n + lr, k0, lg, lr);
      acc[n] = Mma<T>::mma(a, b, acc[n]);
    }
  }
}

// Work-groups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  This bijection of [0, n) gives each XCD a contiguous range of logical
// indices, so that tiles which read the same data (the tiles of one chunk,
// or of one superchunk) share an L2: block b runs on XCD b % 8 and takes
// logical index start(b % 8) + b / 8.
__device__ __forceinline__ int xcd_local(int b, int n) {
  const int x = b & 7, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Block-diagonal memory (NB = 2 blocks of a 64-wide head): the contraction
// over a 64-wide index split at 32, one product per block.
template <typename T, bool AR, bool BR, int NB>
__device__ __forceinline__ void mma64x_blocks(f32x4 (&acc)[NB][4], const T* A, int lda, const T* B, int ldb, int w,
                                              int lane) {
  static_assert(NB == 1 || NB == 2, "one or two memory blocks");
  if constexpr (NB == 1) {
    mma64x<T, AR, BR>(acc[0], A, lda, B, ldb, w, lane);
  } else {
    mma64x<T, AR, BR, 0, 32>(acc[0], A, lda, B, ldb, w, lane);
    mma64x<T, AR, BR, 32, 64>(acc[1], A, lda, B, ldb, w, lane);
  }
}
// Output column tile n (columns 16 n .. 16 n + 15 of a 64-wide tile) lies in
// memory block n * NB / 4; rows of wave w in block w * NB / 4.
template <int NB>
__device__ __forceinline__ constexpr int col_block(int n) { return n * NB / 4; }

// dn~ = o dh / den~ for one element (the same expression in every kernel, so
// that each rounds it identically)
__device__ __forceinline__ float dn_of(float dh, float o, float rden) { return (dh * o) * rden; }

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[4]) {
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// 16 consecutive elements of type S as floats (bytes past the buffer: zero).
template <typename S>
__device__ __forceinline__ void load16f(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float (&x)[16]) {
  if constexpr (sizeof(S) == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off + 16 * h, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * h + 2 * e] = __uint_as_float(u[e] << 16);
        x[8 * h + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off + 16 * h, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * h + e] = __uint_as_float(u[e]);
    }
  }
}

// 16 consecutive elements of type S as loaded (raw words), to be unpacked
// later by unpack16f: a prefetch kept in this form is not waited for until
// its values are used.
template <typename S>
struct Raw16 {
  u32x4 u[sizeof(S) == 2 ? 2 : 4];
};
template <typename S>
__device__ __forceinline__ void load16raw(__amdgpu_buffer_rsrc_t r, unsigned byte_off, Raw16<S>& x) {
#pragma unroll
  for (int h = 0; h < (sizeof(S) == 2 ? 2 : 4); ++h) x.u[h] = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off + 16 * h, 0, 0);
}
template <typename S>
__device__ __forceinline__ void unpack16f(const Raw16<S>& x, float (&y)[16]) {
  if constexpr (sizeof(S) == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * h + 2 * e] = __uint_as_float(x.u[h][e] << 16);
        y[8 * h + 2 * e + 1] = __uint_as_float(x.u[h][e] & 0xffff0000u);
      }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[4 * h + e] = __uint_as_float(x.u[h][e]);
  }
}

// 16 consecutive fp32 values (in bounds).
__device__ __forceinline__ void ld16(const float* src, float (&x)[16]) {
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 u = *reinterpret_cast<const float4*>(src + e);
    x[e] = u.x, x[e + 1] = u.y, x[e + 2] = u.z, x[e + 3] = u.w;
  }
}

// Thread tid of 256 covers row tid >> 2, columns 16 (tid & 3) .. +15 of a 64 x 64 tile.
template <typename T>
__device__ __forceinline__ void st_row16(T* s, int r, int c0, const float (&x)[16]) {
  constexpr int LD = BT<T>::LD;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
      *reinterpret_cast<u32x4*>(s + r * LD + c0 + 8 * h) = u;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<float4*>(s + r * LD + c0 + 4 * h) =
          make_float4(x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]);
  }
}
// x from lane (lr + N) mod 16 of the same row of 16 lanes (DPP row_ror:N)
template <int N>
__device__ __forceinline__ float dpp_ror(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
// Stabiliser quantities of one chunk into LDS (threads 0..63): a_j, M_j,
// alpha_j, e^{-m_j}, w_j; returns nothing, sets *sdec to 2^{m_prev - M_L}.
__device__ __forceinline__ void load_chunk_gates(const BwdParams& p, int bh, int c, int tid, float* sa, float* sM,
                                                 float* sal, float* sem, float* sw) {
  if (tid < BL) {
    const size_t tg = (size_t)bh * p.NC * BL + (size_t)c * BL + tid;
    const float mp = p.ws_min[(size_t)bh * p.NC + c];
    const float a = p.ws_ga[tg];
    const float M = fmaxf(mp, p.ws_gg[tg]);
    const float ML = fmaxf(mp, p.ws_gg[(size_t)bh * p.NC * BL + (size_t)c * BL + BL - 1]);
    sa[tid] = a;
    sM[tid] = M;
    sal[tid] = exp2_fast(mp - M);
    sem[tid] = exp2_fast(-(p.ws_gb[tg] + M));
    sw[tid] = exp2_fast(a - ML);
  }
}

// ---------------------------------------------------------------- kernel 0
// Every chunk's start state from the superchunk start states of the
// forward's passes 1-2: per (batch*head, superchunk, 64 x 64 state tile) the
// superchunk's chunks in order, the tile in registers (MFMA layout: rows
// d = 16 w + 4 lg + i, columns c = 16 n + lr):
//   write S~ (and, column tile 0, n~ and m) as chunk c's start state,
//   S~ <- 2^{m - M_L} S~ + (w . K_c)^T V_c,  n~ <- 2^{m - M_L} n~ + sum_l w_l k_l,
//   m <- b_L + M_L,  with M_L = max(m, g_L) and w_l = 2^{a_l - M_L}
// (the forward's state update; K and V of the next chunk load during the
// current one's product).
template <typename T, int DQK, int NB>
// four waves per SIMD (108 registers, no spills; 2 % of the 7B backward)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void bwd_chunk_states_kernel(BwdParams p) {
  static_assert(NB == 1 || DQK == 64, "two blocks on 64-wide heads only");
  constexpr int LD = BT<T>::LD;
  constexpr unsigned ES = sizeof(T);
  constexpr int NDT = DQK / 64;
  __shared__ __attribute__((aligned(16))) T sK[BL * LD];  // w . K, token-major [l][d]
  __shared__ __attribute__((aligned(16))) T sV[BL * LD];  // V, token-major     [l][c]
  // bf16: w . K - bf16(w . K), so that the chunk states carry w . K to ~2^-16
  // (the backward's cancellations amplify state errors at long lengths)
  __shared__ __attribute__((aligned(16))) T sKl[sizeof(T) == 2 ? BL * LD : 8];
  __shared__ float sw[BL];
  __shared__ float sdec;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int NVT = p.DV / 64;
  const int bid = xcd_local((int)blockIdx.x, (int)gridDim.x);
  const int ct = bid % NVT;
  const int dt = (bid / NVT) % NDT;
  const int bs = bid / (NVT * NDT);
  const int bh = bs / p.NS, sc = bs % p.NS;
  const int r = tid >> 2, c0 = 16 * (tid & 3);
  const size_t NST = (size_t)DQK * p.DV + DQK;
  const bool lead = ct == 0;  // writes n~ and m as well
  const size_t NCL = (size_t)p.NC * BL;
  // The tile is held transposed, so that each lane owns 4 consecutive state
  // columns: acc[n][i] = S~[64 dt + 16 n + lr][64 ct + 16 w + 4 lg + i].
  const size_t toff = (size_t)(dt * 64 + lr) * p.DV + ct * 64 + 16 * w + 4 * lg;
  f32x4 acc[4];
  zero_acc(acc);
  // n~[64 dt + r] lives in thread 4 r of the lead work-group
  float nn = 0.f;
  const bool has = p.has_init || sc > 0;
  const float* S0 = p.sc_state + ((size_t)bh * p.NS + sc) * p.sc_nst;
  if (has) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if constexpr (NB == 1) {
        const float4 u = *reinterpret_cast<const float4*>(S0 + toff + (size_t)16 * n * p.DV);
        acc[n] = f32x4{u.x, u.y, u.z, u.w};
      } else if (col_block<NB>(n) == col_block<NB>(w)) {
        // block layout [NB][32][32]: d = 16 n + lr, c = 16 w + 4 lg + i, same block bb
        const int bb = col_block<NB>(n);
        const float4 u = *reinterpret_cast<const float4*>(S0 + (size_t)bb * 1024 + (16 * n + lr - 32 * bb) * 32 +
                                                          16 * w + 4 * lg - 32 * bb);
        acc[n] = f32x4{u.x, u.y, u.z, u.w};
      }
    }
    if (lead && !p.ret) nn = S0[p.sc_nst - DQK + dt * 64 + r];
  }
  float m = p.sc_min[(size_t)bh * p.NS + sc];  // meaningful in threads below 64
  const int cb = sc * p.G, ce = min(p.NC, cb + p.G);
  // with a gradient arriving at the final state, the last superchunk's walk
  // also applies its last chunk, and iteration ce holds the final state
  const int cend = (p.ws_cT && sc == p.NS - 1) ? ce + 1 : ce;
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
  const auto rnone = make_rsrc(nullptr, 0u);
  // The chunk to update next: its K and V slices (raw, unpacked when staged)
  // and gate logs load one chunk ahead, on every path and in every wave, so
  // that the compiler waits for them alone and not for the state stores
  // issued after them (a load past the walk goes through rnone: zeros).
  Raw16<T> kraw, vraw;
  float ga, gL, bL;
  auto load_next = [&](int cc) __attribute__((always_inline)) {
    const bool in = cc + 1 < cend;
    load16raw<T>(in ? rk : rnone, ((unsigned)(cc * BL + r) * DQK + dt * 64 + c0) * ES, kraw);
    load16raw<T>(in ? rv : rnone, ((unsigned)(cc * BL + r) * p.DV + ct * 64 + c0) * ES, vraw);
    const size_t tg = (size_t)bh * NCL + (size_t)min(cc, p.NC - 1) * BL;
    ga = p.ws_ga[tg + (tid & (BL - 1))];
    gL = p.ws_gg[tg + BL - 1];
    bL = p.ws_gb[tg + BL - 1];
  };
  load_next(cb);
  for (int c = cb; c < cend; ++c) {
    if (c == ce) {
      // the final state: this tile's share of <dC_T, S~_T> (+ <dn_T, n~_T>)
      float a = 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int d = dt * 64 + 16 * n + lr, cc = ct * 64 + 16 * w + 4 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float g;
          if constexpr (NB == 1) {
            g = p.dCT ? p.dCT[(size_t)bh * DQK * p.DV + (size_t)d * p.DV + cc + i] : 0.f;
          } else {  // block layout [NB][32][32]; off-diagonal entries are zero
            const int bb = d / 32;
            g = (p.dCT && (cc + i) / 32 == bb)
                    ? p.dCT[(size_t)bh * 2048 + bb * 1024 + (d - 32 * bb) * 32 + (cc + i - 32 * bb)]
                    : 0.f;
          }
          a += g * acc[n][i];
        }
      }
      if (lead && (tid & 3) == 0 && p.dnT) a += nn * p.dnT[(size_t)bh * DQK + dt * 64 + r];
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) a += __shfl_xor(a, d, 64);
      __syncthreads();  // sw is free
      if (lane == 0) sw[w] = a;
      __syncthreads();
      if (tid == 0) p.ws_cT[(size_t)bh * NDT * NVT + dt * NVT + ct] = sw[0] + sw[1] + sw[2] + sw[3];
      break;
    }
    float* St = p.ws_state + ((size_t)bh * p.NC + c) * NST;
#pragma unroll
    for (int n = 0; n < 4; ++n)
      *reinterpret_cast<float4*>(St + toff + (size_t)16 * n * p.DV) = make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
    if (lead && (tid & 3) == 0) St[(size_t)DQK * p.DV + dt * 64 + r] = nn;
    if (lead && dt == 0 && tid == 0) p.ws_min[(size_t)bh * p.NC + c] = m;
    if (c + 1 == cend) break;  // the next superchunk starts from its own start state
    __syncthreads();  // previous chunk's operands are consumed
    const float ML = fmaxf(m, gL);
    if (tid < BL) {
      sw[tid] = exp2_fast(ga - ML);
      if (tid == 0) sdec = exp2_fast(m - ML);
    }
    m = bL + ML;
    __syncthreads();
    const float wr = sw[r];
    float kx[16], vx[16];
    unpack16f<T>(kraw, kx);
    unpack16f<T>(vraw, vx);
    load_next(c + 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) kx[e] *= wr;
    st_row16<T>(sK, r, c0, kx);
    st_row16<T>(sV, r, c0, vx);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) kx[e] -= to_f32(from_f32<T>(kx[e]));
      st_row16<T>(sKl, r, c0, kx);
    }
    __syncthreads();
    const float dec = sdec;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[n][i] *= dec;
    mma64x<T, true, true>(acc, sV, LD, sK, LD, w, lane);  // S~^T += V^T (w . K)
    if constexpr (sizeof(T) == 2) mma64x<T, true, true>(acc, sV, LD, sKl, LD, w, lane);
    if constexpr (NB > 1) {  // the memory is block-diagonal
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (col_block<NB>(n) != col_block<NB>(w)) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (lead) {  // n~[64 dt + r] += sum_l w_l k_l, four threads per row
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        a += to_f32(sK[(16 * (tid & 3) + e) * LD + r]);
        if constexpr (sizeof(T) == 2) a += to_f32(sKl[(16 * (tid & 3) + e) * LD + r]);
      }
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      nn = dec * nn + a;
    }
  }
}

// ---------------------------------------------------------------- kernel 1
// The chunk's readout is recomputed here in fp32 (num~ = alpha Q S~_prev +
// P V) so that dh . h enters dz~ as sum_l P_jl D_jl + alpha_j dn~_j . (S~^T q_j)
// with the very P, D and dn~ that D' and the dq/dk/dv products use: where the
// denominator nearly cancels the direct term, rounding h (or any operand) on
// one side only would leave the cancellation residue in the gradient.
// RET (retention): no normaliser, so den~ = 1 and dz~ = 0, and the readout
// (needed only for dz~ and d o_pre) is not recomputed.
template <typename T, int DQK, bool RET, int NB>
// Two waves per SIMD (two work-groups per CU where the LDS allows): left to
// itself the compiler spends about 300 registers and runs one; the cap costs
// a few spills at the widest shapes and measured 10 % on the two-block
// backward, 3 % at the 7B head shape.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_scores_kernel(BwdParams p) {
  static_assert(NB == 1 || DQK == 64, "two blocks on 64-wide heads only");
  constexpr int LD = BT<T>::LD;
  constexpr int LDQ = DQK + 16 / (int)sizeof(T);
  constexpr unsigned ES = sizeof(T);
  __shared__ __attribute__((aligned(16))) T sQ[BL * LDQ];  // Q, token-major
  __shared__ __attribute__((aligned(16))) T sX[BL * LD];   // K, dN, S~ tiles  [j][d], [j][c], [d][c]
  __shared__ __attribute__((aligned(16))) T sY[BL * LD];   // V slices                  [l][c]
  __shared__ __attribute__((aligned(16))) T sP[NB][BL * LD];  // P of each memory block   [j][l]
  // bf16 lo parts x - bf16(x) of dn~ and then of the S~ tiles: D, dh . h and
  // the readout see dn~ and the state to ~2^-16 (a near-cancelling
  // dn~ . (v_l - y_j) must not see dn~ rounded; the initial state is exact
  // fp32 input)
  __shared__ __attribute__((aligned(16))) T sXl[sizeof(T) == 2 ? BL * LD : 8];
  // o_pre of the current d_v slice, as loaded (exact in T), unpadded [j][c]:
  // the d o_pre tile reads it in the MFMA layout
  __shared__ __attribute__((aligned(16))) T sO[RET ? 8 : BL * 64];
  __shared__ float sa[BL], sM[BL], sal[BL], sem[BL], sw[BL];
  __shared__ float sqn[BL], srow[BL], sden[BL], ssg[BL], sdz[BL];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
  const int hd = bh % p.H;
  const int r = tid >> 2, c0 = 16 * (tid & 3);
  const int t0 = c * BL;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  load_chunk_gates(p, bh, c, tid, sa, sM, sal, sem, sw);

  const bool has_state = p.has_init || c > 0;
  const float* Sp = p.ws_state + ((size_t)bh * p.NC + c) * NST;
  const float* nprev = Sp + (size_t)DQK * p.DV;
  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);

  // S = Q K^T over feature slices of 64 (Q kept whole); q_j . n~_prev alongside
  f32x4 accP[NB][4];  // per memory block: E . (Q_b K_b^T)
#pragma unroll
  for (int b = 0; b < NB; ++b) zero_acc(accP[b]);
  float qn = 0.f;
  for (int ds = 0; ds < DQK / 64; ++ds) {
    float x[16], y[16];
    load16f<T>(rq, ((unsigned)(t0 + r) * DQK + ds * 64 + c0) * ES, x);
    load16f<T>(rk, ((unsigned)(t0 + r) * DQK + ds * 64 + c0) * ES, y);
    if (has_state) {
#pragma unroll
      for (int e = 0; e < 16; ++e) qn += x[e] * nprev[ds * 64 + c0 + e];
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
        *reinterpret_cast<u32x4*>(sQ + r * LDQ + ds * 64 + c0 + 8 * h) = u;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        *reinterpret_cast<float4*>(sQ + r * LDQ + ds * 64 + c0 + 4 * h) =
            make_float4(x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]);
    }
    st_row16<T>(sX, r, c0, y);
    __syncthreads();
    mma64x_blocks<T, false, false, NB>(accP, sQ + ds * 64, LDQ, sX, LD, w, lane);
  }
  qn += __shfl_xor(qn, 1, 64);
  qn += __shfl_xor(qn, 2, 64);
  if ((tid & 3) == 0) sqn[r] = qn;

  // P = E . S (kept in fp32 registers), its row sums; P and P^T to the
  // workspace, P to LDS for the readout
  T* Ptw = static_cast<T*>(p.wsPt) + ((size_t)bh * p.NC + c) * NB * BL * BL;
  float rs[4] = {0.f, 0.f, 0.f, 0.f};  // the normaliser sums over the whole head
  // the gate logs of this lane's tokens l and j, read in one batch
  float saL[4], smJ[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) saL[n] = sa[16 * n + lr];
#pragma unroll
  for (int i = 0; i < 4; ++i) smJ[i] = sM[16 * w + 4 * lg + i];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int l = 16 * n + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * w + 4 * lg + i;
      const float e = l <= j ? exp2_fast(saL[n] - smJ[i]) : 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        accP[b][n][i] *= e;
        rs[i] += accP[b][n][i];
        sP[b][j * LD + l] = from_f32<T>(accP[b][n][i]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      store4f(Ptw + b * BL * BL + l * BL + 16 * w + 4 * lg, accP[b][n][0], accP[b][n][1], accP[b][n][2],
              accP[b][n][3]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) rs[i] += __shfl_xor(rs[i], d, 64);
    if (lr == 0) srow[16 * w + 4 * lg + i] = rs[i];
  }
  __syncthreads();
  if (tid < BL) {
    if constexpr (RET) {
      sden[tid] = 1.f;
      ssg[tid] = 0.f;
    } else {
      const float bias = p.bias ? p.bias[hd] : 0.f;
      const float z = srow[tid] + sal[tid] * sqn[tid] + bias * sem[tid];
      const float den = fmaxf(fabsf(z), sem[tid]);
      sden[tid] = 1.f / den;
      ssg[tid] = fabsf(z) > sem[tid] ? (z > 0.f ? 1.f : -1.f) : 0.f;
    }
  }
  __syncthreads();

  // over d_v slices: D = dN V^T, the readout num~ = alpha Q S~ + P V, and
  // dn~ . (Q S~) for dh . h; d o_pre from the recomputed outputs
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
  const auto rdh = make_rsrc(static_cast<const T*>(p.dh) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
  const auto ro = make_rsrc(p.o_pre ? static_cast<const T*>(p.o_pre) + (size_t)bh * p.T * p.DV : nullptr,
                            p.o_pre ? (unsigned)(p.T * p.DV) * ES : 0u);
  const auto rdo = make_rsrc(p.d_o ? static_cast<T*>(p.d_o) + (size_t)bh * p.T * p.DV : nullptr,
                             p.d_o ? (unsigned)(p.T * p.DV) * ES : 0u);
  const bool has_o = !RET && p.o_pre;
  const float rden = sden[r];
  f32x4 accD[NB][4];  // per memory block: dN_b V_b^T
#pragma unroll
  for (int b = 0; b < NB; ++b) zero_acc(accD[b]);
  float sint[4] = {0.f, 0.f, 0.f, 0.f};  // rows 16 w + 4 lg + i: dn~ . (Q S~) partials
  // Global loads run one step ahead: slice cs + 1's dh, o_pre, v and the next
  // S~ tile are in flight while the current ones are multiplied.  They are
  // issued on every path (the last step reloads its own slice and tile), so
  // that the compiler counts the same loads in flight everywhere and waits
  // only for the ones it needs.
  const int NCS = p.DV / 64;
  constexpr int NDS = DQK / 64;
  float g[16], x[16], vv[16], sv[16];
  auto load_slice = [&](int cs) {
    const unsigned off = ((unsigned)(t0 + r) * p.DV + cs * 64 + c0) * ES;
    load16f<T>(rdh, off, g);
    load16f<T>(rv, off, vv);
    load16f<T>(ro, off, x);  // zeros without o_pre
  };
  load_slice(0);
  const bool readout = has_state && !RET;
  ld16(Sp + (size_t)r * p.DV + c0, sv);  // (unused without a readout)
  for (int cs = 0; cs < NCS; ++cs) {
    if (p.o_pre) {
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = dn_of(g[e], sigmoidf_(x[e]), rden);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = dn_of(g[e], 1.f, rden);
    }
    __syncthreads();  // the previous slice's operands are consumed
    st_row16<T>(sX, r, c0, g);
    st_row16<T>(sY, r, c0, vv);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] -= to_f32(from_f32<T>(g[e]));
      st_row16<T>(sXl, r, c0, g);
    }
    if constexpr (!RET) {
      if (has_o) {
#pragma unroll
        for (int h = 0; h < 4; ++h) store4f(sO + r * 64 + c0 + 4 * h, x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]);
      }
    }
    load_slice(cs + 1 < NCS ? cs + 1 : cs);
    __syncthreads();
    f32x4 accI[4], accN[4];
    zero_acc(accI);
    zero_acc(accN);
    mma64x_blocks<T, false, false, NB>(accD, sX, LD, sY, LD, w, lane);  // sum_c dn~_jc v_lc
    if constexpr (sizeof(T) == 2) mma64x_blocks<T, false, false, NB>(accD, sXl, LD, sY, LD, w, lane);
    if constexpr (NB == 1) {
      mma64x<T, false, true>(accN, sP[0], LD, sY, LD, w, lane);  // sum_l P_jl v_lc
    } else {  // output column c takes the P of its block
      f32x4 t1[4];
      zero_acc(t1);
      mma64x<T, false, true>(accN, sP[0], LD, sY, LD, w, lane);
      mma64x<T, false, true>(t1, sP[1], LD, sY, LD, w, lane);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (col_block<NB>(n) == 1) accN[n] = t1[n];
    }
    // this lane's dn~ values, so that sX / sXl can hold the S~ tiles next
    float dnv[4][4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * lg + i, col = 16 * n + lr;
        dnv[n][i] = to_f32(sX[j * LD + col]);
        if constexpr (sizeof(T) == 2) dnv[n][i] += to_f32(sXl[j * LD + col]);
      }
    if (readout) {
      for (int ds = 0; ds < NDS; ++ds) {
        __syncthreads();  // sX / sXl are free (dn~ read, previous tile consumed)
        st_row16<T>(sX, r, c0, sv);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 16; ++e) sv[e] -= to_f32(from_f32<T>(sv[e]));
          st_row16<T>(sXl, r, c0, sv);
        }
        {  // the next S~ tile
          const bool more = ds + 1 < NDS;
          const int nds = more ? ds + 1 : 0, ncs = more ? cs : (cs + 1 < NCS ? cs + 1 : cs);
          ld16(Sp + (size_t)(nds * 64 + r) * p.DV + ncs * 64 + c0, sv);
        }
        __syncthreads();
        mma64x<T, false, true>(accI, sQ + ds * 64, LDQ, sX, LD, w, lane);  // sum_d q_jd S~_dc
        if constexpr (sizeof(T) == 2) mma64x<T, false, true>(accI, sQ + ds * 64, LDQ, sXl, LD, w, lane);
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) sint[i] += dnv[n][i] * accI[n][i];
    if constexpr (!RET) {
      // d o_pre = dh h~ sigma'(o_pre) with h~ = num~ / den~ and dn~ = sigma(o) dh / den~:
      // d o_pre = dn~ num~ sigma(-o_pre), num~ = alpha Q S~ + P V (rows past T are dropped)
      if (has_o) {
        float alj[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) alj[i] = sal[16 * w + 4 * lg + i];
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 16 * w + 4 * lg + i, col = 16 * n + lr;
            const float o = to_f32(sO[j * 64 + col]);
            const float d = dnv[n][i] * (alj[i] * accI[n][i] + accN[n][i]) * sigmoidf_(-o);
            bstore1<T>(rdo, ((unsigned)(t0 + j) * p.DV + cs * 64 + col) * ES, d);
          }
      }
    }
  }
  // dh . h = dn~ . num~ = sum_l P_jl D_jl + alpha_j dn~_j . (Q S~)_j
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = 0.f, b = sint[i];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int b = 0; b < NB; ++b) a += accP[b][n][i] * accD[b][n][i];
    const int j = 16 * w + 4 * lg + i;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      a += __shfl_xor(a, d, 64);
      b += __shfl_xor(b, d, 64);
    }
    if (lr == 0) {
      sdz[j] = -(a + sal[j] * b) * ssg[j] * sden[j];
      srow[j] = b;  // dn~_j . (Q S~)_j
    }
  }
  __syncthreads();
  // q_j . dq_j and the in-chunk part of k_j . dk_j from the fp32 products
  // (D'_jl (q_j . k_l) = (D_jl + dz~_j) P_jl):
  //   q_j . dq_j = sum_l D'_jl S_jl + alpha_j (dn~_j . (Q S~)_j + dz~_j q_j . n~),
  //   k_j . dk_j = sum_l D'_lj S_lj + w_j k_j . (G_c v_j + g_c)  (last term later)
  {
    float rsum[4] = {0.f, 0.f, 0.f, 0.f}, csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) x += (accD[b][n][i] + sdz[16 * w + 4 * lg + i]) * accP[b][n][i];
        rsum[i] += x;
        csum[n] += x;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) rsum[i] += __shfl_xor(rsum[i], d, 64);
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      csum[n] += __shfl_xor(csum[n], 16, 64);
      csum[n] += __shfl_xor(csum[n], 32, 64);
    }
    __syncthreads();  // srow (dn~ . (Q S~)) is read below, scol reuses sX
    float* scol = reinterpret_cast<float*>(sX);  // [4 waves][64 columns]
    if (lg == 0) {
#pragma unroll
      for (int n = 0; n < 4; ++n) scol[w * 64 + 16 * n + lr] = csum[n];
    }
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * lg + i;
        sqn[j] = rsum[i] + sal[j] * (srow[j] + sdz[j] * sqn[j]);
      }
    }
  }
  __syncthreads();
  if (tid < BL) {
    const float dz = sdz[tid];
    const size_t tg = (size_t)bh * p.NC * BL + (size_t)c * BL + tid;
    const float* scol = reinterpret_cast<const float*>(sX);
    p.ws_qdq[tg] = sqn[tid];
    p.ws_kdki[tg] = scol[tid] + scol[64 + tid] + scol[128 + tid] + scol[192 + tid];
    p.ws_rden[tg] = sden[tid];
    p.ws_dz[tg] = dz;
    float bsum = (t0 + tid < p.T) ? sem[tid] * dz : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) bsum += __shfl_xor(bsum, d, 64);
    if (tid == 0) p.ws_dbias[(size_t)bh * p.NC + c] = bsum;
  }

  // D' = E . (dN V^T + dz~) per memory block, stored transposed (dq and dk
  // both read D'^T: dq with transposing LDS reads)
  T* Dtw = static_cast<T*>(p.wsDt) + ((size_t)bh * p.NC + c) * NB * BL * BL;
  float saL2[4], smJ2[4], dzJ[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) saL2[n] = sa[16 * n + lr];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    smJ2[i] = sM[16 * w + 4 * lg + i];
    dzJ[i] = sdz[16 * w + 4 * lg + i];
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int l = 16 * n + lr;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float dv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * lg + i;
        const float e = l <= j ? exp2_fast(saL2[n] - smJ2[i]) : 0.f;
        dv4[i] = e * (accD[b][n][i] + dzJ[i]);
      }
      store4f(Dtw + b * BL * BL + l * BL + 16 * w + 4 * lg, dv4[0], dv4[1], dv4[2], dv4[3]);
    }
  }
}

// ---------------------------------------------------------------- kernel 2
template <typename T, int DQK, int NB>
// three waves per SIMD where the LDS allows (162 registers at d_qk = 256, no
// spills; 2 % of the 7B backward)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void bwd_dq_kernel(BwdParams p) {
  static_assert(NB == 1 || DQK == 64, "two blocks on 64-wide heads only");
  __shared__ __attribute__((aligned(16))) T sA2[NB > 1 ? BL * BT<T>::LD : 8];  // D' of block 1
  constexpr int LD = BT<T>::LD;
  constexpr unsigned ES = sizeof(T);
  constexpr int NDT = DQK / 64;
  // alpha_j is per row of dq and per contraction index of U, so one tile of
  // alpha dN serves both: the inter part of dq is alpha_j sum_c dN_jc S~_dc.
  __shared__ __attribute__((aligned(16))) T sA[BL * LD];  // D'^T [l][j], then alpha dN slices [j][c]
  __shared__ __attribute__((aligned(16))) T sB[BL * LD];  // K tile, then S~ slices  [l][d], [d][c]
  __shared__ __attribute__((aligned(16))) T sQ[BL * LD];  // Q of the tile           [j][d]
  // bf16 lo parts, x - bf16(x), of S~ and alpha dN: dq's S~ dn~ and the local
  // backward state then see dn~ as the scores kernel does (hi + lo), so the
  // near-cancellation of dn~ . v against dz~ holds in them too
  __shared__ __attribute__((aligned(16))) T sBl[sizeof(T) == 2 ? BL * LD : 8];
  __shared__ __attribute__((aligned(16))) T sAl[sizeof(T) == 2 ? BL * LD : 8];
  __shared__ float sa[BL], sM[BL], sal[BL], sem[BL], sw[BL], sden[BL], sdz[BL], snp[64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int bid = xcd_local((int)blockIdx.x, (int)gridDim.x);
  const int dt = bid % NDT;
  const int bc = bid / NDT;
  const int bh = bc / p.NC, c = bc % p.NC;
  const int r = tid >> 2, c0 = 16 * (tid & 3);
  const int t0 = c * BL;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  load_chunk_gates(p, bh, c, tid, sa, sM, sal, sem, sw);
  const bool has_state = p.has_init || c > 0;
  const float* Sp = p.ws_state + ((size_t)bh * p.NC + c) * NST;
  if (tid < BL) {
    const size_t tg = (size_t)bh * p.NC * BL + (size_t)c * BL + tid;
    sden[tid] = p.ws_rden[tg];
    sdz[tid] = p.ws_dz[tg];
    snp[tid] = has_state ? Sp[(size_t)DQK * p.DV + dt * 64 + tid] : 0.f;
  }
  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  {
    float x[16], y[16], d[16], d2[16];
    load16f<T>(rq, ((unsigned)(t0 + r) * DQK + dt * 64 + c0) * ES, x);
    load16f<T>(rk, ((unsigned)(t0 + r) * DQK + dt * 64 + c0) * ES, y);
    // D'^T [l][j] of each memory block
    const auto rD = make_rsrc(static_cast<const T*>(p.wsDt) + ((size_t)bh * p.NC + c) * NB * BL * BL,
                              (unsigned)(NB * BL * BL) * ES);
    load16f<T>(rD, (unsigned)(r * BL + c0) * ES, d);
    if constexpr (NB > 1) load16f<T>(rD, (unsigned)(BL * BL + r * BL + c0) * ES, d2);
    st_row16<T>(sQ, r, c0, x);
    st_row16<T>(sB, r, c0, y);
    st_row16<T>(sA, r, c0, d);
    if constexpr (NB > 1) st_row16<T>(sA2, r, c0, d2);
  }
  __syncthreads();
  f32x4 acc[4], accx[4];
  zero_acc(acc);
  zero_acc(accx);
  mma64x<T, true, true>(acc, sA, LD, sB, LD, w, lane);  // sum_l D'_jl k_l (D' held transposed)
  if constexpr (NB > 1) {  // feature column d takes the D' of its block
    f32x4 t1[4];
    zero_acc(t1);
    mma64x<T, true, true>(t1, sA2, LD, sB, LD, w, lane);
#pragma unroll
    for (int n = 0; n < 4; ++n)
      if (col_block<NB>(n) == 1) acc[n] = t1[n];
  }

  const auto rdh = make_rsrc(static_cast<const T*>(p.dh) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
  const auto ro = make_rsrc(p.o_pre ? static_cast<const T*>(p.o_pre) + (size_t)bh * p.T * p.DV : nullptr,
                            p.o_pre ? (unsigned)(p.T * p.DV) * ES : 0u);
  float* Uw = p.ws_U + ((size_t)bh * p.NC + c) * NST;
  const float rden = sden[r], alr = sal[r];
  const int NCS = p.DV / 64;
  // S~ rows [64 dt, 64 dt + 64) of the chunk's start state (zeros without one)
  const auto rS = make_rsrc(Sp + (size_t)dt * 64 * p.DV, has_state ? (unsigned)(64 * p.DV) * 4u : 0u);
  // one slice ahead (see the scores kernel), issued on every path: the last
  // step reloads its own slice
  float g[16], x[16], sv[16];
  auto load_slice = [&](int cs) {
    const unsigned off = ((unsigned)(t0 + r) * p.DV + cs * 64 + c0) * ES;
    load16f<T>(rdh, off, g);
    load16f<T>(ro, off, x);  // zeros without o_pre
    load16f<float>(rS, (unsigned)(r * p.DV + cs * 64 + c0) * 4u, sv);
  };
  load_slice(0);
  for (int cs = 0; cs < NCS; ++cs) {
    if (p.o_pre) {
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = dn_of(g[e], sigmoidf_(x[e]), rden);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = dn_of(g[e], 1.f, rden);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) g[e] *= alr;  // alpha_j dn~_jc
    __syncthreads();  // previous slice's operands (and D') are consumed
    st_row16<T>(sA, r, c0, g);
    st_row16<T>(sB, r, c0, sv);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sv[e] -= to_f32(from_f32<T>(sv[e]));
        g[e] -= to_f32(from_f32<T>(g[e]));
      }
      st_row16<T>(sBl, r, c0, sv);
      st_row16<T>(sAl, r, c0, g);
    }
    load_slice(cs + 1 < NCS ? cs + 1 : cs);
    __syncthreads();
    mma64x<T, false, false>(accx, sA, LD, sB, LD, w, lane);  // sum_c alpha_j dN_jc S~_dc
    if constexpr (sizeof(T) == 2) {
      mma64x<T, false, false>(accx, sA, LD, sBl, LD, w, lane);
      mma64x<T, false, false>(accx, sAl, LD, sB, LD, w, lane);
    }
    // U_dc = sum_j q_jd alpha_j dN_jc, held transposed (u[n][i] = U[16 n + lr][16 w + 4 lg + i])
    // so that each lane stores 4 consecutive columns at once
    f32x4 u[4];
    zero_acc(u);
    mma64x<T, true, true>(u, sA, LD, sQ, LD, w, lane);
    if constexpr (sizeof(T) == 2) mma64x<T, true, true>(u, sAl, LD, sQ, LD, w, lane);
    if constexpr (NB > 1) {  // the memory (and its gradient) is block-diagonal
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (col_block<NB>(n) != col_block<NB>(w)) u[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
      *reinterpret_cast<float4*>(Uw + (size_t)(dt * 64 + 16 * n + lr) * p.DV + cs * 64 + 16 * w + 4 * lg) =
          make_float4(u[n][0], u[n][1], u[n][2], u[n][3]);
  }
  if (tid < 64) {  // normaliser column: sum_j q_jd alpha_j dz~_j
    float a = 0.f;
    for (int j = 0; j < BL; ++j) a += to_f32(sQ[j * LD + tid]) * sal[j] * sdz[j];
    Uw[(size_t)DQK * p.DV + dt * 64 + tid] = a;
  }
  // dq = intra + alpha (S~ dn~ + n~ dz~) (rows past T are dropped)
  const auto rdq = make_rsrc(static_cast<T*>(p.dq) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int d = 16 * n + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * w + 4 * lg + i;
      const float v = acc[n][i] + accx[n][i] + sal[j] * sdz[j] * snp[d];
      bstore1<T>(rdq, ((unsigned)(t0 + j) * DQK + dt * 64 + d) * ES, v);
    }
  }
}

// ---------------------------------------------------------------- kernel 3
// Thread = 4 consecutive entries of the backward state; chunks in reverse,
// in windows of SW whose local states are all loaded before any is replaced.
// dC0, dn0 from the backward state before the first chunk (entries e0 .. e0+3
// of the flattened [S~ | n~] state, full layout); dC0 in the memory's block layout.
__device__ __forceinline__ void store_init_grad(const BwdParams& p, int DQK, int bh, size_t e0, float4 G) {
  const size_t CS = (size_t)DQK * p.DV, NST = CS + DQK;
  const float g4[4] = {G.x, G.y, G.z, G.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t e = e0 + i;
    if (e < CS) {
      if (p.dC0) {
        if (p.NB == 1) {
          p.dC0[(size_t)bh * CS + e] = g4[i];
        } else {  // [nb][d_qk/nb][d_v/nb]; off-diagonal entries are zero
          const int d = (int)(e / p.DV), cc = (int)(e % p.DV);
          const int bq = DQK / p.NB, bv = p.DV / p.NB, b = d / bq;
          if (cc / bv == b)
            p.dC0[(size_t)bh * (CS / p.NB) + (size_t)b * bq * bv + (size_t)(d % bq) * bv + cc % bv] = g4[i];
        }
      }
    } else if (e < NST) {
      if (p.dn0) p.dn0[(size_t)bh * DQK + (e - CS)] = g4[i];
    }
  }
}

// The gradient arriving at the final state for entries e0 .. e0+3 of the
// flattened [S~ | n~] state (full layout; dC_T in the memory's block layout,
// zero off the diagonal blocks); zero without one.
__device__ __forceinline__ float4 load_final_grad(const BwdParams& p, int DQK, int bh, size_t e0) {
  const size_t CS = (size_t)DQK * p.DV, NST = CS + DQK;
  float g4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t e = e0 + i;
    if (e < CS) {
      if (p.dCT) {
        if (p.NB == 1) {
          g4[i] = p.dCT[(size_t)bh * CS + e];
        } else {
          const int d = (int)(e / p.DV), cc = (int)(e % p.DV);
          const int bq = DQK / p.NB, bv = p.DV / p.NB, b = d / bq;
          if (cc / bv == b) g4[i] = p.dCT[(size_t)bh * (CS / p.NB) + (size_t)b * bq * bv + (size_t)(d % bq) * bv + cc % bv];
        }
      }
    } else if (e < NST) {
      if (p.dnT) g4[i] = p.dnT[(size_t)bh * DQK + (e - CS)];
    }
  }
  return make_float4(g4[0], g4[1], g4[2], g4[3]);
}

template <int SW>
__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdParams p, int DQK) {
  const int bh = blockIdx.y;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const bool active = e0 < NST;
  float* base = p.ws_U + (size_t)bh * p.NC * NST;
  const float* gg = p.ws_gg + (size_t)bh * p.NC * BL;
  const float* mn = p.ws_min + (size_t)bh * p.NC;
  float4 G = active ? load_final_grad(p, DQK, bh, e0) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c1 = p.NC - 1; c1 >= 0; c1 -= SW) {
    float4 u[SW];
    float dec[SW];
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      const int c = c1 - j;
      u[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      dec[j] = 0.f;
      if (c >= 0) {
        const float mp = mn[c];
        dec[j] = exp2_fast(mp - fmaxf(mp, gg[(size_t)c * BL + BL - 1]));
        if (active) u[j] = *reinterpret_cast<const float4*>(base + (size_t)c * NST + e0);
      }
    }
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      const int c = c1 - j;
      if (c >= 0) {
        if (active) *reinterpret_cast<float4*>(base + (size_t)c * NST + e0) = G;
        const float f = dec[j];
        G.x = f * G.x + u[j].x;
        G.y = f * G.y + u[j].y;
        G.z = f * G.z + u[j].z;
        G.w = f * G.w + u[j].w;
      }
    }
  }
  if (active) store_init_grad(p, DQK, bh, e0, G);
}

// Two-level form of the same scan for long sequences (many chunks, few
// work-groups per chain): segments of SEG chunks run their local scans in
// parallel (bwd_scan_local_kernel: every slot gets the segment-local
// G_c, and the segment's local total goes to ws_carry), a short chain over
// the segments turns the totals into the carry entering each segment's end
// (bwd_scan_carry_kernel, which also writes dC0, dn0), and a second parallel
// pass adds each carry, decayed to the chunk, to the segment's slots
// (bwd_scan_apply_kernel).
constexpr int SEG = 32;

__device__ __forceinline__ float chunk_decay(const BwdParams& p, int bh, int c) {
  const float mp = p.ws_min[(size_t)bh * p.NC + c];
  return exp2_fast(mp - fmaxf(mp, p.ws_gg[(size_t)bh * p.NC * BL + (size_t)c * BL + BL - 1]));
}

__global__ __launch_bounds__(256) void bwd_scan_local_kernel(BwdParams p, int DQK) {
  const int bh = blockIdx.y, sg = blockIdx.z;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= NST) return;
  float* base = p.ws_U + (size_t)bh * p.NC * NST;
  const int cb = sg * SEG, ce = min(p.NC, cb + SEG);
  float4 G = make_float4(0.f, 0.f, 0.f, 0.f);
  float fs = 1.f;  // decay over the whole segment
  const bool rec = blockIdx.x == 0 && threadIdx.x == 0;  // records r_c for the dk/dv pass
  for (int c = ce - 1; c >= cb; --c) {
    const float4 u = *reinterpret_cast<const float4*>(base + (size_t)c * NST + e0);
    *reinterpret_cast<float4*>(base + (size_t)c * NST + e0) = G;
    if (rec) p.ws_rdec[(size_t)bh * p.NC + c] = fs;  // decay from the end of chunk c to the segment's end
    const float f = chunk_decay(p, bh, c);
    fs *= f;
    G.x = f * G.x + u.x;
    G.y = f * G.y + u.y;
    G.z = f * G.z + u.z;
    G.w = f * G.w + u.w;
  }
  *reinterpret_cast<float4*>(p.ws_carry + ((size_t)bh * p.NSEG + sg) * NST + e0) = G;
  if (e0 == 0) p.ws_segdec[(size_t)bh * p.NSEG + sg] = fs;
}

__global__ __launch_bounds__(256) void bwd_scan_carry_kernel(BwdParams p, int DQK) {
  const int bh = blockIdx.y;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= NST) return;
  float4 G = load_final_grad(p, DQK, bh, e0);  // entering the end of segment sg
  constexpr int W = 8;  // segments whose totals load together
  for (int s1 = p.NSEG - 1; s1 >= 0; s1 -= W) {
    float4 tot[W];
    float f[W];
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const int sg = s1 - j;
      tot[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      f[j] = 0.f;
      if (sg >= 0) {
        tot[j] = *reinterpret_cast<const float4*>(p.ws_carry + ((size_t)bh * p.NSEG + sg) * NST + e0);
        f[j] = p.ws_segdec[(size_t)bh * p.NSEG + sg];
      }
    }
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const int sg = s1 - j;
      if (sg >= 0) {
        *reinterpret_cast<float4*>(p.ws_carry + ((size_t)bh * p.NSEG + sg) * NST + e0) = G;
        G.x = f[j] * G.x + tot[j].x;
        G.y = f[j] * G.y + tot[j].y;
        G.z = f[j] * G.z + tot[j].z;
        G.w = f[j] * G.w + tot[j].w;
      }
    }
  }
  store_init_grad(p, DQK, bh, e0, G);
}

__global__ __launch_bounds__(256) void bwd_scan_apply_kernel(BwdParams p, int DQK) {
  const int bh = blockIdx.y, sg = blockIdx.z;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  // only a final-state gradient enters the last segment
  if (e0 >= NST || (sg == p.NSEG - 1 && !p.dCT && !p.dnT)) return;
  float* base = p.ws_U + (size_t)bh * p.NC * NST;
  const float4 C = *reinterpret_cast<const float4*>(p.ws_carry + ((size_t)bh * p.NSEG + sg) * NST + e0);
  const int cb = sg * SEG, ce = min(p.NC, cb + SEG);
  float r = 1.f;  // decay from the end of chunk c to the end of the segment
  for (int c = ce - 1; c >= cb; --c) {
    float4* slot = reinterpret_cast<float4*>(base + (size_t)c * NST + e0);
    float4 g = *slot;
    g.x += r * C.x;
    g.y += r * C.y;
    g.z += r * C.z;
    g.w += r * C.w;
    *slot = g;
    r *= chunk_decay(p, bh, c);
  }
}

// ---------------------------------------------------------------- kernel 4
// FC: after a two-level scan without its apply pass, the slots hold the
// segment-local states G'_c; G_c = G'_c + r_c C_s (C_s: the state entering the
// end of segment s, r_c: the decay from the end of chunk c to there) is
// formed as the slices load.
template <typename T, int DQK, int NB, bool FC = false>
__global__ __launch_bounds__(256) void bwd_dkv_kernel(BwdParams p) {
  static_assert(NB == 1 || DQK == 64, "two blocks on 64-wide heads only");
  __shared__ __attribute__((aligned(16))) T sA2[NB > 1 ? BL * BT<T>::LD : 8];  // D'^T or P^T of block 1
  constexpr int LD = BT<T>::LD;
  constexpr unsigned ES = sizeof(T);
  constexpr int NDT = DQK / 64;
  __shared__ __attribute__((aligned(16))) T sA[BL * LD];
  __shared__ __attribute__((aligned(16))) T sB[BL * LD];
  __shared__ __attribute__((aligned(16))) T sK[BL * LD];  // dk tiles: K of the tile [j][d]
  // bf16 dk tiles: G - bf16(G), so that k . dk (hence d i_pre, d f_pre) sees G to ~2^-16
  __shared__ __attribute__((aligned(16))) T sBl[sizeof(T) == 2 ? BL * LD : 8];
  __shared__ float sa[BL], sM[BL], sal[BL], sem[BL], sw[BL], sg[64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int NVT = p.DV / 64;
  const int bid = xcd_local((int)blockIdx.x, (int)gridDim.x);
  const int tile = bid % (NDT + NVT);
  const int bc = bid / (NDT + NVT);
  const int bh = bc / p.NC, c = bc % p.NC;
  const int r = tid >> 2, c0 = 16 * (tid & 3);
  const int t0 = c * BL;
  const size_t NST = (size_t)DQK * p.DV + DQK;
  load_chunk_gates(p, bh, c, tid, sa, sM, sal, sem, sw);
  const float* Gc = p.ws_U + ((size_t)bh * p.NC + c) * NST;  // G_c, then g_c
  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
  // G_c; a load through rnone reads zeros and touches no memory: the next
  // slice's loads are issued on every path, so that the compiler counts the
  // same loads in flight everywhere
  const auto rG = make_rsrc(Gc, (unsigned)(DQK * p.DV) * 4u);
  const auto rnone = make_rsrc(nullptr, 0u);
  const float* Cs = FC ? p.ws_carry + ((size_t)bh * p.NSEG + c / SEG) * NST : nullptr;
  const auto rC = make_rsrc(Cs, FC ? (unsigned)(DQK * p.DV) * 4u : 0u);
  const float rc = FC ? p.ws_rdec[(size_t)bh * p.NC + c] : 0.f;
  float cv[FC ? 16 : 1];  // the carry's slice beside each G slice
  auto add_carry = [&](float (&g)[16]) __attribute__((always_inline)) {
    if constexpr (FC) {
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] += rc * cv[e];
    }
  };
  // this chunk's D'^T and P^T tiles of each memory block
  const size_t tile0 = ((size_t)bh * p.NC + c) * NB * BL * BL;
  f32x4 acc[4], accx[4];
  zero_acc(acc);
  zero_acc(accx);
  if (tile < NDT) {
    // dk_j = sum_l D'_lj q_l + w_j (G_c v_j + g_c), features [64 dt, 64 dt + 64)
    const int dt = tile;
    if (tid < 64)
      sg[tid] = Gc[(size_t)DQK * p.DV + dt * 64 + tid] + (FC ? rc * Cs[(size_t)DQK * p.DV + dt * 64 + tid] : 0.f);
    const int NCS = p.DV / 64;
    float vv[16], sv[16];  // V and G slices, one ahead (the first in flight with Q, K, D'^T)
    {
      float x[16], y[16], d[16], d2[16];
      load16f<T>(rq, ((unsigned)(t0 + r) * DQK + dt * 64 + c0) * ES, x);
      load16f<T>(rk, ((unsigned)(t0 + r) * DQK + dt * 64 + c0) * ES, y);
      const auto rD = make_rsrc(static_cast<const T*>(p.wsDt) + tile0, (unsigned)(NB * BL * BL) * ES);
      load16f<T>(rD, (unsigned)(r * BL + c0) * ES, d);
      if constexpr (NB > 1) load16f<T>(rD, (unsigned)(BL * BL + r * BL + c0) * ES, d2);
      load16f<T>(rv, ((unsigned)(t0 + r) * p.DV + c0) * ES, vv);
      load16f<float>(rG, (unsigned)((dt * 64 + r) * p.DV + c0) * 4u, sv);
      if constexpr (FC) load16f<float>(rC, (unsigned)((dt * 64 + r) * p.DV + c0) * 4u, cv);
      st_row16<T>(sA, r, c0, d);
      if constexpr (NB > 1) st_row16<T>(sA2, r, c0, d2);
      st_row16<T>(sB, r, c0, x);  // Q [l][d]
      st_row16<T>(sK, r, c0, y);
    }
    __syncthreads();
    mma64x<T, false, true>(acc, sA, LD, sB, LD, w, lane);  // sum_l D'_lj q_ld
    if constexpr (NB > 1) {  // feature column d takes the D' of its block
      f32x4 t1[4];
      zero_acc(t1);
      mma64x<T, false, true>(t1, sA2, LD, sB, LD, w, lane);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (col_block<NB>(n) == 1) acc[n] = t1[n];
    }
    for (int cs = 0; cs < NCS; ++cs) {
      __syncthreads();
      st_row16<T>(sA, r, c0, vv);
      add_carry(sv);
      st_row16<T>(sB, r, c0, sv);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] -= to_f32(from_f32<T>(sv[e]));
        st_row16<T>(sBl, r, c0, sv);
      }
      {
        const bool more = cs + 1 < NCS;
        load16f<T>(more ? rv : rnone, ((unsigned)(t0 + r) * p.DV + (cs + 1) * 64 + c0) * ES, vv);
        load16f<float>(more ? rG : rnone, (unsigned)((dt * 64 + r) * p.DV + (cs + 1) * 64 + c0) * 4u, sv);
        if constexpr (FC)
          load16f<float>(more ? rC : rnone, (unsigned)((dt * 64 + r) * p.DV + (cs + 1) * 64 + c0) * 4u, cv);
      }
      __syncthreads();
      mma64x<T, false, false>(accx, sA, LD, sB, LD, w, lane);  // sum_c v_jc G_dc
      if constexpr (sizeof(T) == 2) mma64x<T, false, false>(accx, sA, LD, sBl, LD, w, lane);
    }
    // (rows past T are dropped by the descriptor)
    const auto rdk = make_rsrc(static_cast<T*>(p.dk) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
    float kd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int d = 16 * n + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * lg + i;
        const float x = sw[j] * (accx[n][i] + sg[d]);
        bstore1<T>(rdk, ((unsigned)(t0 + j) * DQK + dt * 64 + d) * ES, acc[n][i] + x);
        kd[i] += to_f32(sK[j * LD + d]) * x;  // w_j k_j . (G_c v_j + g_c)
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // row sums over the 16 lanes lr
      kd[i] += dpp_ror<8>(kd[i]);
      kd[i] += dpp_ror<4>(kd[i]);
      kd[i] += dpp_ror<2>(kd[i]);
      kd[i] += dpp_ror<1>(kd[i]);
      if (lr == 0) p.ws_kdk[((size_t)bh * p.NC * BL + (size_t)c * BL + 16 * w + 4 * lg + i) * NDT + dt] = kd[i];
    }
  } else {
    // dv_j = sum_l P_lj dn~_l + w_j G_c^T k_j, columns [64 ct, 64 ct + 64)
    const int ct = tile - NDT;
    const auto rdh = make_rsrc(static_cast<const T*>(p.dh) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
    const auto ro = make_rsrc(p.o_pre ? static_cast<const T*>(p.o_pre) + (size_t)bh * p.T * p.DV : nullptr,
                              p.o_pre ? (unsigned)(p.T * p.DV) * ES : 0u);
    float y[16], sv[16];  // K and G slices, one ahead (the first in flight with dh, P^T)
    {
      const float rden = p.ws_rden[(size_t)bh * p.NC * BL + (size_t)c * BL + r];
      float g[16], x[16], d[16], d2[16];
      const unsigned off = ((unsigned)(t0 + r) * p.DV + ct * 64 + c0) * ES;
      load16f<T>(rdh, off, g);
      load16f<T>(ro, off, x);  // zeros without o_pre
      const auto rP = make_rsrc(static_cast<const T*>(p.wsPt) + tile0, (unsigned)(NB * BL * BL) * ES);
      load16f<T>(rP, (unsigned)(r * BL + c0) * ES, d);
      if constexpr (NB > 1) load16f<T>(rP, (unsigned)(BL * BL + r * BL + c0) * ES, d2);
      load16f<T>(rk, ((unsigned)(t0 + r) * DQK + c0) * ES, y);
      load16f<float>(rG, (unsigned)(r * p.DV + ct * 64 + c0) * 4u, sv);
      if constexpr (FC) load16f<float>(rC, (unsigned)(r * p.DV + ct * 64 + c0) * 4u, cv);
      if (p.o_pre) {
#pragma unroll
        for (int e = 0; e < 16; ++e) g[e] = dn_of(g[e], sigmoidf_(x[e]), rden);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) g[e] = dn_of(g[e], 1.f, rden);
      }
      st_row16<T>(sA, r, c0, d);
      if constexpr (NB > 1) st_row16<T>(sA2, r, c0, d2);
      st_row16<T>(sB, r, c0, g);  // dN [l][c]
    }
    __syncthreads();
    mma64x<T, false, true>(acc, sA, LD, sB, LD, w, lane);  // sum_l P_lj dn~_lc
    if constexpr (NB > 1) {  // value column c takes the P of its block
      f32x4 t1[4];
      zero_acc(t1);
      mma64x<T, false, true>(t1, sA2, LD, sB, LD, w, lane);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (col_block<NB>(n) == 1) acc[n] = t1[n];
    }
    for (int ds = 0; ds < NDT; ++ds) {
      __syncthreads();
      st_row16<T>(sA, r, c0, y);
      add_carry(sv);
      st_row16<T>(sB, r, c0, sv);  // G [d][c]
      {
        const bool more = ds + 1 < NDT;
        load16f<T>(more ? rk : rnone, ((unsigned)(t0 + r) * DQK + (ds + 1) * 64 + c0) * ES, y);
        load16f<float>(more ? rG : rnone, (unsigned)(((ds + 1) * 64 + r) * p.DV + ct * 64 + c0) * 4u, sv);
        if constexpr (FC)
          load16f<float>(more ? rC : rnone, (unsigned)(((ds + 1) * 64 + r) * p.DV + ct * 64 + c0) * 4u, cv);
      }
      __syncthreads();
      mma64x<T, false, true>(accx, sA, LD, sB, LD, w, lane);  // sum_d k_jd G_dc
    }
    // (rows past T are dropped by the descriptor)
    const auto rdv = make_rsrc(static_cast<T*>(p.dv) + (size_t)bh * p.T * p.DV, (unsigned)(p.T * p.DV) * ES);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int col = 16 * n + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * lg + i;
        bstore1<T>(rdv, ((unsigned)(t0 + j) * p.DV + ct * 64 + col) * ES, acc[n][i] + sw[j] * accx[n][i]);
      }
    }
  }
}

// dk and dv of one chunk in one work-group of 8 waves (bf16, d_qk = 64 NDT,
// one memory block).  G_c is read from memory once, in 64 x 64 blocks (feature
// block a inner, value-column block b outer).  Each block is staged in LDS as
// its hi and lo bf16 parts and serves both products:
//   waves 0..3, dk: wave w takes token strips 2 (w >> 1) and 2 (w >> 1) + 1
//     (16 rows each) and feature columns [32 (w & 1), +32) of every feature
//     block: dk_inter[., a] += V[., b] G[a, b]^T (hi and lo parts), and at the
//     end dk = D'^T Q + w (dk_inter + g_c) and the rows' partials of k . dk;
//   waves 4..7, dv: wave w takes token strip s = w - 4: dv[s, b] += K[s, a] G[a, b]
//     (hi part) over the feature blocks, plus P^T dN[:, b]; value block b is
//     complete, and stored, when its inner loop over a ends.
// The G blocks are loaded NDT ahead into registers, with one barrier per block
// (two LDS buffers).  The V and dN column blocks are double-buffered too and load
// one outer step ahead.  Q, K and D'^T stay in LDS for the whole chunk.
template <int NDT>
__global__ __launch_bounds__(512) void bwd_dkv_chunk_kernel(BwdParams p) {
  using T = __bf16;
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int DQK = 64 * NDT;
  constexpr int PF = NDT;         // G blocks in flight (register slots)
  constexpr int QLD = DQK + 8;    // row stride of sQ, sK (bf16)
  constexpr int GLD = BT<T>::LD;  // row stride of the 64 x 64 blocks
  constexpr unsigned ES = 2;
  static_assert(NDT >= 2 && (NDT & (NDT - 1)) == 0, "feature blocks: a power of two, at least 2");
  __shared__ __attribute__((aligned(16))) T sQ[BL * QLD];
  __shared__ __attribute__((aligned(16))) T sK[BL * QLD];
  __shared__ __attribute__((aligned(16))) T sGh[2][BL * GLD];
  __shared__ __attribute__((aligned(16))) T sGl[2][BL * GLD];
  __shared__ __attribute__((aligned(16))) T sV[2][BL * GLD];
  __shared__ __attribute__((aligned(16))) T sN[2][BL * GLD];
  __shared__ __attribute__((aligned(16))) T sDt[BL * GLD];
  __shared__ float sa[BL], sM[BL], sal[BL], sem[BL], sw[BL], sg[DQK];
  __shared__ float skd[2][BL];  // k . dk partials of the two feature halves
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const bool dk_wave = w < 4;
  const int s = w & 3;                  // dv waves: token strip
  const int sp = (w >> 1) & 1, fh = w & 1;  // dk waves: strip pair, feature half
  const int bh = (int)blockIdx.x / p.NC, c = (int)blockIdx.x % p.NC;
  const int t0 = c * BL;
  const int DV = p.DV, NVT = DV / 64, NIT = NDT * NVT;
  const size_t NST = (size_t)DQK * DV + DQK;
  const int r = tid >> 3, c8 = 8 * (tid & 7);  // staging of a 64 x 64 block: row, 8 columns
  load_chunk_gates(p, bh, c, tid, sa, sM, sal, sem, sw);
  const float* Gc = p.ws_U + ((size_t)bh * p.NC + c) * NST;  // G_c, then g_c
  if (tid < DQK) sg[tid] = Gc[(size_t)DQK * DV + tid];
  const float rden = p.ws_rden[(size_t)bh * p.NC * BL + (size_t)c * BL + r];
  const bool has_o = p.o_pre != nullptr;
  const auto rG = make_rsrc(Gc, (unsigned)(DQK * DV) * 4u);
  const auto rq = make_rsrc(static_cast<const T*>(p.q) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rk = make_rsrc(static_cast<const T*>(p.k) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rv = make_rsrc(static_cast<const T*>(p.v) + (size_t)bh * p.T * DV, (unsigned)(p.T * DV) * ES);
  const auto rdh = make_rsrc(static_cast<const T*>(p.dh) + (size_t)bh * p.T * DV, (unsigned)(p.T * DV) * ES);
  const auto ro = make_rsrc(has_o ? static_cast<const T*>(p.o_pre) + (size_t)bh * p.T * DV : nullptr,
                            has_o ? (unsigned)(p.T * DV) * ES : 0u);
  // outputs: 16-byte stores through descriptors that end at token T (rows past it are dropped)
  const auto rdk = make_rsrc(static_cast<T*>(p.dk) + (size_t)bh * p.T * DQK, (unsigned)(p.T * DQK) * ES);
  const auto rdv = make_rsrc(static_cast<T*>(p.dv) + (size_t)bh * p.T * DV, (unsigned)(p.T * DV) * ES);
  const size_t tile0 = ((size_t)bh * p.NC + c) * BL * BL;  // this chunk's D'^T and P^T tiles
  const auto rdt = make_rsrc(static_cast<const T*>(p.wsDt) + tile0, (unsigned)(BL * BL) * ES);
  const auto rpt = make_rsrc(static_cast<const T*>(p.wsPt) + tile0, (unsigned)(BL * BL) * ES);
  // Every load below is issued unconditionally, so that the compiler counts
  // the same loads in flight on every path and waits only for the one it
  // needs; a load with nothing to fetch goes through a zero-size descriptor
  // (reads zero, touches no memory).
  const auto rnone = make_rsrc(nullptr, 0u);

  // G block i (a = i % NDT, b = i / NDT): this thread's 8 floats (zero past the last block)
  u32x4 gr[PF][2];
  auto g_load = [&](int i, u32x4(&dst)[2]) __attribute__((always_inline)) {
    const int b = i / NDT, a = i % NDT;
    const auto rg = i < NIT ? rG : rnone;
    const unsigned off = ((unsigned)(64 * a + r) * DV + 64 * b + c8) * 4u;
    dst[0] = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0);
    dst[1] = __builtin_amdgcn_raw_buffer_load_b128(rg, off + 16, 0, 0);
  };
  // ... into LDS buffer buf as hi = bf16(G) and lo = bf16(G - hi)
  auto g_store = [&](int buf, const u32x4(&src)[2]) __attribute__((always_inline)) {
    u32x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = __uint_as_float(src[e >> 1][2 * (e & 1)]);
      const float x1 = __uint_as_float(src[e >> 1][2 * (e & 1) + 1]);
      hi[e] = pack_bf16x2(x0, x1);
      lo[e] = pack_bf16x2(x0 - __uint_as_float(hi[e] << 16), x1 - __uint_as_float(hi[e] & 0xffff0000u));
    }
    *reinterpret_cast<u32x4*>(&sGh[buf][r * GLD + c8]) = hi;
    *reinterpret_cast<u32x4*>(&sGl[buf][r * GLD + c8]) = lo;
  };
  // value-column block b of V and of dh (and o_pre): this thread's 8
  // elements (zero past the last block)
  u32x4 nh, no, nv;
  auto nv_load = [&](int b) __attribute__((always_inline)) {
    const bool in = b < NVT;
    const unsigned off = ((unsigned)(t0 + r) * DV + 64 * b + c8) * ES;
    nh = __builtin_amdgcn_raw_buffer_load_b128(in ? rdh : rnone, off, 0, 0);
    no = __builtin_amdgcn_raw_buffer_load_b128(in ? ro : rnone, off, 0, 0);
    nv = __builtin_amdgcn_raw_buffer_load_b128(in ? rv : rnone, off, 0, 0);
  };
  // ... into LDS buffer buf: V as loaded, dN = o dh / den~ rounded to bf16
  auto nv_store = [&](int buf) __attribute__((always_inline)) {
    u32x4 dn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float g0 = __uint_as_float(nh[e] << 16), g1 = __uint_as_float(nh[e] & 0xffff0000u);
      if (has_o) {
        g0 = dn_of(g0, sigmoidf_(__uint_as_float(no[e] << 16)), rden);
        g1 = dn_of(g1, sigmoidf_(__uint_as_float(no[e] & 0xffff0000u)), rden);
      } else {
        g0 = dn_of(g0, 1.f, rden);
        g1 = dn_of(g1, 1.f, rden);
      }
      dn[e] = pack_bf16x2(g0, g1);
    }
    *reinterpret_cast<u32x4*>(&sN[buf][r * GLD + c8]) = dn;
    *reinterpret_cast<u32x4*>(&sV[buf][r * GLD + c8]) = nv;
  };

  // prologue: Q, K, D'^T, P^T rows, the first G blocks, V and dN of block 0
  // in flight together
  frag afr[2];  // dv waves: P^T rows 16 s + lr along the tokens l (k order of frag_krows)
  {
    u32x4 qr[NDT], kr[NDT];
#pragma unroll
    for (int it = 0; it < NDT; ++it) {
      const int u = tid + 512 * it, row = u / (DQK / 8), col = (u % (DQK / 8)) * 8;
      const unsigned off = ((unsigned)(t0 + row) * DQK + col) * ES;
      qr[it] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      kr[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    }
    const u32x4 dtr = __builtin_amdgcn_raw_buffer_load_b128(rdt, (unsigned)(r * BL + c8) * ES, 0, 0);
    u32x2 pr[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pr[kk][h] = __builtin_amdgcn_raw_buffer_load_b64(rpt, (unsigned)((16 * s + lr) * BL + 32 * kk + 16 * h + 4 * lg) * ES,
                                                         0, 0);
#pragma unroll
    for (int i = 0; i < PF; ++i) g_load(i, gr[i]);
    nv_load(0);
#pragma unroll
    for (int it = 0; it < NDT; ++it) {
      const int u = tid + 512 * it, row = u / (DQK / 8), col = (u % (DQK / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sQ[row * QLD + col]) = qr[it];
      *reinterpret_cast<u32x4*>(&sK[row * QLD + col]) = kr[it];
    }
    *reinterpret_cast<u32x4*>(&sDt[r * GLD + c8]) = dtr;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x4 lo4 = __builtin_bit_cast(bf16x4, pr[kk][0]);
      const bf16x4 hi4 = __builtin_bit_cast(bf16x4, pr[kk][1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        afr[kk][e] = lo4[e];
        afr[kk][4 + e] = hi4[e];
      }
    }
    g_store(0, gr[0]);
    nv_store(0);
  }
  // dk waves: acc[a][2 ms + nn] = V G^T of feature block a, rows of strip
  // 2 sp + ms, columns 16 (2 fh + nn) + lr; dv waves: acc[0] = K G and
  // acc[1] = P^T dN of the current value block
  f32x4 acc[NDT][4];
#pragma unroll
  for (int a = 0; a < NDT; ++a) zero_acc(acc[a]);
  frag vfr[2][2];  // dk waves: V rows of the two strips, current value block
  for (int b = 0; b < NVT; ++b) {
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
      const int i = b * NDT + a;
      __syncthreads();
      // (the last block's store is skipped: its buffer stages dk afterwards;
      // after the last value block nv_store writes zeros nobody reads)
      if (i + 1 < NIT) g_store((a + 1) & 1, gr[(a + 1) % PF]);
      if (a == NDT - 1) nv_store((b + 1) & 1);
      if (a == 0) nv_load(b + 1);
      g_load(i + PF, gr[a]);
      const T* gh = sGh[a & 1];
      if (dk_wave) {
        const T* gl = sGl[a & 1];
        if (a == 0) {
#pragma unroll
          for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              vfr[ms][kk] =
                  *reinterpret_cast<const frag*>(&sV[b & 1][(16 * (2 * sp + ms) + lr) * GLD + 32 * kk + 8 * lg]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            const int o = (16 * (2 * fh + nn) + lr) * GLD + 32 * kk + 8 * lg;  // G rows d, k = value column
            const frag bh_ = *reinterpret_cast<const frag*>(gh + o);
            const frag bl_ = *reinterpret_cast<const frag*>(gl + o);
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
              acc[a][2 * ms + nn] = M::mma(vfr[ms][kk], bh_, acc[a][2 * ms + nn]);
              acc[a][2 * ms + nn] = M::mma(vfr[ms][kk], bl_, acc[a][2 * ms + nn]);
            }
          }
      } else {
        if (a == 0) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int n = 0; n < 4; ++n)
              acc[1][n] = M::mma(afr[kk], frag_krows(sN[b & 1], GLD, 16 * n, 32 * kk, lg, lr), acc[1][n]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const frag ka = frag_kcols(sK, QLD, 16 * s + lr, 64 * a + 32 * kk, lg, lr);
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[0][n] = M::mma(ka, frag_krows(gh, GLD, 16 * n, 32 * kk, lg, lr), acc[0][n]);
        }
        if (a == NDT - 1) {
          // dv_j = sum_l P_lj dn~_l + w_j G_c^T k_j, value block b: staged in
          // this wave's 16 rows of sN[b & 1] (read only at a = 0, rewritten
          // one value block later), then stored as 16-byte row pieces
          T* st = sN[b & 1];
          float wj[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) wj[ii] = sw[16 * s + 4 * lg + ii];
#pragma unroll
          for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              st[(16 * s + 4 * lg + ii) * GLD + 16 * n + lr] = from_f32<T>(acc[1][n][ii] + wj[ii] * acc[0][n][ii]);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 16 * s + 8 * h + (lane >> 3), col = 8 * (lane & 7);
            const u32x4 u = *reinterpret_cast<const u32x4*>(&st[row * GLD + col]);
            __builtin_amdgcn_raw_buffer_store_b128(u, rdv, ((unsigned)(t0 + row) * DV + 64 * b + col) * ES, 0, 0);
          }
          zero_acc(acc[0]);
          zero_acc(acc[1]);
        }
      }
    }
  }
  if (dk_wave) {
    // dk_j = sum_l D'_lj q_l + w_j (G_c v_j + g_c); k_j . w_j (G_c v_j + g_c)
    // over this wave's 32 features of each feature block.  dk is staged in
    // this wave's 32 x 32 corner of sGh[0] (no longer read: the last block
    // sits in sGh[1]), then stored as 16-byte row pieces.
    T* st = sGh[0];
    float wj[2][4];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) wj[ms][ii] = sw[16 * (2 * sp + ms) + 4 * lg + ii];
    float kd[2][4] = {};  // k_j . x_j over this lane's features of every block
    frag dfr[2][2];       // D'^T rows of the two strips
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) dfr[ms][kk] = frag_kcols(sDt, GLD, 16 * (2 * sp + ms) + lr, 32 * kk, lg, lr);
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
      f32x4 t[4];
      zero_acc(t);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
          const frag qb = frag_krows(sQ, QLD, 64 * a + 16 * (2 * fh + nn), 32 * kk, lg, lr);
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) t[2 * ms + nn] = M::mma(dfr[ms][kk], qb, t[2 * ms + nn]);
        }
      float gd[2];
      T kv[2][2][4];
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int d = 64 * a + 16 * (2 * fh + nn) + lr;
        gd[nn] = sg[d];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) kv[ms][nn][ii] = sK[(16 * (2 * sp + ms) + 4 * lg + ii) * QLD + d];
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int j = 16 * (2 * sp + ms) + 4 * lg + ii;
            const float x = wj[ms][ii] * (acc[a][2 * ms + nn][ii] + gd[nn]);
            st[j * GLD + 32 * fh + 16 * nn + lr] = from_f32<T>(t[2 * ms + nn][ii] + x);
            kd[ms][ii] += to_f32(kv[ms][nn][ii]) * x;
          }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 32 * sp + 16 * h + (lane >> 2), col = 32 * fh + 8 * (lane & 3);
        const u32x4 u = *reinterpret_cast<const u32x4*>(&st[row * GLD + col]);
        __builtin_amdgcn_raw_buffer_store_b128(u, rdk, ((unsigned)(t0 + row) * DQK + 64 * a + col) * ES, 0, 0);
      }
    }
    // row sums over the 16 lanes lr (DPP rotations within rows of 16)
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        kd[ms][ii] += dpp_ror<8>(kd[ms][ii]);
        kd[ms][ii] += dpp_ror<4>(kd[ms][ii]);
        kd[ms][ii] += dpp_ror<2>(kd[ms][ii]);
        kd[ms][ii] += dpp_ror<1>(kd[ms][ii]);
        if (lr == 0) skd[fh][16 * (2 * sp + ms) + 4 * lg + ii] = kd[ms][ii];
      }
  }
  __syncthreads();
  // the rest of k . dk, one slot per token (the launcher passes 1 slot)
  if (tid < BL) p.ws_kdk[(size_t)bh * p.NC * BL + (size_t)c * BL + tid] = skd[0][tid] + skd[1][tid];
}

// ---------------------------------------------------------------- kernel 5
// d i_pre_t = k_t . dk_t; d log f_t = sum_{s >= t} (q_s . dq_s - k_s . dk_s);
// d f_pre = d log f * sigmoid(-f_pre).  Two passes over (batch*head, chunk)
// work-groups of one wave: the chunk totals of q.dq - k.dk, then each chunk's
// in-chunk suffix sums plus the totals of the chunks after it.
// slots: partials of k . dk per token that the dk kernel left in ws_kdk.
__global__ __launch_bounds__(64) void bwd_gate_total_kernel(BwdParams p, int slots) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
  const size_t tg = (size_t)bh * p.NC * BL + (size_t)c * BL + lane;
  float kdk = p.ws_kdki[tg];
  for (int d = 0; d < slots; ++d) kdk += p.ws_kdk[tg * slots + d];
  float dF = c * BL + lane < p.T ? p.ws_qdq[tg] - kdk : 0.f;
  p.ws_kdki[tg] = kdk;  // k . dk, complete
  p.ws_qdq[tg] = dF;    // q . dq - k . dk
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) dF += __shfl_xor(dF, d, 64);
  if (lane == 0) p.ws_ctot[(size_t)bh * p.NC + c] = dF;
}

template <typename T>
__global__ __launch_bounds__(64) void bwd_gate_kernel(BwdParams p, int NCT) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
  const size_t tg = (size_t)bh * p.NC * BL + (size_t)c * BL + lane;
  float carry = 0.f;
  for (int c2 = c + 1 + lane; c2 < p.NC; c2 += 64) carry += p.ws_ctot[(size_t)bh * p.NC + c2];
  // <dC_T, S~_T> + <dn_T, n~_T> from the walk's tile partials
  if (p.ws_cT)
    for (int i = lane; i < NCT; i += 64) carry += p.ws_cT[(size_t)bh * NCT + i];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) carry += __shfl_xor(carry, d, 64);
  // suffix sum within the chunk: lane 63 - l takes token l
  const int l = 63 - lane;
  const size_t tl = (size_t)bh * p.NC * BL + (size_t)c * BL + l;
  float s = p.ws_qdq[tl];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(s, d, 64);
    if (lane >= d) s += y;
  }
  const int t = c * BL + l;
  if (t < p.T) {
    const size_t o = (size_t)bh * p.T + t;
    const float f = to_f32(static_cast<const T*>(p.f_pre)[o]);
    static_cast<T*>(p.di)[o] = from_f32<T>(p.ws_kdki[tl]);
    static_cast<T*>(p.df)[o] = from_f32<T>((carry + s) * sigmoidf_(-f));
  }
  (void)tg;
}

// d bias_h = sum over the batch and the chunks of the bias partials: one
// work-group per head, a strided sum per thread, then a tree over the group.
__global__ __launch_bounds__(256) void bwd_bias_kernel(BwdParams p) {
  __shared__ float sred[4];
  const int hd = blockIdx.x, tid = threadIdx.x;
  float a = 0.f;
  const int n = p.B * p.NC;
  for (int e = tid; e < n; e += 256) {
    const int b = e / p.NC, c = e % p.NC;
    a += p.ws_dbias[((size_t)b * p.H + hd) * p.NC + c];
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) a += __shfl_xor(a, d, 64);
  if ((tid & 63) == 0) sred[tid >> 6] = a;
  __syncthreads();
  if (tid == 0) p.dbias[hd] = sred[0] + sred[1] + sred[2] + sred[3];
}

template <typename T, int DQK, int NB = 1>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const unsigned BH = (unsigned)(p.B * p.H);
  const unsigned nch = BH * (unsigned)p.NC;
  hipLaunchKernelGGL((bwd_chunk_states_kernel<T, DQK, NB>), dim3(BH * p.NS * (DQK / 64) * (p.DV / 64)), dim3(256), 0,
                     stream, p);
  if (p.ret)
    hipLaunchKernelGGL((bwd_scores_kernel<T, DQK, true, NB>), dim3(nch), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_scores_kernel<T, DQK, false, NB>), dim3(nch), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((bwd_dq_kernel<T, DQK, NB>), dim3(nch * (DQK / 64)), dim3(256), 0, stream, p);
  const size_t NST = (size_t)DQK * p.DV + DQK;
  // long sequences of small states leave few work-groups for a long chain:
  // keep more chunks' loads in flight per step of it
  const unsigned ge = (unsigned)((NST / 4 + 255) / 256);
  // the 7B head shape has its own dk/dv kernel, which reads finished states
  constexpr bool CHUNK_DKV = sizeof(T) == 2 && NB == 1 && DQK == 256;
  const bool two_level = p.ws_carry && p.NSEG > 1;
  if (two_level) {  // two-level scan (long sequences)
    const dim3 g3(ge, BH, (unsigned)p.NSEG);
    hipLaunchKernelGGL(bwd_scan_local_kernel, g3, dim3(256), 0, stream, p, DQK);
    hipLaunchKernelGGL(bwd_scan_carry_kernel, dim3(ge, BH), dim3(256), 0, stream, p, DQK);
    // the generic dk/dv kernel adds the decayed carries as it loads the
    // states (no apply pass over them)
    if (CHUNK_DKV) hipLaunchKernelGGL(bwd_scan_apply_kernel, g3, dim3(256), 0, stream, p, DQK);
  } else {
    hipLaunchKernelGGL(bwd_scan_kernel<8>, dim3(ge, BH), dim3(256), 0, stream, p, DQK);
  }
  // slots per token of the k . dk partials the dk kernel leaves
  int kdk_slots = DQK / 64;
  if constexpr (sizeof(T) == 2 && NB == 1 && DQK == 256) {
    hipLaunchKernelGGL((bwd_dkv_chunk_kernel<DQK / 64>), dim3(nch), dim3(512), 0, stream, p);
    kdk_slots = 1;
  } else {
    const dim3 gk(nch * (DQK / 64 + p.DV / 64));
    if (two_level)
      hipLaunchKernelGGL((bwd_dkv_kernel<T, DQK, NB, true>), gk, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dkv_kernel<T, DQK, NB, false>), gk, dim3(256), 0, stream, p);
  }
  if (!p.ret) {  // retention has no gates or normaliser to differentiate
    hipLaunchKernelGGL(bwd_gate_total_kernel, dim3(nch), dim3(64), 0, stream, p, kdk_slots);
    hipLaunchKernelGGL((bwd_gate_kernel<T>), dim3(nch), dim3(64), 0, stream, p, (DQK / 64) * (p.DV / 64));
    if (p.dbias) hipLaunchKernelGGL(bwd_bias_kernel, dim3((unsigned)p.H), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

bool bwd_supported(int dtype, int dqk, int dv, int nb) {
  if (dv % 64) return false;
  if (nb == 2) return dqk == 64 && dv == 64;  // two 32-wide blocks of a 64-wide head
  if (nb != 1) return false;
  if (dtype == 1) return dqk == 64 || dqk == 128 || dqk == 256;
  return dqk == 64;
}

hipError_t launch_bwd(int dtype, const BwdParams& p, hipStream_t stream) {
  if (p.NB == 2) {
    if (p.DQK != 64 || p.DV != 64 || p.ret) return hipErrorInvalidValue;
    return dtype == 1 ? launch_bwd_t<__bf16, 64, 2>(p, stream) : launch_bwd_t<float, 64, 2>(p, stream);
  }
  if (dtype == 1) {
    if (p.DQK == 64) return launch_bwd_t<__bf16, 64>(p, stream);
    if (p.DQK == 128) return launch_bwd_t<__bf16, 128>(p, stream);
    if (p.DQK == 256) return launch_bwd_t<__bf16, 256>(p, stream);
  } else if (p.DQK == 64) {
    return launch_bwd_t<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mlstm
