// Fused single-token mLSTM decode step for gfx950 (HBM-bound).
//
// One step of the recurrence on every (batch, head), state updated in place
// (the carried, in-place state of the "FusedRecurrent" mode doc of burn-gdn2's
// Gdn2Mode; matrix memory update of the "mLSTM Model" page, "Core idea";
// block-diagonal memory and biased normaliser of the
// "Edifice.Recurrent.XLSTMv2" page, "Key Improvements" items 1-2):
//   m'  = max(log f + m, log i);  f' = 2^{log2 f + m - m'};  i' = 2^{log2 i - m'}
//   S~ <- f' S~ + i' k v^T        (per memory block)
//   n~ <- f' n~ + i' k
//   h   = o * (S~^T q) / max(|n~.q + bias 2^{-m'}|, 2^{-m'})
// The readout uses the updated state.
//
// Retention decode (recurrent form of the "Edifice.Attention.RetNet" page,
// "Key Innovation: Retention Mechanism", one step of its recurrent mode in
// "Triple Paradigm"): the same kernel with f' = gamma_h, i' = 1 and no
// normaliser, output gate or stabiliser:  S <- gamma_h S + k v^T, o = S^T q.
//
// Two launches.  step_kernel streams the matrix state: work-group (b*h,
// slice) owns a slice of WS columns and all rows, so its readout columns are
// complete and it writes h for them.  The updated normaliser enters only
// through n~'.q = f' (n~.q) + i' (k.q), computed from the old n~, so no
// work-group depends on another's writes; step_norm_kernel then updates n~
// and m in place.  Thread (g, t) of a slice owns columns 4t..4t+3 and rows
// g, g+RG, ... of their memory block: every state element is read and written
// once with 16-byte accesses, consecutive threads touch consecutive 16-byte
// words of a row, and short work-groups keep the HBM streams of the whole
// chip busy.  The RG partial sums of a column meet in LDS.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace mlstm {

// gate factors of one (batch, head) in log2 units
struct StepGates {
  float mn2, fdec, iw;
};
template <typename T, bool RET = false>
__device__ __forceinline__ StepGates step_gates(const StepParams& p, int bh) {
  if constexpr (RET) {
    const int hd = bh % p.H;
    StepGates s;
    s.mn2 = 0.f;
    s.fdec = p.gamma ? p.gamma[hd] : 1.f - exp2f(-5.f - (float)hd);
    s.iw = 1.f;
    return s;
  }
  const float lf2 = log2_sigmoid(to_f32(static_cast<const T*>(p.f_pre)[bh]));
  const float li2 = to_f32(static_cast<const T*>(p.i_pre)[bh]) * kLog2e;
  const float m2 = p.m[bh] * kLog2e;
  StepGates s;
  s.mn2 = fmaxf(lf2 + m2, li2);
  s.fdec = exp2_fast(lf2 + m2 - s.mn2);
  s.iw = exp2_fast(li2 - s.mn2);
  return s;
}

// SN: the scalar normaliser n~ = f' n~ + i' (n [B,H]), denominator
// |n~ + bias 2^{-m'}| (no k, no q).  PB: one denominator per memory block
// (at most kStepMaxBlocks blocks).
constexpr int kStepMaxBlocks = 8;
template <typename T, int RG, bool RET, bool SN = false, bool PB = false>
__global__ __launch_bounds__(512) void step_kernel(StepParams p, int WS) {
  extern __shared__ float smem[];
  const int DQK = p.DQK, DV = p.DV, NB = p.NB;
  const int DQKB = DQK / NB, DVB = DV / NB;
  const int TPC = WS / 4;  // column threads
  const int nth = TPC * RG;
  const int nsl = DV / WS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = tid / TPC, t = tid - g * TPC;
  const int bh = blockIdx.x / nsl, slice = blockIdx.x - bh * nsl;
  float* sq = smem;              // [DQK]
  float* sk = sq + DQK;          // [DQK]
  float* sacc = sk + DQK;        // [RG][WS]
  float* sred = sacc + RG * WS;  // [2][nth / 64], per block with PB
  constexpr int NBA = PB ? kStepMaxBlocks : 1;

  const T* q = static_cast<const T*>(p.q) + (size_t)bh * DQK;
  const T* k = static_cast<const T*>(p.k) + (size_t)bh * DQK;
  const T* v = static_cast<const T*>(p.v) + (size_t)bh * DV;

  const int col = slice * WS + t * 4;
  const int blk = col / DVB, cl = col - blk * DVB;
  float* S = p.C + (size_t)bh * DQK * DVB + (size_t)blk * DQKB * DVB + cl;
  constexpr int U = 16;  // rows in flight per thread (16 x 16 B loads)
  f32x4 s[U];
  // the first batch of state rows goes out before anything else
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = g + u * RG;
    if (r < DQKB) s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)r * DVB));
  }
  const StepGates gt = step_gates<T, RET>(p, bh);
  const float bias = (!RET && p.bias) ? p.bias[bh % p.H] : 0.f;
  // q, k to LDS; n~.q and k.q over the head
  float nqa[NBA], kqa[NBA];  // per block with PB (registers: fixed indices only)
#pragma unroll
  for (int bb = 0; bb < NBA; ++bb) nqa[bb] = kqa[bb] = 0.f;
  for (int r = tid; r < DQK; r += nth) {
    const float qr = to_f32(q[r]), kr = to_f32(k[r]);
    sq[r] = qr;
    sk[r] = kr;
    if constexpr (!RET && !SN) {
      const float nx = p.n[(size_t)bh * DQK + r] * qr, kx = kr * qr;
      const int rb = PB ? r / DQKB : 0;
#pragma unroll
      for (int bb = 0; bb < NBA; ++bb)
        if (bb == rb) {
          nqa[bb] += nx;
          kqa[bb] += kx;
        }
    }
  }
  if constexpr (!RET && !SN) {
    const int nw = nth / 64;
#pragma unroll
    for (int bb = 0; bb < NBA; ++bb) {
      if (bb < (PB ? NB : 1)) {
        float nq = nqa[bb], kq = kqa[bb];
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) {
          nq += __shfl_xor(nq, d, 64);
          kq += __shfl_xor(kq, d, 64);
        }
        if (lane == 0) {
          sred[2 * bb * nw + (tid >> 6)] = nq;
          sred[(2 * bb + 1) * nw + (tid >> 6)] = kq;
        }
      }
    }
  }
  __syncthreads();

  float vv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vv[i] = gt.iw * to_f32(v[col + i]);
  const float* kb = sk + blk * DQKB;
  const float* qb = sq + blk * DQKB;
  const float fdec = gt.fdec;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = g; r0 < DQKB; r0 += U * RG) {
    if (r0 != g) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RG;
        if (r < DQKB) s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)r * DVB));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RG;
      if (r < DQKB) {
        const float kr = kb[r], qr = qb[r];
        s[u].x = fdec * s[u].x + kr * vv[0];
        s[u].y = fdec * s[u].y + kr * vv[1];
        s[u].z = fdec * s[u].z + kr * vv[2];
        s[u].w = fdec * s[u].w + kr * vv[3];
        acc[0] += s[u].x * qr;
        acc[1] += s[u].y * qr;
        acc[2] += s[u].z * qr;
        acc[3] += s[u].w * qr;
        __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4*>(S + (size_t)r * DVB));
      }
    }
  }
  if constexpr (RG > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sacc[g * WS + t * 4 + i] = acc[i];
  }
  __syncthreads();
  if (g == 0) {
    if constexpr (RG > 1) {
      for (int gg = 1; gg < RG; ++gg)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += sacc[gg * WS + t * 4 + i];
    }
    if constexpr (RET) {
      store4(static_cast<T*>(p.h) + (size_t)bh * DV + col, from_f32<T>(acc[0]), from_f32<T>(acc[1]),
             from_f32<T>(acc[2]), from_f32<T>(acc[3]));
      return;
    }
    float n_q = 0.f, k_q = 0.f;
    if constexpr (SN) {
      n_q = p.n[bh];  // the old scalar n~; its new value is f' n~ + i'
      k_q = 1.f;
    } else {
      const int nw = nth / 64, db = PB ? blk : 0;  // this thread's columns lie in block blk
      for (int i = 0; i < nw; ++i) {
        n_q += sred[2 * db * nw + i];
        k_q += sred[(2 * db + 1) * nw + i];
      }
    }
    const float cl2 = exp2_fast(-gt.mn2);
    const float den = fdec * n_q + gt.iw * k_q + bias * cl2;  // n~' . q + bias 2^{-m'}
    const float inv = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), cl2));
    const T* op = static_cast<const T*>(p.o_pre);
    T hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = op ? sigmoidf_(to_f32(op[(size_t)bh * DV + col + i])) : 1.f;
      hv[i] = from_f32<T>(o * acc[i] * inv);
    }
    store4(static_cast<T*>(p.h) + (size_t)bh * DV + col, hv[0], hv[1], hv[2], hv[3]);
  }
}

// n~ <- f' n~ + i' k and m <- m' in place, after step_kernel has read them.
// A work-group owns RPB = max(1, 256 / d_qk) whole rows (b, h), so every
// reader of a row's m is in the work-group that rewrites it, after a barrier;
// all loads of a thread are issued before any result is needed.
template <typename T, bool SN = false>
__global__ __launch_bounds__(256) void step_norm_kernel(StepParams p, int RPB) {
  const int DQK = SN ? 1 : p.DQK, BH = p.B * p.H;  // normaliser entries per row
  const int bh0 = blockIdx.x * RPB;
  const int nrow = min(RPB, BH - bh0);
  for (int e = threadIdx.x; e < nrow * DQK; e += 256) {
    const int bh = bh0 + e / DQK;
    const size_t idx = (size_t)bh0 * DQK + e;
    const float nv = p.n[idx];
    const float kv = SN ? 1.f : to_f32(static_cast<const T*>(p.k)[idx]);
    const StepGates gt = step_gates<T>(p, bh);
    p.n[idx] = gt.fdec * nv + gt.iw * kv;
  }
  __syncthreads();  // every read of m in this work-group is done
  if (threadIdx.x < nrow) {
    const StepGates gt = step_gates<T>(p, bh0 + threadIdx.x);
    p.m[bh0 + threadIdx.x] = gt.mn2 * kLn2;
  }
}

// Slice width: the largest of 128, 64, 32, 16 columns that divides d_v.
static int pick_ws(int dv) {
  for (int ws : {128, 64, 32, 16})
    if (dv % ws == 0) return ws;
  return 0;
}
// Row groups: the most (up to 16) that keep the work-group at <= 512
// threads with a whole number of waves (the dot products reduce per wave).
// MLSTM_STEP_RG (1 .. 16, a power of two) overrides the choice for tuning
// when it fits.
static int pick_rg(int ws) {
  const int tpc = ws / 4;
  const auto fits = [tpc](int rg, int cap) { return tpc * rg <= cap && (tpc * rg) % 64 == 0; };
  const char* e = getenv("MLSTM_STEP_RG");
  if (e) {
    const int x = atoi(e);
    if ((x == 1 || x == 2 || x == 4 || x == 8 || x == 16) && fits(x, 512)) return x;
  }
  for (int rg = 16; rg >= 1; rg >>= 1)
    if (fits(rg, 512)) return rg;
  return 0;
}

bool step_supported(int dqk, int dv, int nb) {
  if (nb <= 0 || dqk % nb || dv % nb) return false;
  if ((dv / nb) % 4 || pick_ws(dv) == 0) return false;
  return pick_rg(pick_ws(dv)) > 0;
}

template <typename T, bool RET, bool SN = false, bool PB = false>
static hipError_t launch_rg(const StepParams& p, int ws, int rg, hipStream_t stream) {
  const int tpc = ws / 4;
  const dim3 grid((unsigned)(p.B * p.H * (p.DV / ws)));
  const dim3 block((unsigned)(tpc * rg));
  const size_t smem = ((size_t)2 * p.DQK + (size_t)rg * ws + 2 * 16 * (PB ? kStepMaxBlocks : 1)) * sizeof(float);
  switch (rg) {
    case 1: hipLaunchKernelGGL((step_kernel<T, 1, RET, SN, PB>), grid, block, smem, stream, p, ws); break;
    case 2: hipLaunchKernelGGL((step_kernel<T, 2, RET, SN, PB>), grid, block, smem, stream, p, ws); break;
    case 4: hipLaunchKernelGGL((step_kernel<T, 4, RET, SN, PB>), grid, block, smem, stream, p, ws); break;
    case 8: hipLaunchKernelGGL((step_kernel<T, 8, RET, SN, PB>), grid, block, smem, stream, p, ws); break;
    default: hipLaunchKernelGGL((step_kernel<T, 16, RET, SN, PB>), grid, block, smem, stream, p, ws); break;
  }
  if constexpr (RET) return hipGetLastError();  // no normaliser or stabiliser
  const int nent = SN ? 1 : p.DQK;  // normaliser entries per (b, h)
  const int rpb = nent >= 256 ? 1 : 256 / nent;
  const int nwg = (p.B * p.H + rpb - 1) / rpb;
  hipLaunchKernelGGL((step_norm_kernel<T, SN>), dim3((unsigned)nwg), dim3(256), 0, stream, p, rpb);
  return hipGetLastError();
}

hipError_t launch_step(int dtype, const StepParams& p, hipStream_t stream, int norm_mode) {
  const int ws = pick_ws(p.DV);
  const int rg = pick_rg(ws);
  if (norm_mode == 1)
    return dtype == 1 ? launch_rg<__bf16, false, true>(p, ws, rg, stream)
                      : launch_rg<float, false, true>(p, ws, rg, stream);
  if (norm_mode == 2 && p.NB > 1)
    return dtype == 1 ? launch_rg<__bf16, false, false, true>(p, ws, rg, stream)
                      : launch_rg<float, false, false, true>(p, ws, rg, stream);
  return dtype == 1 ? launch_rg<__bf16, false>(p, ws, rg, stream) : launch_rg<float, false>(p, ws, rg, stream);
}

hipError_t launch_retention_step(int dtype, const StepParams& p, hipStream_t stream) {
  const int ws = pick_ws(p.DV);
  const int rg = pick_rg(ws);
  return dtype == 1 ? launch_rg<__bf16, true>(p, ws, rg, stream) : launch_rg<float, true>(p, ws, rg, stream);
}

}  // namespace mlstm
