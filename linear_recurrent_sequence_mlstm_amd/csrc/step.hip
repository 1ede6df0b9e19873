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
// Thread layout: one work-group per (batch, head).  Its threads form
// RG row groups x (d_v / 4) column threads; thread (g, t) owns columns
// 4t..4t+3 and rows g, g+RG, ... of its memory block, so every state element
// is read and written exactly once with 16-byte accesses, and consecutive
// threads touch consecutive 16-byte words of a row.  The RG partial readout
// sums of a column meet in LDS.  Many short work-groups keep the HBM
// streams of the whole chip in flight.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace mlstm {

template <typename T, int RG>
__global__ __launch_bounds__(1024) void step_kernel(StepParams p) {
  extern __shared__ float smem[];
  const int DQK = p.DQK, DV = p.DV, NB = p.NB;
  const int DQKB = DQK / NB, DVB = DV / NB;
  const int TPC = DV / 4;  // column threads
  const int nth = TPC * RG;
  const int tid = threadIdx.x;
  const int g = tid / TPC, t = tid - g * TPC;
  const int bh = blockIdx.x;
  float* sq = smem;              // [DQK]
  float* sk = sq + DQK;          // [DQK]
  float* sacc = sk + DQK;        // [RG][DV]
  float* sred = sacc + RG * DV;  // [nth / 64]

  const T* q = static_cast<const T*>(p.q);
  const T* k = static_cast<const T*>(p.k);
  const T* v = static_cast<const T*>(p.v);
  const T* ip = static_cast<const T*>(p.i_pre);
  const T* fp = static_cast<const T*>(p.f_pre);
  const T* op = static_cast<const T*>(p.o_pre);
  T* h = static_cast<T*>(p.h);

  const float lf2 = log2_sigmoid(to_f32(fp[bh]));
  const float li2 = to_f32(ip[bh]) * kLog2e;
  const float m2 = p.m[bh] * kLog2e;
  const float mn2 = fmaxf(lf2 + m2, li2);
  const float fdec = exp2_fast(lf2 + m2 - mn2);
  const float iw = exp2_fast(li2 - mn2);
  const float bias = p.bias ? p.bias[bh % p.H] : 0.f;
  for (int r = tid; r < DQK; r += nth) {
    sq[r] = to_f32(q[(size_t)bh * DQK + r]);
    sk[r] = to_f32(k[(size_t)bh * DQK + r]);
  }
  __syncthreads();

  const int col = t * 4;
  const int blk = col / DVB, cl = col - blk * DVB;
  float vv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vv[i] = iw * to_f32(v[(size_t)bh * DV + col + i]);
  float* S = p.C + (size_t)bh * DQK * DVB + (size_t)blk * DQKB * DVB + cl;
  const float* kb = sk + blk * DQKB;
  const float* qb = sq + blk * DQKB;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 16;  // rows in flight per thread (16 x 16 B loads)
  for (int r0 = g; r0 < DQKB; r0 += U * RG) {
    f32x4 s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RG;
      if (r < DQKB) s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)r * DVB));
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
  // n~ update and n~.q over the whole work-group
  float dot = 0.f;
  for (int r = tid; r < DQK; r += nth) {
    float* np = p.n + (size_t)bh * DQK + r;
    const float nn = fdec * *np + iw * sk[r];
    *np = nn;
    dot += nn * sq[r];
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) dot += __shfl_xor(dot, d, 64);
  if ((tid & 63) == 0) sred[tid >> 6] = dot;
  if constexpr (RG > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sacc[g * DV + col + i] = acc[i];
  }
  __syncthreads();
  if (g == 0) {
    dot = 0.f;
    for (int i = 0; i < nth / 64; ++i) dot += sred[i];
    if constexpr (RG > 1) {
      for (int gg = 1; gg < RG; ++gg)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += sacc[gg * DV + col + i];
    }
    const float cl2 = exp2_fast(-mn2);
    const float inv = __builtin_amdgcn_rcpf(fmaxf(fabsf(dot + bias * cl2), cl2));
    T hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = op ? sigmoidf_(to_f32(op[(size_t)bh * DV + col + i])) : 1.f;
      hv[i] = from_f32<T>(o * acc[i] * inv);
    }
    store4(h + (size_t)bh * DV + col, hv[0], hv[1], hv[2], hv[3]);
    if (t == 0) p.m[bh] = mn2 * kLn2;
  }
}

// Row groups per (batch, head): the most (up to 8) that keep the work-group
// at <= 512 threads, else at <= 1024, with a whole number of waves (the n~.q
// sum reduces per wave).  0 if no choice fits.  MLSTM_STEP_RG (1, 2, 4, 8)
// overrides the choice for tuning when it fits.
static int pick_rg(int dv) {
  const int tpc = dv / 4;
  const auto fits = [tpc](int rg, int cap) { return tpc * rg <= cap && (tpc * rg) % 64 == 0; };
  const char* e = getenv("MLSTM_STEP_RG");
  if (e) {
    const int x = atoi(e);
    if ((x == 1 || x == 2 || x == 4 || x == 8) && fits(x, 1024)) return x;
  }
  for (int cap : {512, 1024})
    for (int rg = 8; rg >= 1; rg >>= 1)
      if (fits(rg, cap)) return rg;
  return 0;
}

bool step_supported(int dqk, int dv, int nb) {
  if (nb <= 0 || dqk % nb || dv % nb) return false;
  if (dv % 4 || (dv / nb) % 4) return false;
  return pick_rg(dv) > 0;
}

template <typename T>
static hipError_t launch_rg(const StepParams& p, int rg, hipStream_t stream) {
  const int tpc = p.DV / 4;
  const dim3 grid((unsigned)(p.B * p.H));
  const dim3 block((unsigned)(tpc * rg));
  const size_t smem = ((size_t)2 * p.DQK + (size_t)rg * p.DV + 16) * sizeof(float);
  switch (rg) {
    case 1: hipLaunchKernelGGL((step_kernel<T, 1>), grid, block, smem, stream, p); break;
    case 2: hipLaunchKernelGGL((step_kernel<T, 2>), grid, block, smem, stream, p); break;
    case 4: hipLaunchKernelGGL((step_kernel<T, 4>), grid, block, smem, stream, p); break;
    default: hipLaunchKernelGGL((step_kernel<T, 8>), grid, block, smem, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_step(int dtype, const StepParams& p, hipStream_t stream) {
  const int rg = pick_rg(p.DV);
  return dtype == 1 ? launch_rg<__bf16>(p, rg, stream) : launch_rg<float>(p, rg, stream);
}

}  // namespace mlstm
