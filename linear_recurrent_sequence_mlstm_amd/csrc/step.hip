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
// Thread layout: a (batch, head) is served by DV/4 threads; thread t owns
// columns 4t..4t+3 of d_v for every row of its memory block, so it reads and
// writes each state element exactly once with 16-byte accesses, and consecutive
// threads touch consecutive 16-byte words of a row.  The d_qk-long readout
// sum stays in the thread; only the scalar n~.q needs a reduction.
#include "common.h"
#include "kernels.h"

namespace mlstm {

template <typename T>
__global__ __launch_bounds__(256) void step_kernel(StepParams p, int tph, int ppw) {
  extern __shared__ float smem[];
  const int DQK = p.DQK, DV = p.DV, NB = p.NB;
  const int DQKB = DQK / NB, DVB = DV / NB;
  const int sub = threadIdx.x / tph, lt = threadIdx.x - sub * tph;
  const int bh = blockIdx.x * ppw + sub;
  const bool active = sub < ppw && bh < p.B * p.H;
  float* sq = smem + (size_t)sub * 2 * DQK;
  float* sk = sq + DQK;
  float* sred = smem + (size_t)ppw * 2 * DQK;  // [ppw][4]

  const T* q = static_cast<const T*>(p.q);
  const T* k = static_cast<const T*>(p.k);
  const T* v = static_cast<const T*>(p.v);
  const T* ip = static_cast<const T*>(p.i_pre);
  const T* fp = static_cast<const T*>(p.f_pre);
  const T* op = static_cast<const T*>(p.o_pre);
  T* h = static_cast<T*>(p.h);

  float m2 = 0.f, mn2 = 0.f, fdec = 0.f, iw = 0.f, bias = 0.f;
  if (active) {
    const float lf2 = log2_sigmoid(to_f32(fp[bh]));
    const float li2 = to_f32(ip[bh]) * kLog2e;
    m2 = p.m[bh] * kLog2e;
    mn2 = fmaxf(lf2 + m2, li2);
    fdec = exp2_fast(lf2 + m2 - mn2);
    iw = exp2_fast(li2 - mn2);
    bias = p.bias ? p.bias[bh % p.H] : 0.f;
    for (int r = lt; r < DQK; r += tph) {
      sq[r] = to_f32(q[(size_t)bh * DQK + r]);
      sk[r] = to_f32(k[(size_t)bh * DQK + r]);
    }
  }
  __syncthreads();

  float dot = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int col = lt * 4;
  const int blk = col / DVB, cl = col - blk * DVB;
  if (active) {
    float vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = iw * to_f32(v[(size_t)bh * DV + col + i]);
    float* S = p.C + (size_t)bh * DQK * DVB + (size_t)blk * DQKB * DVB + cl;
    const float* kb = sk + blk * DQKB;
    const float* qb = sq + blk * DQKB;
    for (int r0 = 0; r0 < DQKB; r0 += 8) {
      f32x4 s[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(r0 + u) * DVB));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float kr = kb[r0 + u], qr = qb[r0 + u];
        s[u].x = fdec * s[u].x + kr * vv[0];
        s[u].y = fdec * s[u].y + kr * vv[1];
        s[u].z = fdec * s[u].z + kr * vv[2];
        s[u].w = fdec * s[u].w + kr * vv[3];
        acc[0] += s[u].x * qr;
        acc[1] += s[u].y * qr;
        acc[2] += s[u].z * qr;
        acc[3] += s[u].w * qr;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4*>(S + (size_t)(r0 + u) * DVB));
    }
    for (int r = lt; r < DQK; r += tph) {
      float* np = p.n + (size_t)bh * DQK + r;
      const float nn = fdec * *np + iw * sk[r];
      *np = nn;
      dot += nn * sq[r];
    }
  }
  // reduce n~.q over the tph threads of this (batch, head)
  const int width = tph < 64 ? tph : 64;
  for (int d = width >> 1; d > 0; d >>= 1) dot += __shfl_xor(dot, d, width);
  if (tph > 64) {
    if (active && (lt & 63) == 0) sred[sub * 4 + (lt >> 6)] = dot;
    __syncthreads();
    if (active) {
      dot = 0.f;
      for (int i = 0; i < tph / 64; ++i) dot += sred[sub * 4 + i];
    }
  }
  if (active) {
    const float cl2 = exp2_fast(-mn2);
    const float inv = __builtin_amdgcn_rcpf(fmaxf(fabsf(dot + bias * cl2), cl2));
    T hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = op ? sigmoidf_(to_f32(op[(size_t)bh * DV + col + i])) : 1.f;
      hv[i] = from_f32<T>(o * acc[i] * inv);
    }
    store4(h + (size_t)bh * DV + col, hv[0], hv[1], hv[2], hv[3]);
    if (lt == 0) p.m[bh] = mn2 * kLn2;
  }
}

bool step_supported(int dqk, int dv, int nb) {
  if (nb <= 0 || dqk % nb || dv % nb) return false;
  if (dv % 4 || (dv / nb) % 4) return false;
  if ((dqk / nb) % 8) return false;
  const int tph = dv / 4;
  if (tph > 256 || 256 % tph) return false;
  if (tph > 64 && tph / 64 > 4) return false;
  return true;
}

hipError_t launch_step(int dtype, const StepParams& p, hipStream_t stream) {
  const int tph = p.DV / 4;
  const int ppw = 256 / tph;
  const int BH = p.B * p.H;
  const dim3 grid((unsigned)((BH + ppw - 1) / ppw));
  const size_t smem = ((size_t)ppw * 2 * p.DQK + (size_t)ppw * 4) * sizeof(float);
  if (dtype == 1)
    hipLaunchKernelGGL(step_kernel<__bf16>, grid, dim3(256), smem, stream, p, tph, ppw);
  else
    hipLaunchKernelGGL(step_kernel<float>, grid, dim3(256), smem, stream, p, tph, ppw);
  return hipGetLastError();
}

}  // namespace mlstm
