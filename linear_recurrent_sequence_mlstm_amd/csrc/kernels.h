// Host-side view of the kernels: launch parameter blocks and variant lookup.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace mlstm {

// Chunkwise forward (mLSTM or retention).  All pointers are device pointers.
struct ChunkParams {
  int B, H, T, DV;
  int NC, G, NS, nslices;  // chunks, chunks per superchunk, superchunks, d_v slices
  const void* q;
  const void* k;
  const void* v;
  const void* i_pre;
  const void* f_pre;
  const void* o_pre;
  const float* bias;       // [H] or null
  const float* ret_gamma;  // retention: [H] gamma_h, or null for 1 - 2^(-5-h)
  float* ws_state;         // [B*H][NS][CS (+ d_qk)] superchunk start states
  float* ws_scal;          // [B*H][NS][2] (total log2 decay, local log2 scale)
  float* ws_min;           // [B*H][NS] stabiliser (log2) at superchunk starts
  float* ws_ga;            // [B*H][NC*L] chunk-local log2 gate sums a_j, prefix maxima g_j,
  float* ws_gg;            //   forget-gate sums b_j (gate pass -> pass 3)
  float* ws_gb;
  int has_init;
  // one-superchunk plan run as pass 3 alone: it takes its start state from
  // C0 / n0 / m0 (null: zero) and forms the chunk-local gate logs from i_pre,
  // f_pre itself, so the gate pass and pass 2 are not launched
  int direct;
  // few superchunks of a small state: pass 3 composes its start state from
  // pass 1's local states itself (pass 2's arithmetic), so pass 2 is not
  // launched
  int fuse_scan;
  // superchunk state slots in the register order of the 7B-shape pass 3
  // (set by the launcher; the slots' d_qk entries of n~ stay in order)
  int perm_state;
  const float* C0;
  const float* n0;
  const float* m0;
  void* h;
  float* C_out;
  float* n_out;
  float* m_out;
  // fused group norm of retention outputs: [H*d_v] weight and bias (null:
  // 1 and 0) and epsilon
  const float* gn_w;
  const float* gn_b;
  float gn_eps;
  // group norm of a head whose d_v spans several work-groups: pass 3 writes
  // the unnormalised outputs here in fp32 ([B*H*T][d_v]) and a row pass
  // normalises them into h (null: the work-group holds the whole row)
  float* gn_ws;
};

struct ScanParams {
  int NS;
  size_t CS;
  int DQK;
  float* ws_state;
  float* ws_scal;
  float* ws_min;
  int has_init;
  const float* C0;
  const float* n0;
  const float* m0;
  int scalar_n;  // n0 is [B,H] (scalar normaliser)
  int perm;      // the slots use the 7B-shape pass 3 register order (C0 is gathered into it)
};

// ev0/ev1 (may be null) are recorded right before / after the main kernel.
typedef hipError_t (*ChunkLaunchFn)(ChunkParams, hipStream_t, hipEvent_t ev0, hipEvent_t ev1);

struct ChunkVariant {
  ChunkLaunchFn launch;
  ChunkLaunchFn launch_scalar_norm;  // mLSTM with the scalar normaliser (null: none)
  ChunkLaunchFn launch_block_norm;   // mLSTM, one denominator per memory block (null: none)
  size_t lds_bytes;
  int wc;  // d_v columns per wave
  int w;   // d_v columns per work-group (the d_v slice)
};

// dtype: 0 = fp32, 1 = bf16.
bool find_chunk_variant(int dtype, int dqk, int nb, int L, bool ret, ChunkVariant* out);
// Retention with the group norm of each head's output fused (d_v = out->w).
bool find_retention_groupnorm_variant(int dtype, int dqk, int L, ChunkVariant* out);

// Decode step.
struct StepParams {
  int B, H, DQK, DV, NB;
  const void* q;
  const void* k;
  const void* v;
  const void* i_pre;
  const void* f_pre;
  const void* o_pre;
  const float* bias;
  float* C;
  float* n;
  float* m;
  void* h;
  const float* gamma;  // retention: [H] decay, or null for 1 - 2^(-5-h)
};

// norm_mode: 0 vector, 1 scalar (n is [B,H], denominator |n~ + bias 2^{-m}|),
// 2 one denominator per memory block
hipError_t launch_step(int dtype, const StepParams& p, hipStream_t stream, int norm_mode = 0);
// Retention decode: C is S [B,H,d_k,d_v]; q, k, v, h and gamma are read.
hipError_t launch_retention_step(int dtype, const StepParams& p, hipStream_t stream);
bool step_supported(int dqk, int dv, int nb);

// Chunkwise backward (mLSTM, vector normaliser, one memory block, chunks of
// 64 tokens), after the forward plan's state passes ran.
struct BwdParams {
  int B, H, T, DQK, DV, NC, G, NS;
  int NB;         // memory blocks (1, or 2 on 64-wide heads)
  int ret;        // retention: no gates, no normaliser
  size_t sc_nst;  // floats per superchunk state slot of the forward plan
  const void* q;
  const void* k;
  const void* v;
  const void* f_pre;
  const void* o_pre;
  const float* bias;
  const void* dh;
  int has_init;
  const float* sc_state;  // [B*H][NS][d_qk d_v + d_qk] superchunk start states (forward pass 2)
  const float* sc_min;    // [B*H][NS] stabiliser (log2) at superchunk starts
  float* ws_state;        // [B*H][NC][d_qk d_v + d_qk] chunk start states
  float* ws_min;          // [B*H][NC] stabiliser (log2) at chunk starts
  const float* ws_ga;     // [B*H][NC*64] a_j, prefix maxima g_j, b_j (log2)
  const float* ws_gg;
  const float* ws_gb;
  void* wsPt;  // [B*H][NC][NB][64][64] (E.(Q_b K_b^T))^T
  void* wsDt;  // [B*H][NC][NB][64][64] D'_b^T
  float* ws_rden;     // [B*H][NC*64] 1 / den~
  float* ws_dz;       // [B*H][NC*64] dz~
  float* ws_dbias;    // [B*H][NC] bias partials of the chunks
  float* ws_ctot;     // [B*H][NC] chunk totals of q . dq - k . dk
  float* ws_U;        // [B*H][NC][d_qk d_v + d_qk] local, then scanned, backward states
  float* ws_carry;    // [B*H][NSEG][d_qk d_v + d_qk] segment totals / carries (two-level scan), or null
  float* ws_segdec;   // [B*H][NSEG] decay over each segment (two-level scan)
  int NSEG;           // segments of 32 chunks of the two-level scan
  float* ws_rdec;     // [B*H][NC] decay from the end of chunk c to the end of its segment (two-level scan)
  float* ws_qdq;      // [B*H][NC*64] q . dq
  float* ws_kdki;     // [B*H][NC*64] in-chunk part of k . dk
  float* ws_kdk;      // [B*H][NC*64][d_qk/64 or 1] partials of the rest of k . dk
  void* dq;
  void* dk;
  void* dv;
  void* di;
  void* df;
  void* d_o;
  float* dbias;
  float* dC0;
  float* dn0;
  // gradient arriving at the stabilised final state (S~_T, n~_T at fixed
  // m_T), layouts of dC0 / dn0, or null; ws_cT [B*H][(d_qk/64)(d_v/64)]
  // receives the walk tiles' partials of <dC_T, S~_T> + <dn_T, n~_T>
  const float* dCT;
  const float* dnT;
  float* ws_cT;
};
bool bwd_supported(int dtype, int dqk, int dv, int nb);
hipError_t launch_bwd(int dtype, const BwdParams& p, hipStream_t stream);

}  // namespace mlstm
