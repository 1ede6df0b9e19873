/*
 * libmlstm -- mLSTM matrix-memory recurrence and RetNet retention on AMD
 * Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The method.
 *   Matrix memory, exponential input gate, log-space stabilised gating:
 *     "mLSTM Model" page (DeepChrInteract-v2), section "Core idea" and its
 *     display equation C_t = f_t C_{t-1} + i_t (v_t (x) k_t).
 *   Normaliser with learnable bias and block-diagonal memory:
 *     "Edifice.Recurrent.XLSTMv2" page, section "Key Improvements over
 *     xLSTM v1", items 1 and 2 (normaliser read as the vector n_t = f n + i k
 *     with readout n_t . q_t; the page prints a scalar form without q).
 *   Retention (s_n = gamma s_{n-1} + K_n^T V_n, o_n = Q_n s_n) and
 *   gamma_h = 1 - 2^(-5-h): "Edifice.Attention.RetNet" page, sections
 *   "Key Innovation: Retention Mechanism" and "Multi-Scale Retention (MSR)";
 *   the parallel, recurrent and chunkwise modes of its "Triple Paradigm".
 *   In-place [B,H,K,V] state and chunk_size 64: burn-gdn2 config.rs,
 *   Gdn2Mode::FusedRecurrent / Gdn2Mode::Chunk and Gdn2Config::chunk_size.
 *
 * Per (batch b, head h), with f = sigmoid(f_pre), i = exp(i_pre),
 * o = sigmoid(o_pre) (or 1 when o_pre is NULL):
 *     C_t = f_t C_{t-1} + i_t v_t k_t^T       n_t = f_t n_{t-1} + i_t k_t
 *     h_t = o_t * (C_t q_t) / max(|n_t . q_t + bias_h|, 1)
 * computed on the stabilised state S~ = C^T e^{-m}, n~ = n e^{-m} with
 * m_t = max(log f_t + m_{t-1}, i_pre_t), m_0 = 0.  With num_blocks = nb > 1
 * q, k, v are split into nb contiguous slices and C is block diagonal; gates,
 * m, n and the denominator stay per head.
 *
 * Conventions for every entry point.
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *   - q, k, v, gate preactivations, o_pre and outputs h use the call's dtype;
 *     states (C, n, m, S), norm_bias and gamma are always fp32.
 *   - The caller owns every buffer.  No call allocates memory, and no
 *     compute call keeps a pointer after returning.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = default stream) and the call returns
 *     without synchronising.
 *   - State the library holds: per calling thread, the last error message
 *     and the two events of mlstm_set_profile_events (until it is called with
 *     NULL, NULL); per GPU, the 64 MiB device array that only
 *     mlstm_chunkwise_fwd_noalloc uses (module memory, part of the library's
 *     code object on that device, held until the process ends).
 *   - Return value: 0 on success, a negative MLSTM_E_* code otherwise.  All
 *     argument checks happen before anything is enqueued, so on error no
 *     output has been touched.  mlstm_last_error() describes the last error of
 *     the calling thread.
 *   - Checks run on the host and need no GPU; MLSTM_E_HIP reports a failed
 *     kernel launch.
 */
#ifndef MLSTM_H_
#define MLSTM_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLSTM_ABI_VERSION 2

typedef enum { MLSTM_F32 = 0, MLSTM_BF16 = 1 } mlstm_dtype;

enum {
  MLSTM_OK = 0,
  MLSTM_E_NULL = -1,        /* a required pointer is NULL */
  MLSTM_E_SHAPE = -2,       /* a size is out of range or inconsistent */
  MLSTM_E_DTYPE = -3,       /* unknown dtype */
  MLSTM_E_UNSUPPORTED = -4, /* valid request without a compiled kernel variant */
  MLSTM_E_WORKSPACE = -5,   /* workspace missing or too small */
  MLSTM_E_HIP = -6          /* the HIP runtime reported an error */
};

/* Version of this ABI (MLSTM_ABI_VERSION of the library that was built). */
int mlstm_abi_version(void);

/* Message for the last error returned on the calling thread ("" if none).
 * The string stays valid until the next call on that thread. */
const char* mlstm_last_error(void);

/*
 * Profiling hook.  While set, every mlstm_chunkwise_fwd and
 * retention_chunkwise_fwd call made on the calling thread records ev_start
 * (a hipEvent_t) on its stream right before its main kernel (the per-chunk
 * readout/update kernel) and ev_stop right after it, so that
 * hipEventElapsedTime(ev_start, ev_stop) is that kernel's duration.  The
 * caller owns the events.  (NULL, NULL) disables; giving only one of them is
 * MLSTM_E_NULL.
 */
int mlstm_set_profile_events(void* ev_start, void* ev_stop);

/*
 * Workspace size in bytes for mlstm_chunkwise_fwd with these arguments
 * (0 if none is needed).  Returns 0 and sets the error message for invalid
 * arguments; call mlstm_chunkwise_fwd to get the error code.
 */
size_t mlstm_chunkwise_workspace_bytes(int B, int H, int T, int d_qk, int d_v,
                                       int num_blocks, int chunk,
                                       mlstm_dtype dt);

/*
 * Chunkwise-parallel forward (prefill / training forward) over T tokens.
 *   q, k     [B,H,T,d_qk]        dtype dt
 *   v        [B,H,T,d_v]         dtype dt
 *   i_pre    [B,H,T]             input-gate preactivation (i = exp(i_pre))
 *   f_pre    [B,H,T]             forget-gate preactivation (f = sigmoid)
 *   o_pre    [B,H,T,d_v] or NULL output-gate preactivation (o = sigmoid)
 *   norm_bias [H] fp32 or NULL   normaliser bias (NULL = 0)
 *   C0       [B,H,nb,d_qk/nb,d_v/nb] fp32 or NULL   initial S~ (NULL = 0)
 *   n0       [B,H,d_qk] fp32 or NULL                initial n~ (NULL = 0)
 *   m0       [B,H] fp32 or NULL                     initial m  (NULL = 0)
 *   h        [B,H,T,d_v]         output, dtype dt
 *   C_out, n_out, m_out          final stabilised state, same layouts as
 *                                C0/n0/m0, or NULL to skip; each may alias
 *                                its initial-state counterpart.
 *   workspace, workspace_bytes   device scratch of at least
 *                                mlstm_chunkwise_workspace_bytes(...) bytes,
 *                                256-byte aligned; overwritten by the call.
 * chunk is the chunk length L (64 for bf16; 16, 32 or 64 for fp32).
 * Supported (d_qk, num_blocks): bf16 {(64,1),(64,2),(128,1),(256,1),(256,2)},
 * fp32 {(64,1),(64,2)}.  d_v must be a multiple of 128 when d_qk/num_blocks
 * >= 128 (bf16), else of 64, and d_v/num_blocks a multiple of 32 resp. 16.
 * Any T >= 1.  Other combinations return MLSTM_E_UNSUPPORTED.
 * A call whose plan has one superchunk (T <= chunk always; longer T when
 * B*H fills the GPU) is one kernel launch that reads C0/n0/m0 directly (the
 * parallel form of a short sequence); otherwise three launches.  The results
 * are the same bit for bit either way.
 */
int mlstm_chunkwise_fwd(int B, int H, int T, int d_qk, int d_v, int num_blocks,
                        int chunk, mlstm_dtype dt, const void* q, const void* k,
                        const void* v, const void* i_pre, const void* f_pre,
                        const void* o_pre, const float* norm_bias,
                        const float* C0, const float* n0, const float* m0,
                        float* C_out, float* n_out, float* m_out, void* h,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Normaliser readings (norm_mode of the _ex entry points).
 *   MLSTM_NORM_VECTOR  n_t = f n + i k_t, denominator |n_t . q_t + bias| (the
 *                      reading of every other entry point);
 *   MLSTM_NORM_SCALAR  n_t = f n + i (one scalar per head), denominator
 *                      |n_t + bias|: the normaliser exactly as the
 *                      "Edifice.Recurrent.XLSTMv2" page prints it in "Key
 *                      Improvements over xLSTM v1", item 2 (no k, no q);
 *   MLSTM_NORM_BLOCK   n_t as for VECTOR, but memory block b divides by its
 *                      own |n_t,b . q_t,b + bias| over the block's features
 *                      (the block-diagonal memory of item 1 read as
 *                      independent cells; the same as VECTOR with one block;
 *                      the decode step takes at most 8 blocks).
 * All take max(., 1) as on that page (in stabilised units).
 */
#define MLSTM_NORM_VECTOR 0
#define MLSTM_NORM_SCALAR 1
#define MLSTM_NORM_BLOCK 2

/*
 * mlstm_chunkwise_fwd with a choice of normaliser.  With MLSTM_NORM_SCALAR
 * n0 and n_out are [B,H] fp32 (one value per head); everything else, the
 * supported shapes and the workspace size are those of mlstm_chunkwise_fwd.
 * Unknown modes return MLSTM_E_UNSUPPORTED.
 */
int mlstm_chunkwise_fwd_ex(int B, int H, int T, int d_qk, int d_v, int num_blocks,
                           int chunk, mlstm_dtype dt, int norm_mode,
                           const void* q, const void* k, const void* v,
                           const void* i_pre, const void* f_pre,
                           const void* o_pre, const float* norm_bias,
                           const float* C0, const float* n0, const float* m0,
                           float* C_out, float* n_out, float* m_out, void* h,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * mlstm_chunkwise_fwd_ex without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Its kernels use a scratch array
 * that the library holds in device memory: one copy of
 * mlstm_noalloc_scratch_bytes() bytes (64 MiB) per GPU, created when the
 * library's code loads on that GPU and kept until the process ends.  This
 * call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Its first call on a device looks the array's address up once
 * (hipGetSymbolAddress) with that device current.  A call whose
 * mlstm_chunkwise_workspace_bytes(...) exceeds the scratch size returns
 * MLSTM_E_WORKSPACE before anything runs.  Every call on one GPU uses the
 * same array and leaves its contents behind (nothing in it needs to start at
 * zero): calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and must not be made.  Arguments,
 * outputs and supported shapes are those of mlstm_chunkwise_fwd_ex.
 */
int mlstm_chunkwise_fwd_noalloc(int B, int H, int T, int d_qk, int d_v,
                                int num_blocks, int chunk, mlstm_dtype dt,
                                int norm_mode, const void* q, const void* k,
                                const void* v, const void* i_pre,
                                const void* f_pre, const void* o_pre,
                                const float* norm_bias, const float* C0,
                                const float* n0, const float* m0,
                                float* C_out, float* n_out, float* m_out,
                                void* h, void* stream);

/* Size in bytes of the per-GPU scratch array of mlstm_chunkwise_fwd_noalloc. */
size_t mlstm_noalloc_scratch_bytes(void);

/*
 * Fused single-token decode step on every (b, h); the fp32 state is updated
 * IN PLACE and the readout uses the updated state.
 *   q, k  [B,H,d_qk]; v [B,H,d_v]; i_pre, f_pre [B,H]; o_pre [B,H,d_v] or
 *   NULL (dtype dt); norm_bias [H] fp32 or NULL;
 *   C [B,H,nb,d_qk/nb,d_v/nb], n [B,H,d_qk], m [B,H] fp32, read and written;
 *   h [B,H,d_v] output (dtype dt).
 * Requires d_v a multiple of 16 and d_v/nb a multiple of 4; other shapes
 * return MLSTM_E_UNSUPPORTED.  Two kernels are enqueued (the matrix state
 * with the outputs, then n and m).
 */
int mlstm_step(int B, int H, int d_qk, int d_v, int num_blocks, mlstm_dtype dt,
               const void* q, const void* k, const void* v, const void* i_pre,
               const void* f_pre, const void* o_pre, const float* norm_bias,
               float* C, float* n, float* m, void* h, void* stream);

/*
 * mlstm_step with a choice of normaliser (see MLSTM_NORM_*).  With
 * MLSTM_NORM_SCALAR n is [B,H] fp32.  Unknown modes return
 * MLSTM_E_UNSUPPORTED.
 */
int mlstm_step_ex(int B, int H, int d_qk, int d_v, int num_blocks, mlstm_dtype dt,
                  int norm_mode, const void* q, const void* k, const void* v,
                  const void* i_pre, const void* f_pre, const void* o_pre,
                  const float* norm_bias, float* C, float* n, float* m,
                  void* h, void* stream);

/* Workspace size in bytes for retention_chunkwise_fwd (0 if none). */
size_t retention_chunkwise_workspace_bytes(int B, int H, int T, int d_k,
                                           int d_v, int chunk, mlstm_dtype dt);

/*
 * RetNet retention, chunkwise form: out_t = sum_{s<=t} gamma_h^{t-s}
 * (q_t . k_s) v_s + gamma_h^{t+1} q_t S0, i.e. the recurrence
 * S_t = gamma_h S_{t-1} + k_t v_t^T, out_t = S_t^T q_t.  No normaliser, no
 * gates, no stabiliser.
 *   q, k [B,H,T,d_k]; v, out [B,H,T,d_v] (dtype dt);
 *   gamma [H] fp32 in (0,1), or NULL for gamma_h = 1 - 2^(-5-h), h = 0..H-1;
 *   S0, S_out [B,H,d_k,d_v] fp32 or NULL (S_out may alias S0).
 * Supported d_k: bf16 {64, 128}, fp32 {64}; d_v as for mlstm_chunkwise_fwd.
 */
int retention_chunkwise_fwd(int B, int H, int T, int d_k, int d_v, int chunk,
                            mlstm_dtype dt, const void* q, const void* k,
                            const void* v, const float* gamma, const float* S0,
                            float* S_out, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Workspace size in bytes for retention_chunkwise_groupnorm_fwd: that of
 * retention_chunkwise_fwd, plus B*H*T*d_v fp32 when d_v is wider than one
 * work-group (0, with the error message set, for arguments it does not take).
 */
size_t retention_chunkwise_groupnorm_workspace_bytes(int B, int H, int T, int d_k,
                                                     int d_v, int chunk,
                                                     mlstm_dtype dt);

/*
 * retention_chunkwise_fwd with the per-head group norm of the "Multi-Scale
 * Retention (MSR)" section of the "Edifice.Attention.RetNet" page applied to
 * the outputs: each output row of each head is normalised over its d_v
 * channels,
 *     out = (y - mean(y)) / sqrt(var(y) + gn_eps) * gn_weight + gn_bias
 * with y the retention output, mean and (biased) variance over the row, and
 * per-channel gn_weight, gn_bias [H*d_v] fp32 (NULL: 1 and 0), as a group
 * norm with one group per head over the H*d_v channels.  Statistics are
 * taken in fp32 before rounding to dt.  Same arguments and S0/S_out as
 * retention_chunkwise_fwd; gn_eps > 0; the workspace size comes from
 * retention_chunkwise_groupnorm_workspace_bytes.  Requires d_v a multiple of
 * W, the d_v width one work-group holds (64 for d_k = 64, 128 for d_k = 128).
 * With d_v = W the norm is applied in the output write.  With d_v > W the
 * output pass writes the unnormalised rows in fp32 to the workspace and one
 * more kernel normalises them into out (the same arithmetic, at the cost of
 * one fp32 write and read of the outputs).  Other shapes return
 * MLSTM_E_UNSUPPORTED; more than 2^33 output rows (B*H*T) return
 * MLSTM_E_SHAPE.
 */
int retention_chunkwise_groupnorm_fwd(int B, int H, int T, int d_k, int d_v,
                                      int chunk, mlstm_dtype dt, const void* q,
                                      const void* k, const void* v,
                                      const float* gamma, const float* S0,
                                      float* S_out, const float* gn_weight,
                                      const float* gn_bias, float gn_eps,
                                      void* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * RetNet retention, one decode step on every (b, h), in the recurrent form of
 * the "Edifice.Attention.RetNet" page ("Key Innovation: Retention
 * Mechanism"; recurrent mode of "Triple Paradigm"):
 *     S <- gamma_h S + k v^T     (IN PLACE),     out = S^T q
 * (the readout uses the updated state, as one token of
 * retention_chunkwise_fwd does).
 *   q, k [B,H,d_k]; v, out [B,H,d_v] (dtype dt);
 *   gamma [H] fp32, or NULL for gamma_h = 1 - 2^(-5-h), h = 0..H-1;
 *   S [B,H,d_k,d_v] fp32, read and written.
 * Requires d_v a multiple of 16 (any d_k >= 1); other shapes return
 * MLSTM_E_UNSUPPORTED.  One kernel is enqueued.
 */
int retention_step(int B, int H, int d_k, int d_v, mlstm_dtype dt,
                   const void* q, const void* k, const void* v,
                   const float* gamma, float* S, void* out, void* stream);

/*
 * Workspace size in bytes for mlstm_chunkwise_bwd (0, with the error message
 * set, for arguments it does not take).
 */
size_t mlstm_chunkwise_bwd_workspace_bytes(int B, int H, int T, int d_qk, int d_v,
                                           int num_blocks, int chunk, mlstm_dtype dt);

/*
 * Chunkwise backward pass of the mLSTM (vector normaliser): the gradients of
 * L = sum(dh * h) for h = mlstm_chunkwise_fwd(...) with the same inputs and
 * initial state (vector normaliser).  The pages run training on the parallel and chunked forms
 * ("Triple Paradigm" section of the "Edifice.Attention.RetNet" page; the
 * chunked-scan mode of Gdn2Mode on the "burn-gdn2" page); this is the
 * gradient of the same chunkwise computation, recomputing the stabiliser, the
 * chunk states and the outputs from the inputs (nothing is kept from the
 * forward call).
 *   q, k, v, i_pre, f_pre, o_pre, norm_bias, C0, n0, m0   as passed to the
 *                  forward (o_pre, norm_bias, C0, n0, m0 may be NULL);
 *   dh       [B,H,T,d_v]  gradient of the loss with respect to h (dtype dt);
 *   dC_T [B,H,nb,d_qk/nb,d_v/nb], dn_T [B,H,d_qk] fp32 or NULL (zero): the
 *                  gradient arriving at the final stabilised state (C_out,
 *                  n_out of the forward) at fixed m_out, i.e. e^{m_T} times
 *                  the gradient with respect to the true final C_T, n_T.  The
 *                  loss is taken to depend on the final state only through
 *                  the true state, as a continuation of the recurrence does
 *                  (its outputs do not depend on the stabiliser), so m_out
 *                  gets no gradient of its own.  A following call's dC0, dn0
 *                  are exactly this call's dC_T, dn_T, so calls chain;
 *   dq, dk   [B,H,T,d_qk], dv [B,H,T,d_v], di_pre, df_pre [B,H,T]  outputs,
 *                  dtype dt (gradients of q, k, v and of the gate
 *                  preactivations i_pre, f_pre);
 *   do_pre   [B,H,T,d_v] dtype dt: gradient of o_pre; required exactly when
 *                  o_pre is given, else NULL;
 *   dbias    [H] fp32 or NULL: gradient of norm_bias, summed over the batch;
 *   dC0 [B,H,nb,d_qk/nb,d_v/nb], dn0 [B,H,d_qk] fp32 or NULL: gradients of
 *                  the stabilised initial state C0, n0 (also for a zero state).
 *                  The gradient of m0 is <dC0, C0> + <dn0, n0>.
 * Requires chunk = 64 and either num_blocks = 1 with d_v a multiple of 64 and
 * d_qk in {64, 128, 256} (bf16) or 64 (fp32), or num_blocks = 2 with
 * d_qk = d_v = 64 (the block-diagonal memory of the "Edifice.Recurrent.XLSTMv2"
 * page, "Key Improvements" item 1: one numerator per block, the normaliser
 * over the head); other shapes return MLSTM_E_UNSUPPORTED.  workspace: at least mlstm_chunkwise_bwd_workspace_bytes
 * bytes, 256-byte aligned (it holds the start state of every chunk and the
 * backward state at every chunk end, fp32: 2 (d_qk d_v + d_qk) 4 bytes per
 * chunk and batch*head).  Enqueues the forward's state passes and eight
 * backward kernels on stream; profile events set by mlstm_set_profile_events
 * bracket the backward kernels.
 */
int mlstm_chunkwise_bwd(int B, int H, int T, int d_qk, int d_v, int num_blocks,
                        int chunk, mlstm_dtype dt, const void* q, const void* k,
                        const void* v, const void* i_pre, const void* f_pre,
                        const void* o_pre, const float* norm_bias,
                        const float* C0, const float* n0, const float* m0,
                        const void* dh, const float* dC_T, const float* dn_T,
                        void* dq, void* dk, void* dv, void* di_pre, void* df_pre,
                        void* do_pre, float* dbias, float* dC0, float* dn0,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace size in bytes for retention_chunkwise_bwd (0 for arguments it
 * does not take, with the error message set). */
size_t retention_chunkwise_bwd_workspace_bytes(int B, int H, int T, int d_k, int d_v,
                                               int chunk, mlstm_dtype dt);

/*
 * Chunkwise backward pass of RetNet retention: the gradients of
 * L = sum(dout * out) for out = retention_chunkwise_fwd(...) with the same
 * q, k, v, gamma and S0.  The RetNet page trains with the parallel form
 * ("Triple Paradigm": parallel mode is the training mode); this is the
 * gradient of the same function, computed chunkwise:
 *     dq_t = S_t dout_t,  dk_t = G_t v_t,  dv_t = G_t^T k_t,
 *     G_t = gamma_h G_{t+1} + q_t dout_t^T,  G_T = dS_T,  dS0 = gamma_h G_0.
 *   q, k [B,H,T,d_k]; v, dout [B,H,T,d_v] (dtype dt); gamma [H] fp32 or NULL
 *   (1 - 2^(-5-h)); S0 [B,H,d_k,d_v] fp32 or NULL (zero);
 *   dS_T [B,H,d_k,d_v] fp32 or NULL (zero): gradient arriving at the final
 *   state S_out (a following call's dS0), so that calls chain;
 *   dq, dk [B,H,T,d_k], dv [B,H,T,d_v] outputs, dtype dt;
 *   dS0 [B,H,d_k,d_v] fp32 or NULL: gradient of S0 (also for a zero S0).
 * Requires chunk = 64, d_v a multiple of 64 and d_k in {64, 128} (bf16) or 64
 * (fp32); other shapes return MLSTM_E_UNSUPPORTED.  workspace: at least
 * retention_chunkwise_bwd_workspace_bytes bytes, 256-byte aligned.  Enqueues
 * the forward's state passes and the backward kernels of mlstm_chunkwise_bwd
 * (without the gate and bias ones) on stream.
 */
int retention_chunkwise_bwd(int B, int H, int T, int d_k, int d_v, int chunk,
                            mlstm_dtype dt, const void* q, const void* k,
                            const void* v, const float* gamma, const float* S0,
                            const void* dout, const float* dS_T, void* dq, void* dk,
                            void* dv, float* dS0, void* workspace,
                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_H_ */
