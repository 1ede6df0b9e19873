// C ABI of libmlstm (declared in include/mlstm.h): argument checks, kernel
// variant selection, workspace layout and launches on the caller's stream.
// Every check runs before any HIP call, so invalid calls need no GPU and
// touch no output.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/mlstm.h"
#include "kernels.h"

// Scratch of mlstm_chunkwise_fwd_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a host
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress (per device, see scratch_ptr) and only that address is
// handed to kernels.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512];
thread_local hipEvent_t g_ev0 = nullptr, g_ev1 = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MLSTM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Pass 3 folds pass 2 in (composes its own start state from pass 1's local
// states) when a head has at most this many superchunks of at most this many
// state entries: each of its work-groups then reads at most 7 local states.
constexpr long long kFuseScanMaxNS = 8;
constexpr size_t kFuseScanMaxState = 64 * 64;

// Optional tuning override: chunks per superchunk.
int env_superchunk_chunks() {
  const char* s = getenv("MLSTM_SUPERCHUNK_CHUNKS");
  if (!s) return 0;
  const int g = atoi(s);
  return g > 0 ? g : 0;
}

struct Plan {
  mlstm::ChunkVariant var;
  int L, NC, G, NS, nslices;
  size_t CS, nstate;
  size_t off_scal, off_min, off_g, bytes;
};

// Checks shared by the mLSTM and retention chunkwise entry points and the
// workspace queries; fills the plan.  Returns MLSTM_OK or an error code.
int plan_chunkwise(int B, int H, int T, int dqk, int dv, int nb, int chunk, int dt, bool ret,
                   Plan* pl, bool for_bwd = false) {
  if (dt != MLSTM_F32 && dt != MLSTM_BF16) return fail(MLSTM_E_DTYPE, "unknown dtype %d", dt);
  if (B < 1 || H < 1 || T < 1 || dqk < 1 || dv < 1 || nb < 1)
    return fail(MLSTM_E_SHAPE, "sizes must be positive (B=%d H=%d T=%d d_qk=%d d_v=%d nb=%d)", B, H, T,
                dqk, dv, nb);
  if (dqk % nb || dv % nb)
    return fail(MLSTM_E_SHAPE, "d_qk=%d and d_v=%d must be multiples of num_blocks=%d", dqk, dv, nb);
  // The kernels address one (batch, head) of q, k, v, h, o_pre, dh and the
  // gradients through buffer resources with 32-bit byte offsets (and a signed
  // 32-bit scalar part): that slice must stay below 2^31 bytes.
  const long long es = dt == MLSTM_BF16 ? 2 : 4;
  if ((long long)T * (dqk > dv ? dqk : dv) * es >= (1LL << 31))
    return fail(MLSTM_E_SHAPE, "one (batch, head) of T x d = %d x %d %s elements exceeds 2^31 bytes", T,
                dqk > dv ? dqk : dv, dt == MLSTM_BF16 ? "bf16" : "fp32");
  if ((long long)B * H >= (1LL << 24)) return fail(MLSTM_E_SHAPE, "B * H too large");
  if (chunk != 16 && chunk != 32 && chunk != 64)
    return fail(MLSTM_E_SHAPE, "chunk must be 16, 32 or 64 (got %d)", chunk);
  if (!mlstm::find_chunk_variant(dt, dqk, nb, chunk, ret, &pl->var))
    return fail(MLSTM_E_UNSUPPORTED,
                "no kernel for dtype=%s d_qk=%d num_blocks=%d chunk=%d%s", dt ? "bf16" : "fp32", dqk, nb,
                chunk, ret ? " (retention)" : "");
  const int W = pl->var.w;
  if (dv % W || (dv / nb) % pl->var.wc)
    return fail(MLSTM_E_UNSUPPORTED, "d_v=%d must be a multiple of %d with d_v/num_blocks a multiple of %d",
                dv, W, pl->var.wc);
  pl->L = chunk;
  pl->nslices = dv / W;
  pl->NC = (T + chunk - 1) / chunk;
  // Superchunks: enough work-groups to fill 256 CUs at the occupancy the
  // LDS footprint allows.
  int per_cu = (int)(160 * 1024 / pl->var.lds_bytes);
  if (per_cu < 1) per_cu = 1;
  if (per_cu > 4) per_cu = 4;
  const long long base = (long long)B * H * pl->nslices;
  long long ns = (256LL * per_cu + base - 1) / base;
  // In a forward call a small state (at most 64 x 64 per head) gets at most
  // kFuseScanMaxNS superchunks, so that pass 3 can compose its start state
  // itself.  The backward keeps the plan its precision was measured with
  // (with the cap, a bf16 case of 257 chunks and a final-state gradient
  // measured a dq error of 2.3e-2 against the 2e-2 bar).
  if (!for_bwd && (size_t)dqk * dv / nb <= kFuseScanMaxState && ns > kFuseScanMaxNS) ns = kFuseScanMaxNS;
  if (ns < 1) ns = 1;
  if (ns > pl->NC) ns = pl->NC;
  int G = (int)((pl->NC + ns - 1) / ns);
  if (env_superchunk_chunks()) G = env_superchunk_chunks();
  if (G * chunk > 1024) G = 1024 / chunk;  // pass 1 holds the gate factors of <= 1024 tokens
  if (G > pl->NC) G = pl->NC;
  pl->G = G;
  pl->NS = (pl->NC + G - 1) / G;
  pl->CS = (size_t)dqk * dv / nb;
  pl->nstate = pl->CS + (ret ? 0 : dqk);
  const size_t BH = (size_t)B * H;
  pl->off_scal = align256(BH * pl->NS * pl->nstate * sizeof(float));
  pl->off_min = pl->off_scal + align256(BH * pl->NS * 2 * sizeof(float));
  pl->off_g = pl->off_min + align256(BH * pl->NS * sizeof(float));
  pl->bytes = pl->off_g + 3 * align256(BH * (size_t)pl->NC * chunk * sizeof(float));
  return MLSTM_OK;
}

int launch(const Plan& pl, mlstm::ChunkParams& p, void* workspace, size_t workspace_bytes,
           void* stream) {
  if (!workspace) return fail(MLSTM_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", pl.bytes);
  if (workspace_bytes < pl.bytes)
    return fail(MLSTM_E_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, pl.bytes);
  if ((size_t)workspace & 255) return fail(MLSTM_E_WORKSPACE, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  p.NC = pl.NC;
  p.G = pl.G;
  p.NS = pl.NS;
  p.nslices = pl.nslices;
  p.ws_state = reinterpret_cast<float*>(ws);
  p.ws_scal = reinterpret_cast<float*>(ws + pl.off_scal);
  p.ws_min = reinterpret_cast<float*>(ws + pl.off_min);
  const size_t gsz = align256((size_t)p.B * p.H * pl.NC * pl.L * sizeof(float));
  p.ws_ga = reinterpret_cast<float*>(ws + pl.off_g);
  p.ws_gg = reinterpret_cast<float*>(ws + pl.off_g + gsz);
  p.ws_gb = reinterpret_cast<float*>(ws + pl.off_g + 2 * gsz);
  // A plan of one superchunk runs as pass 3 alone, straight from the caller's
  // initial state: one launch instead of three.  Not when the final n~ or m
  // overwrites an initial-state array that the other d_v slices of the head
  // still read (each slice reads and rewrites only its own columns of C).
  const bool clobbers = pl.nslices > 1 && ((p.n_out && p.n_out == p.n0) || (p.m_out && p.m_out == p.m0));
  p.direct = (pl.NS == 1 && !clobbers) ? 1 : 0;
  // With few superchunks of a small state, pass 3 composes each start state
  // itself and pass 2 is not launched.  Every work-group then reads the
  // caller's initial state, so not when the final state overwrites it.
  const bool in_place = (p.C_out && p.C_out == p.C0) || (p.n_out && p.n_out == p.n0) || (p.m_out && p.m_out == p.m0);
  p.fuse_scan = (pl.NS > 1 && pl.NS <= kFuseScanMaxNS && pl.CS <= kFuseScanMaxState && !in_place) ? 1 : 0;
  const hipError_t e = pl.var.launch(p, static_cast<hipStream_t>(stream), g_ev0, g_ev1);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Backward workspace: the forward plan with one chunk per superchunk, then
// the backward's own arrays.
struct BwdPlan {
  Plan fwd;
  size_t off_carry, off_segdec, off_rdec, nseg, off_cst, off_cmin, off_U, off_Pt, off_Dt, off_rden, off_dz, off_db, off_dbh, off_qdq, off_kdki,
      off_kdk, off_cT, bytes;
};

int plan_bwd(int B, int H, int T, int dqk, int dv, int nb, int chunk, int dt, BwdPlan* bp, bool ret = false) {
  const int rc = plan_chunkwise(B, H, T, dqk, dv, nb, chunk, dt, ret, &bp->fwd, true);
  if (rc != MLSTM_OK) return rc;
  if (nb != 1 && !(nb == 2 && dqk == 64 && dv == 64 && !ret))
    return fail(MLSTM_E_UNSUPPORTED, "the backward pass takes num_blocks = 1, or 2 with d_qk = d_v = 64 (got %d)", nb);
  if (chunk != 64) return fail(MLSTM_E_UNSUPPORTED, "the backward pass takes chunk = 64 (got %d)", chunk);
  if (!mlstm::bwd_supported(dt, dqk, dv, nb))
    return fail(MLSTM_E_UNSUPPORTED, "no backward kernel for dtype=%s d_qk=%d d_v=%d", dt ? "bf16" : "fp32", dqk,
                dv);
  const size_t BH = (size_t)B * H, NC = bp->fwd.NC, NCL = NC * 64, es = dt ? 2 : 4;
  size_t o = align256(bp->fwd.bytes);
  bp->off_cst = o;
  o += align256(BH * NC * ((size_t)dqk * dv + dqk) * 4);
  bp->off_cmin = o;
  o += align256(BH * NC * 4);
  bp->off_U = o;
  o += align256(BH * NC * ((size_t)dqk * dv + dqk) * 4);
  const size_t tile = align256(BH * NC * nb * 64 * 64 * es);  // one 64 x 64 per chunk and memory block
  bp->off_Pt = o;
  bp->off_Dt = o + tile;
  o += 2 * tile;
  bp->off_rden = o;
  o += align256(BH * NCL * 4);
  bp->off_dz = o;
  o += align256(BH * NCL * 4);
  bp->off_db = o;
  o += align256(BH * NC * 4);
  bp->off_dbh = o;
  o += align256(BH * NC * 4);
  bp->off_qdq = o;
  o += align256(BH * NCL * 4);
  bp->off_kdki = o;
  o += align256(BH * NCL * 4);
  bp->off_kdk = o;
  o += align256(BH * NCL * (dqk / 64) * 4);
  // two-level backward scan for long sequences (256 chunks or more): segment
  // totals / carries, one state per 32 chunks
  bp->nseg = NC >= 256 ? (NC + 31) / 32 : 0;
  bp->off_carry = o;
  o += align256(BH * bp->nseg * ((size_t)dqk * dv + dqk) * 4);
  bp->off_segdec = o;
  o += align256(BH * bp->nseg * 4);
  bp->off_rdec = o;  // per chunk, with the two-level scan only
  o += align256(BH * (bp->nseg ? NC : 0) * 4);
  // partials of <dC_T, S~_T> + <dn_T, n~_T>, one per 64 x 64 state tile
  bp->off_cT = o;
  o += align256(BH * (size_t)(dqk / 64 > 0 ? dqk / 64 : 1) * (dv / 64 > 0 ? dv / 64 : 1) * 4);
  bp->bytes = o;
  return MLSTM_OK;
}

}  // namespace

namespace {

// The device address of this device's copy of `scratch`, looked up once per
// device (with that device current, as the caller's stream requires).
int scratch_ptr(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLSTM_E_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLSTM_E_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return MLSTM_OK;
}

// Shared by mlstm_chunkwise_fwd(_ex) (the caller's workspace) and
// mlstm_chunkwise_fwd_noalloc (this device's scratch array).
int chunkwise_fwd_impl(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk, mlstm_dtype dt,
                              int norm_mode, const void* q, const void* k, const void* v, const void* i_pre,
                              const void* f_pre, const void* o_pre, const float* norm_bias, const float* C0,
                              const float* n0, const float* m0, float* C_out, float* n_out, float* m_out, void* h,
                              void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  if (norm_mode != MLSTM_NORM_VECTOR && norm_mode != MLSTM_NORM_SCALAR && norm_mode != MLSTM_NORM_BLOCK)
    return fail(MLSTM_E_UNSUPPORTED, "unknown norm_mode %d", norm_mode);
  Plan pl;
  const int rc = plan_chunkwise(B, H, T, d_qk, d_v, num_blocks, chunk, dt, false, &pl);
  if (rc != MLSTM_OK) return rc;
  if (!q || !k || !v || !i_pre || !f_pre || !h)
    return fail(MLSTM_E_NULL, "q, k, v, i_pre, f_pre and h are required");
  if (noalloc) {
    if (pl.bytes > kScratchBytes)
      return fail(MLSTM_E_WORKSPACE, "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu",
                  pl.bytes, kScratchBytes);
    const int rs = scratch_ptr(&workspace);
    if (rs != MLSTM_OK) return rs;
    workspace_bytes = kScratchBytes;
  }
  if (norm_mode == MLSTM_NORM_SCALAR) {
    if (!pl.var.launch_scalar_norm) return fail(MLSTM_E_UNSUPPORTED, "no scalar-normaliser kernel");
    pl.var.launch = pl.var.launch_scalar_norm;  // same plan and workspace
  }
  if (norm_mode == MLSTM_NORM_BLOCK && num_blocks > 1) {  // one block: the vector normaliser
    if (!pl.var.launch_block_norm) return fail(MLSTM_E_UNSUPPORTED, "no per-block-normaliser kernel");
    pl.var.launch = pl.var.launch_block_norm;
  }
  mlstm::ChunkParams p{};
  p.B = B;
  p.H = H;
  p.T = T;
  p.DV = d_v;
  p.q = q;
  p.k = k;
  p.v = v;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.o_pre = o_pre;
  p.bias = norm_bias;
  p.ret_gamma = nullptr;
  p.has_init = (C0 || n0 || m0) ? 1 : 0;
  p.C0 = C0;
  p.n0 = n0;
  p.m0 = m0;
  p.h = h;
  p.C_out = C_out;
  p.n_out = n_out;
  p.m_out = m_out;
  return launch(pl, p, workspace, workspace_bytes, stream);
}

}  // namespace

extern "C" {

size_t mlstm_chunkwise_bwd_workspace_bytes(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk,
                                           mlstm_dtype dt) {
  BwdPlan bp;
  if (plan_bwd(B, H, T, d_qk, d_v, num_blocks, chunk, dt, &bp) != MLSTM_OK) return 0;
  return bp.bytes;
}

int mlstm_chunkwise_bwd(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk, mlstm_dtype dt,
                        const void* q, const void* k, const void* v, const void* i_pre, const void* f_pre,
                        const void* o_pre, const float* norm_bias, const float* C0, const float* n0,
                        const float* m0, const void* dh, const float* dC_T, const float* dn_T, void* dq,
                        void* dk, void* dv, void* di_pre, void* df_pre, void* do_pre, float* dbias, float* dC0,
                        float* dn0, void* workspace, size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  const int rc = plan_bwd(B, H, T, d_qk, d_v, num_blocks, chunk, dt, &bp);
  if (rc != MLSTM_OK) return rc;
  if (!q || !k || !v || !i_pre || !f_pre || !dh)
    return fail(MLSTM_E_NULL, "q, k, v, i_pre, f_pre and dh are required");
  if (!dq || !dk || !dv || !di_pre || !df_pre) return fail(MLSTM_E_NULL, "dq, dk, dv, di_pre and df_pre are required");
  if ((o_pre == nullptr) != (do_pre == nullptr)) return fail(MLSTM_E_NULL, "do_pre is required exactly when o_pre is given");
  if (!workspace) return fail(MLSTM_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", bp.bytes);
  if (workspace_bytes < bp.bytes)
    return fail(MLSTM_E_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, bp.bytes);
  if ((size_t)workspace & 255) return fail(MLSTM_E_WORKSPACE, "workspace must be 256-byte aligned");
  const Plan& pl = bp.fwd;
  char* ws = static_cast<char*>(workspace);
  // forward state passes only (h = NULL skips the output pass)
  mlstm::ChunkParams p{};
  p.B = B;
  p.H = H;
  p.T = T;
  p.DV = d_v;
  p.q = q;
  p.k = k;
  p.v = v;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.o_pre = o_pre;
  p.bias = norm_bias;
  p.has_init = (C0 || n0 || m0) ? 1 : 0;
  p.C0 = C0;
  p.n0 = n0;
  p.m0 = m0;
  p.h = nullptr;
  p.NC = pl.NC;
  p.G = pl.G;
  p.NS = pl.NS;
  p.nslices = pl.nslices;
  p.ws_state = reinterpret_cast<float*>(ws);
  p.ws_scal = reinterpret_cast<float*>(ws + pl.off_scal);
  p.ws_min = reinterpret_cast<float*>(ws + pl.off_min);
  const size_t gsz = align256((size_t)B * H * pl.NC * pl.L * sizeof(float));
  p.ws_ga = reinterpret_cast<float*>(ws + pl.off_g);
  p.ws_gg = reinterpret_cast<float*>(ws + pl.off_g + gsz);
  p.ws_gb = reinterpret_cast<float*>(ws + pl.off_g + 2 * gsz);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = pl.var.launch(p, st, nullptr, nullptr);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  mlstm::BwdParams b{};
  b.B = B;
  b.H = H;
  b.T = T;
  b.DQK = d_qk;
  b.DV = d_v;
  b.NC = pl.NC;
  b.G = pl.G;
  b.NS = pl.NS;
  b.NB = num_blocks;
  b.sc_nst = pl.nstate;
  b.q = q;
  b.k = k;
  b.v = v;
  b.f_pre = f_pre;
  b.o_pre = o_pre;
  b.bias = norm_bias;
  b.dh = dh;
  b.has_init = p.has_init;
  b.sc_state = p.ws_state;
  b.sc_min = p.ws_min;
  b.ws_state = reinterpret_cast<float*>(ws + bp.off_cst);
  b.ws_min = reinterpret_cast<float*>(ws + bp.off_cmin);
  b.ws_ga = p.ws_ga;
  b.ws_gg = p.ws_gg;
  b.ws_gb = p.ws_gb;
  b.wsPt = ws + bp.off_Pt;
  b.wsDt = ws + bp.off_Dt;
  b.ws_rden = reinterpret_cast<float*>(ws + bp.off_rden);
  b.ws_dz = reinterpret_cast<float*>(ws + bp.off_dz);
  b.ws_dbias = reinterpret_cast<float*>(ws + bp.off_db);
  b.ws_ctot = reinterpret_cast<float*>(ws + bp.off_dbh);
  b.ws_U = reinterpret_cast<float*>(ws + bp.off_U);
  b.ws_qdq = reinterpret_cast<float*>(ws + bp.off_qdq);
  b.ws_kdki = reinterpret_cast<float*>(ws + bp.off_kdki);
  b.ws_kdk = reinterpret_cast<float*>(ws + bp.off_kdk);
  b.NSEG = (int)bp.nseg;
  b.ws_carry = bp.nseg ? reinterpret_cast<float*>(ws + bp.off_carry) : nullptr;
  b.ws_segdec = bp.nseg ? reinterpret_cast<float*>(ws + bp.off_segdec) : nullptr;
  b.ws_rdec = bp.nseg ? reinterpret_cast<float*>(ws + bp.off_rdec) : nullptr;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.di = di_pre;
  b.df = df_pre;
  b.d_o = do_pre;
  b.dbias = dbias;
  b.dC0 = dC0;
  b.dn0 = dn0;
  b.dCT = dC_T;
  b.dnT = dn_T;
  b.ws_cT = (dC_T || dn_T) ? reinterpret_cast<float*>(ws + bp.off_cT) : nullptr;
  if (g_ev0) (void)hipEventRecord(g_ev0, st);
  e = mlstm::launch_bwd(dt, b, st);
  if (g_ev1) (void)hipEventRecord(g_ev1, st);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t retention_chunkwise_bwd_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk, mlstm_dtype dt) {
  BwdPlan bp;
  if (plan_bwd(B, H, T, d_k, d_v, 1, chunk, dt, &bp, true) != MLSTM_OK) return 0;
  return bp.bytes;
}

int retention_chunkwise_bwd(int B, int H, int T, int d_k, int d_v, int chunk, mlstm_dtype dt, const void* q,
                            const void* k, const void* v, const float* gamma, const float* S0, const void* dout,
                            const float* dS_T, void* dq, void* dk, void* dv, float* dS0, void* workspace,
                            size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  const int rc = plan_bwd(B, H, T, d_k, d_v, 1, chunk, dt, &bp, true);
  if (rc != MLSTM_OK) return rc;
  if (!q || !k || !v || !dout) return fail(MLSTM_E_NULL, "q, k, v and dout are required");
  if (!dq || !dk || !dv) return fail(MLSTM_E_NULL, "dq, dk and dv are required");
  if (!workspace) return fail(MLSTM_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", bp.bytes);
  if (workspace_bytes < bp.bytes)
    return fail(MLSTM_E_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, bp.bytes);
  if ((size_t)workspace & 255) return fail(MLSTM_E_WORKSPACE, "workspace must be 256-byte aligned");
  const Plan& pl = bp.fwd;
  char* ws = static_cast<char*>(workspace);
  mlstm::ChunkParams p{};  // the forward's state passes only
  p.B = B;
  p.H = H;
  p.T = T;
  p.DV = d_v;
  p.q = q;
  p.k = k;
  p.v = v;
  p.ret_gamma = gamma;
  p.has_init = S0 ? 1 : 0;
  p.C0 = S0;
  p.h = nullptr;
  p.NC = pl.NC;
  p.G = pl.G;
  p.NS = pl.NS;
  p.nslices = pl.nslices;
  p.ws_state = reinterpret_cast<float*>(ws);
  p.ws_scal = reinterpret_cast<float*>(ws + pl.off_scal);
  p.ws_min = reinterpret_cast<float*>(ws + pl.off_min);
  const size_t gsz = align256((size_t)B * H * pl.NC * pl.L * sizeof(float));
  p.ws_ga = reinterpret_cast<float*>(ws + pl.off_g);
  p.ws_gg = reinterpret_cast<float*>(ws + pl.off_g + gsz);
  p.ws_gb = reinterpret_cast<float*>(ws + pl.off_g + 2 * gsz);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = pl.var.launch(p, st, nullptr, nullptr);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  mlstm::BwdParams b{};
  b.B = B;
  b.H = H;
  b.T = T;
  b.DQK = d_k;
  b.DV = d_v;
  b.NC = pl.NC;
  b.G = pl.G;
  b.NS = pl.NS;
  b.NB = 1;
  b.ret = 1;
  b.sc_nst = pl.nstate;
  b.q = q;
  b.k = k;
  b.v = v;
  b.dh = dout;
  b.has_init = p.has_init;
  b.sc_state = p.ws_state;
  b.sc_min = p.ws_min;
  b.ws_state = reinterpret_cast<float*>(ws + bp.off_cst);
  b.ws_min = reinterpret_cast<float*>(ws + bp.off_cmin);
  b.ws_ga = p.ws_ga;
  b.ws_gg = p.ws_gg;
  b.ws_gb = p.ws_gb;
  b.wsPt = ws + bp.off_Pt;
  b.wsDt = ws + bp.off_Dt;
  b.ws_rden = reinterpret_cast<float*>(ws + bp.off_rden);
  b.ws_dz = reinterpret_cast<float*>(ws + bp.off_dz);
  b.ws_dbias = reinterpret_cast<float*>(ws + bp.off_db);
  b.ws_ctot = reinterpret_cast<float*>(ws + bp.off_dbh);
  b.ws_U = reinterpret_cast<float*>(ws + bp.off_U);
  b.ws_qdq = reinterpret_cast<float*>(ws + bp.off_qdq);
  b.ws_kdki = reinterpret_cast<float*>(ws + bp.off_kdki);
  b.ws_kdk = reinterpret_cast<float*>(ws + bp.off_kdk);
  b.NSEG = (int)bp.nseg;
  b.ws_carry = bp.nseg ? reinterpret_cast<float*>(ws + bp.off_carry) : nullptr;
  b.ws_segdec = bp.nseg ? reinterpret_cast<float*>(ws + bp.off_segdec) : nullptr;
  b.ws_rdec = bp.nseg ? reinterpret_cast<float*>(ws + bp.off_rdec) : nullptr;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dC0 = dS0;
  b.dCT = dS_T;  // retention has no gates: the walk needs no final-state dot product
  if (g_ev0) (void)hipEventRecord(g_ev0, st);
  e = mlstm::launch_bwd(dt, b, st);
  if (g_ev1) (void)hipEventRecord(g_ev1, st);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int mlstm_abi_version(void) { return MLSTM_ABI_VERSION; }

const char* mlstm_last_error(void) { return g_err; }

int mlstm_set_profile_events(void* ev_start, void* ev_stop) {
  if ((ev_start == nullptr) != (ev_stop == nullptr))
    return fail(MLSTM_E_NULL, "give both events or neither");
  g_ev0 = static_cast<hipEvent_t>(ev_start);
  g_ev1 = static_cast<hipEvent_t>(ev_stop);
  return ok();
}

size_t mlstm_chunkwise_workspace_bytes(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk,
                                       mlstm_dtype dt) {
  Plan pl;
  if (plan_chunkwise(B, H, T, d_qk, d_v, num_blocks, chunk, dt, false, &pl) != MLSTM_OK) return 0;
  return pl.bytes;
}

size_t retention_chunkwise_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk, mlstm_dtype dt) {
  Plan pl;
  if (plan_chunkwise(B, H, T, d_k, d_v, 1, chunk, dt, true, &pl) != MLSTM_OK) return 0;
  return pl.bytes;
}

int mlstm_chunkwise_fwd(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk, mlstm_dtype dt,
                        const void* q, const void* k, const void* v, const void* i_pre, const void* f_pre,
                        const void* o_pre, const float* norm_bias, const float* C0, const float* n0,
                        const float* m0, float* C_out, float* n_out, float* m_out, void* h, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return mlstm_chunkwise_fwd_ex(B, H, T, d_qk, d_v, num_blocks, chunk, dt, MLSTM_NORM_VECTOR, q, k, v, i_pre,
                                f_pre, o_pre, norm_bias, C0, n0, m0, C_out, n_out, m_out, h, workspace,
                                workspace_bytes, stream);
}

int mlstm_chunkwise_fwd_ex(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk, mlstm_dtype dt,
                           int norm_mode, const void* q, const void* k, const void* v, const void* i_pre,
                           const void* f_pre, const void* o_pre, const float* norm_bias, const float* C0,
                           const float* n0, const float* m0, float* C_out, float* n_out, float* m_out, void* h,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return chunkwise_fwd_impl(B, H, T, d_qk, d_v, num_blocks, chunk, dt, norm_mode, q, k, v, i_pre, f_pre, o_pre,
                            norm_bias, C0, n0, m0, C_out, n_out, m_out, h, workspace, workspace_bytes, stream,
                            false);
}

int mlstm_chunkwise_fwd_noalloc(int B, int H, int T, int d_qk, int d_v, int num_blocks, int chunk, mlstm_dtype dt,
                                int norm_mode, const void* q, const void* k, const void* v, const void* i_pre,
                                const void* f_pre, const void* o_pre, const float* norm_bias, const float* C0,
                                const float* n0, const float* m0, float* C_out, float* n_out, float* m_out,
                                void* h, void* stream) {
  return chunkwise_fwd_impl(B, H, T, d_qk, d_v, num_blocks, chunk, dt, norm_mode, q, k, v, i_pre, f_pre, o_pre,
                            norm_bias, C0, n0, m0, C_out, n_out, m_out, h, nullptr, 0, stream, true);
}

size_t mlstm_noalloc_scratch_bytes(void) { return kScratchBytes; }


int retention_chunkwise_fwd(int B, int H, int T, int d_k, int d_v, int chunk, mlstm_dtype dt, const void* q,
                            const void* k, const void* v, const float* gamma, const float* S0, float* S_out,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  const int rc = plan_chunkwise(B, H, T, d_k, d_v, 1, chunk, dt, true, &pl);
  if (rc != MLSTM_OK) return rc;
  if (!q || !k || !v || !out) return fail(MLSTM_E_NULL, "q, k, v and out are required");
  mlstm::ChunkParams p{};
  p.B = B;
  p.H = H;
  p.T = T;
  p.DV = d_v;
  p.q = q;
  p.k = k;
  p.v = v;
  p.ret_gamma = gamma;
  p.has_init = S0 ? 1 : 0;
  p.C0 = S0;
  p.h = out;
  p.C_out = S_out;
  return launch(pl, p, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Group-norm plan: the retention plan; a head wider than the fused variant's
// work-group (d_v = nslices x W) adds an fp32 [B*H*T][d_v] array of
// unnormalised outputs after the retention workspace.
int plan_groupnorm(int B, int H, int T, int d_k, int d_v, int chunk, mlstm_dtype dt, Plan* pl,
                   size_t* gn_off) {
  const int rc = plan_chunkwise(B, H, T, d_k, d_v, 1, chunk, dt, true, pl);
  if (rc != MLSTM_OK) return rc;
  mlstm::ChunkVariant gv;
  if (!mlstm::find_retention_groupnorm_variant(dt, d_k, chunk, &gv) || d_v % gv.w)
    return fail(MLSTM_E_UNSUPPORTED, "group norm needs d_v a multiple of %d for d_k=%d (got d_v=%d)",
                mlstm::find_retention_groupnorm_variant(dt, d_k, chunk, &gv) ? gv.w : 0, d_k, d_v);
  pl->var.launch = gv.launch;  // same plan as without the norm
  if ((long long)B * H * T >= (1LL << 33))
    return fail(MLSTM_E_SHAPE, "B * H * T = %lld output rows is too many for the group norm",
                (long long)B * H * T);
  *gn_off = 0;
  if (d_v > gv.w) {
    *gn_off = pl->bytes;
    pl->bytes += align256((size_t)B * H * T * d_v * sizeof(float));
  }
  return MLSTM_OK;
}

}  // namespace

extern "C" {

size_t retention_chunkwise_groupnorm_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk,
                                                     mlstm_dtype dt) {
  Plan pl;
  size_t gn_off;
  if (plan_groupnorm(B, H, T, d_k, d_v, chunk, dt, &pl, &gn_off) != MLSTM_OK) return 0;
  return pl.bytes;
}

int retention_chunkwise_groupnorm_fwd(int B, int H, int T, int d_k, int d_v, int chunk, mlstm_dtype dt,
                                      const void* q, const void* k, const void* v, const float* gamma,
                                      const float* S0, float* S_out, const float* gn_weight,
                                      const float* gn_bias, float gn_eps, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  Plan pl;
  size_t gn_off;
  const int rc = plan_groupnorm(B, H, T, d_k, d_v, chunk, dt, &pl, &gn_off);
  if (rc != MLSTM_OK) return rc;
  if (!(gn_eps > 0.f)) return fail(MLSTM_E_SHAPE, "gn_eps must be positive (got %g)", (double)gn_eps);
  if (!q || !k || !v || !out) return fail(MLSTM_E_NULL, "q, k, v and out are required");
  mlstm::ChunkParams p{};
  p.B = B;
  p.H = H;
  p.T = T;
  p.DV = d_v;
  p.q = q;
  p.k = k;
  p.v = v;
  p.ret_gamma = gamma;
  p.has_init = S0 ? 1 : 0;
  p.C0 = S0;
  p.h = out;
  p.C_out = S_out;
  p.gn_w = gn_weight;
  p.gn_b = gn_bias;
  p.gn_eps = gn_eps;
  p.gn_ws = gn_off ? reinterpret_cast<float*>(static_cast<char*>(workspace) + gn_off) : nullptr;
  return launch(pl, p, workspace, workspace_bytes, stream);
}

int mlstm_step(int B, int H, int d_qk, int d_v, int num_blocks, mlstm_dtype dt, const void* q, const void* k,
               const void* v, const void* i_pre, const void* f_pre, const void* o_pre, const float* norm_bias,
               float* C, float* n, float* m, void* h, void* stream) {
  return mlstm_step_ex(B, H, d_qk, d_v, num_blocks, dt, MLSTM_NORM_VECTOR, q, k, v, i_pre, f_pre, o_pre,
                       norm_bias, C, n, m, h, stream);
}

int mlstm_step_ex(int B, int H, int d_qk, int d_v, int num_blocks, mlstm_dtype dt, int norm_mode, const void* q,
                  const void* k, const void* v, const void* i_pre, const void* f_pre, const void* o_pre,
                  const float* norm_bias, float* C, float* n, float* m, void* h, void* stream) {
  if (norm_mode != MLSTM_NORM_VECTOR && norm_mode != MLSTM_NORM_SCALAR && norm_mode != MLSTM_NORM_BLOCK)
    return fail(MLSTM_E_UNSUPPORTED, "unknown norm_mode %d", norm_mode);
  if (norm_mode == MLSTM_NORM_BLOCK && num_blocks > 8)
    return fail(MLSTM_E_UNSUPPORTED, "per-block normaliser decode supports at most 8 blocks (got %d)", num_blocks);
  if (dt != MLSTM_F32 && dt != MLSTM_BF16) return fail(MLSTM_E_DTYPE, "unknown dtype %d", dt);
  if (B < 1 || H < 1 || d_qk < 1 || d_v < 1 || num_blocks < 1)
    return fail(MLSTM_E_SHAPE, "sizes must be positive");
  if (d_qk % num_blocks || d_v % num_blocks)
    return fail(MLSTM_E_SHAPE, "d_qk=%d and d_v=%d must be multiples of num_blocks=%d", d_qk, d_v,
                num_blocks);
  if ((long long)B * H >= (1LL << 24)) return fail(MLSTM_E_SHAPE, "B * H too large");
  if (!mlstm::step_supported(d_qk, d_v, num_blocks))
    return fail(MLSTM_E_UNSUPPORTED, "no step kernel for d_qk=%d d_v=%d num_blocks=%d", d_qk, d_v, num_blocks);
  if (!q || !k || !v || !i_pre || !f_pre || !C || !n || !m || !h)
    return fail(MLSTM_E_NULL, "q, k, v, i_pre, f_pre, C, n, m and h are required");
  mlstm::StepParams p{};
  p.B = B;
  p.H = H;
  p.DQK = d_qk;
  p.DV = d_v;
  p.NB = num_blocks;
  p.q = q;
  p.k = k;
  p.v = v;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.o_pre = o_pre;
  p.bias = norm_bias;
  p.C = C;
  p.n = n;
  p.m = m;
  p.h = h;
  const hipError_t e = mlstm::launch_step(dt, p, static_cast<hipStream_t>(stream), norm_mode);
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int retention_step(int B, int H, int d_k, int d_v, mlstm_dtype dt, const void* q, const void* k, const void* v,
                   const float* gamma, float* S, void* out, void* stream) {
  if (dt != MLSTM_F32 && dt != MLSTM_BF16) return fail(MLSTM_E_DTYPE, "unknown dtype %d", dt);
  if (B < 1 || H < 1 || d_k < 1 || d_v < 1) return fail(MLSTM_E_SHAPE, "sizes must be positive");
  if ((long long)B * H >= (1LL << 24)) return fail(MLSTM_E_SHAPE, "B * H too large");
  if (!mlstm::step_supported(d_k, d_v, 1))
    return fail(MLSTM_E_UNSUPPORTED, "no retention step kernel for d_k=%d d_v=%d", d_k, d_v);
  if (!q || !k || !v || !S || !out) return fail(MLSTM_E_NULL, "q, k, v, S and out are required");
  mlstm::StepParams p{};
  p.B = B;
  p.H = H;
  p.DQK = d_k;
  p.DV = d_v;
  p.NB = 1;
  p.q = q;
  p.k = k;
  p.v = v;
  p.C = S;
  p.h = out;
  p.gamma = gamma;
  const hipError_t e = mlstm::launch_retention_step(dt, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLSTM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
