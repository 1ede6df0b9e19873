#!/usr/bin/env python3
"""Benchmark of the mLSTM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Step = one chunkwise prefill (mlstm_chunkwise_fwd) of the xLSTM-7B-shaped
layer: B=1, 8 heads, d_qk=256, d_v=512, T=8192, chunk 64, bf16 q/k/v/gates,
fp32 state, inputs resident in HBM.  K steps are timed between two device
synchronisations; four input sets are rotated so that successive steps do not
find their inputs in the 256 MB Infinity Cache.  ``value`` is prefill
tokens/s = B*T*K / wall time.

The decode part (``decode``) runs the xLSTM-7B-shaped fused decode step:
B=256, 8 heads, fp32 state [256,8,256,512] (1 GiB) updated in place, 128 steps
with a fresh bf16 token per step; it reports achieved HBM GB/s.

``variants`` times the other chunkwise workloads through the same kernels
(RetNet retention B=8 H=4 d=64 T=2048, also with its per-head group norm
fused; xLSTM-v2 block-diagonal B=4 H=4 d=64 nb=2 T=65536, also with per-block
denominators; the 7B prefill with an output gate, and with the scalar
normaliser), the retention decode step on the RetNet shape, and the backward
passes of the 7B prefill, the RetNet and the xLSTM-v2 block-diagonal
workloads: tokens/s per call and its algorithmic bytes against HBM
(``backward`` runs the backward passes alone).

``roofline`` is measured live over the whole prefill call: two HIP events on
the launch stream around the K timed calls give the GPU time per call, and
achieved = algorithmic bytes (or flops) per call / that time.  Its
``main_kernel`` part gives the same for the per-chunk output kernel alone,
from events the library records right before and after it
(mlstm_set_profile_events).  ``traffic`` sums the committed rocprofv3
FETCH_SIZE / WRITE_SIZE readings of the call's kernels.  The variant and
decode legs run before the prefill leg (the decode leg right before it), so
that the prefill's warm-up and timed steps find the GPU at its steady
clocks.  ``cpu_baseline`` times the fp64 CPU oracle on the host cores on a
bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mLSTM prefill tokens/s (7B-shape, T=8192) + decode-step HBM GB/s, % roofline"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA


def prefill_work(B, H, T, dqk, dv, L=64):
    """Algorithmic bytes and flops of one chunkwise forward: every input read
    once, h written once, final state written once; flops with dense LxL
    intra-chunk tiles (2L(d_qk+d_v) + 4 d_qk d_v per token and head)."""
    e = 2  # bf16
    byts = B * H * T * (2 * dqk + dv) * e + B * H * T * 2 * e + B * H * T * dv * e
    byts += B * H * (dqk * dv + dqk + 1) * 4
    flops = B * H * T * (2 * L * (dqk + dv) + 4 * dqk * dv)
    return byts, flops


def decode_work(B, H, dqk, dv):
    """Algorithmic bytes per decode step: fp32 C, n, m read and written once,
    one bf16 token (q, k, v, i, f) read, h written."""
    byts = 2 * B * H * (dqk * dv + dqk + 1) * 4
    byts += B * H * (2 * dqk + dv + 2) * 2 + B * H * dv * 2
    flops = B * H * (5 * dqk * dv + 4 * dqk)
    return byts, flops


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_recurrent_sequence_mlstm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the launches of one prefill call, in order
PREFILL_KERNELS = ("local_state_kernel", "superchunk_scan_kernel", "chunk_kernel_ws")


def traffic_from_profiles(kernels, sha):
    """HBM bytes of one launch of each named kernel, summed, from the
    committed rocprofv3 counter summary; None when any is missing or its
    source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    tot = 0.0
    for k in kernels:
        rec = recs.get(k)
        if not rec or rec.get("source_sha") != sha:
            return None
        tot += rec.get("bytes_per_launch")
    return tot


def workload_traffic(name):
    """HBM bytes of one whole call of a variant workload (every launch of it)
    from the committed rocprofv3 counter summary, taken in a run of that
    workload alone; None when missing or when the kernels' sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get("workloads", {}).get(name)
    except (OSError, ValueError):
        return None
    if name.endswith("_backward"):
        sha = source_sha("backward.hip", "chunkwise.hip", "common.h")
    elif "decode" in name:
        sha = source_sha("step.hip", "common.h")
    else:
        sha = source_sha("chunkwise.hip", "common.h")
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_call")


class _KernelEvents:
    """Pairs of HIP events for the library's profile hooks, created without
    the system-scope fence (hipEventDisableSystemFence): a timing event with
    that fence costs several microseconds of idle GPU per record here, which
    would show up in the timed steps.  They still order with the stream."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.pairs = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                e = ctypes.c_void_p()
                rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.FLAGS))
                if rc != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
                pair.append(e)
            self.pairs.append(tuple(pair))

    def mean_ms(self):
        tot = 0.0
        for a, b in self.pairs:
            ms = self.ct.c_float()
            rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
            if rc != 0:
                raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
            tot += ms.value
        return tot / len(self.pairs)

    def close(self):
        for pair in self.pairs:
            for e in pair:
                self.hip.hipEventDestroy(e)


def prepare_prefill(torch, mlstm, x, dev):
    """Device buffers of the prefill leg: four input sets with the same
    values, their outputs, the final state and the workspace."""
    spec = dict(B=1, H=8, T=8192, dqk=256, dv=512)
    sets = [x.to(dev)]
    for _ in range(3):  # distinct buffers with the same values
        g = sets[0]
        sets.append(type(g)(*(None if t is None else t.clone() for t in
                              (g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias)), g.num_blocks, g.chunk))
    B, H, T, dqk, dv = (spec[k] for k in ("B", "H", "T", "dqk", "dv"))
    hs = [torch.empty(B, H, T, dv, dtype=torch.bfloat16, device=dev) for _ in sets]
    st = (torch.empty(B, H, 1, dqk, dv, device=dev), torch.empty(B, H, dqk, device=dev),
          torch.empty(B, H, device=dev))
    ws = torch.empty(mlstm.chunkwise_workspace_bytes(B, H, T, dqk, dv), dtype=torch.uint8, device=dev)
    return dict(spec=spec, sets=sets, hs=hs, st=st, ws=ws)


def prefill_events(torch, K):
    """The prefill leg's events: K pairs around the main kernel and the two
    around the timed steps.  Made ahead of time (before the decode leg in
    the full run): creating them takes the host longer than the warm-up's GPU
    work, and the idle GPU would lower its clocks right before the timed
    steps."""
    return dict(kev=_KernelEvents(K), e0=torch.cuda.Event(enable_timing=True), e1=torch.cuda.Event(enable_timing=True))


def bench_prefill(torch, mlstm, prep, args, dev, events=None):
    spec, sets, hs, st, ws = (prep[k] for k in ("spec", "sets", "hs", "st", "ws"))
    B, H, T, dqk, dv = (spec[k] for k in ("B", "H", "T", "dqk", "dv"))

    def call(i):
        g = sets[i % len(sets)]
        mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, h=hs[i % len(sets)],
                            state_out=st, workspace=ws)

    K = args.steps
    ev = events or prefill_events(torch, K)
    kev, e0, e1 = ev["kev"], ev["e0"], ev["e1"]  # kev: around the main kernel, in a second loop of K calls
    L = mlstm.lib()
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / K
    # the main kernel's time: the same K calls again, each with the library's
    # events around pass 3 (kept out of the timed steps: a pair of event
    # records costs about 2.5 us of GPU time per call)
    for i in range(K):
        L.mlstm_set_profile_events(*kev.pairs[i])
        call(i)
    torch.cuda.synchronize()
    mlstm.set_profile_events()
    kern_ms = kev.mean_ms()
    kev.close()
    byts, flops = prefill_work(B, H, T, dqk, dv)
    return dict(spec=spec, wall=wall, K=K, step_ms=step_ms, kern_ms=kern_ms, bytes=byts, flops=flops,
                tokens=B * T)


def bench_decode(torch, mlstm, workload, args, dev, finish_later=False):
    """The decode leg; with finish_later, returns a function that reads its
    events out afterwards, so that the next leg starts on a busy GPU."""
    d = workload("xlstm7b_decode_B256", steps=args.decode_steps).to(dev)
    S, B, H, dqk = d.q.shape
    dv = d.v.shape[-1]
    C = torch.zeros(B, H, 1, dqk, dv, device=dev)
    n = torch.zeros(B, H, dqk, device=dev)
    m = torch.zeros(B, H, device=dev)
    h = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)

    def call(s):
        mlstm.step(d.q[s], d.k[s], d.v[s], d.i_pre[s], d.f_pre[s], C, n, m, bias=d.bias, h=h)

    ev = _KernelEvents(S)  # around every step (both launches of a step); made before the warm-up
    for s in range(min(args.warmup, S)):
        call(s)
    for t in (C, n, m):
        t.zero_()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rec = ev.hip.hipEventRecord
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(S):
        rec(ev.pairs[s][0], ev.ct.c_void_p(stream))
        call(s)
        rec(ev.pairs[s][1], ev.ct.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def finish():
        step_ms = ev.mean_ms()
        ev.close()
        byts, flops = decode_work(B, H, dqk, dv)
        return dict(B=B, H=H, dqk=dqk, dv=dv, S=S, wall=wall, step_ms=step_ms, bytes=byts, flops=flops)

    return finish if finish_later else finish()


def retention_work(B, H, T, dk, dv, L=64):
    """Algorithmic bytes and flops of one retention forward: q, k, v read
    once, the output written once, the final fp32 state written once."""
    byts = B * H * T * (2 * dk + 2 * dv) * 2 + B * H * dk * dv * 4
    flops = B * H * T * (2 * L * (dk + dv) + 4 * dk * dv)
    return byts, flops


def backward_work(B, H, T, dqk, dv, L=64):
    """Algorithmic bytes and flops of one chunkwise backward: q, k, v, dh and
    the gates read once, dq, dk, dv and the gate gradients written once, the
    fp32 initial-state gradient written once; flops of the products the
    chunkwise backward performs, the recompute of the chunk states included:
    12 d_qk d_v + 6 L (d_qk + d_v) per token and head (six state-sized
    products, three L x L x d_qk and three L x L x d_v ones)."""
    e = 2
    byts = B * H * T * (2 * dqk + 2 * dv + 2) * e + B * H * T * (2 * dqk + dv + 2) * e
    byts += B * H * (dqk * dv + dqk) * 4
    flops = B * H * T * (12 * dqk * dv + 6 * L * (dqk + dv))
    return byts, flops


def retention_backward_work(B, H, T, dk, dv, L=64):
    """Algorithmic bytes and flops of one retention backward: q, k, v and dout
    read once, dq, dk, dv written once, the fp32 initial-state gradient
    written once; flops of the chunkwise products, the state recompute
    included: 10 d_k d_v + 2L (3 d_k + 2 d_v) per token and head."""
    byts = B * H * T * (2 * dk + 2 * dv) * 2 + B * H * T * (2 * dk + dv) * 2 + B * H * dk * dv * 4
    flops = B * H * T * (10 * dk * dv + 2 * L * (3 * dk + 2 * dv))
    return byts, flops


def bench_variants(torch, mlstm, workload, args, dev, only_backward=False):
    """The retention and block-diagonal workloads through the same chunkwise
    kernels: fence-free events around every call (all launches of it) and
    the library's events around its main kernel.  Enough distinct input sets
    rotate that the inputs do not stay in the 256 MB Infinity Cache.
    ``args.variant`` (a list of workload names, or None for all) limits the
    leg to those workloads, so that a counter run sees one workload only."""
    out = []
    pick = getattr(args, "variant", None)

    def want(*names):
        return pick is None or any(n in pick for n in names)
    L = mlstm.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def timed(call, nsets, K, W, chunkwise=True):
        # chunkwise calls also record the library's events around pass 3;
        # the events exist before the warm-up (see bench_prefill)
        ev = _KernelEvents(K)
        kev = _KernelEvents(K) if chunkwise else None
        rec = ev.hip.hipEventRecord
        for i in range(W):
            call(i % nsets)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            if kev:
                L.mlstm_set_profile_events(*kev.pairs[i])
            rec(ev.pairs[i][0], ev.ct.c_void_p(stream))
            call(i % nsets)
            rec(ev.pairs[i][1], ev.ct.c_void_p(stream))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mlstm.set_profile_events()
        r = dict(call_ms=ev.mean_ms(), kernel_ms=kev.mean_ms() if kev else ev.mean_ms(), wall_ms=wall / K * 1e3)
        ev.close()
        if kev:
            kev.close()
        return r

    from linear_recurrent_sequence_mlstm_amd.workloads import grad_output
    nb_steps = max(1, args.variant_steps // 4)  # timed calls of each backward workload
    if want("xlstm7b_prefill_T8192_backward"):
        # backward pass of the 7B prefill workload (state passes recomputed,
        # gradients of all inputs and of the initial state); the library's events
        # bracket its six backward kernels
        x = workload("xlstm7b_prefill_T8192")
        B, H, T, dqk = x.q.shape
        dv = x.v.shape[-1]
        sets = [x.to(dev), x.to(dev)]
        dhs = [grad_output((B, H, T, dv), seed=7000 + i).to(dev) for i in range(len(sets))]
        ws = torch.empty(mlstm.lib().mlstm_chunkwise_bwd_workspace_bytes(B, H, T, dqk, dv, 1, 64, mlstm.BF16),
                         dtype=torch.uint8, device=dev)

        def call_bwd(i):
            g = sets[i]
            mlstm.chunkwise_bwd(g.q, g.k, g.v, g.i_pre, g.f_pre, dhs[i], None, g.bias, workspace=ws)

        r = timed(call_bwd, len(sets), nb_steps, nb_steps)
        byts, flops = backward_work(B, H, T, dqk, dv)
        out.append(dict(workload="xlstm7b_prefill_T8192_backward", B=B, H=H, T=T, d_qk=dqk, d_v=dv, **r,
                        bytes=byts, flops=flops, tokens=B * T))
        del sets, dhs, ws

    if want("retnet_msr_T2048_backward"):
        # retention backward on the RetNet workload (B=8, H=4, d=64, T=2048)
        q, k, v = workload("retnet_msr_T2048")
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        rsets = [tuple(t.to(dev) for t in (q, k, v)) for _ in range(4)]
        douts = [grad_output((B, H, T, dv), seed=7100 + i, scale=1 / 8).to(dev) for i in range(len(rsets))]
        ws = torch.empty(mlstm.lib().retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, 64, mlstm.BF16),
                         dtype=torch.uint8, device=dev)
        r = timed(lambda i: mlstm.retention_chunkwise_bwd(*rsets[i], douts[i], workspace=ws), len(rsets),
                  args.variant_steps, args.variant_steps)
        byts, flops = retention_backward_work(B, H, T, dk, dv)
        out.append(dict(workload="retnet_msr_T2048_backward", B=B, H=H, T=T, d_k=dk, d_v=dv, **r, bytes=byts,
                        flops=flops, tokens=B * T))
        del rsets, douts, ws

    if want("xlstm2_blockdiag_T65536_backward"):
        # block-diagonal backward on the xLSTM-v2 workload (B=4, H=4, d=64, nb=2, T=65536)
        x = workload("xlstm2_blockdiag_T65536")
        B, H, T, dqk = x.q.shape
        dv = x.v.shape[-1]
        nb = x.num_blocks
        bsets = [x.to(dev), x.to(dev)]
        dhs = [grad_output((B, H, T, dv), seed=7200 + i).to(dev) for i in range(len(bsets))]
        ws = torch.empty(mlstm.lib().mlstm_chunkwise_bwd_workspace_bytes(B, H, T, dqk, dv, nb, 64, mlstm.BF16),
                         dtype=torch.uint8, device=dev)

        def call_bd(i):
            g = bsets[i]
            mlstm.chunkwise_bwd(g.q, g.k, g.v, g.i_pre, g.f_pre, dhs[i], g.o_pre, g.bias, workspace=ws,
                                num_blocks=nb)

        r = timed(call_bd, len(bsets), nb_steps, nb_steps)
        byts, flops = backward_work(B, H, T, dqk, dv)
        # block-diagonal: the six state-sized products are nb times smaller
        byts -= B * H * (dqk * dv - dqk * dv // nb) * 4
        flops -= B * H * T * 12 * (dqk * dv - dqk * dv // nb)
        out.append(dict(workload="xlstm2_blockdiag_T65536_backward", B=B, H=H, T=T, d_qk=dqk, d_v=dv, num_blocks=nb,
                        **r, bytes=byts, flops=flops, tokens=B * T))
        del bsets, dhs, ws
    if only_backward:
        return out

    if want("retnet_msr_T2048", "retnet_msr_T2048_groupnorm"):
        # RetNet multi-scale retention: B=8, H=4, d=64, T=2048 (34 MB per call)
        q, k, v = workload("retnet_msr_T2048")
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        sets = [tuple(t.to(dev) for t in (q, k, v)) for _ in range(8)]
        outs = [torch.empty(B, H, T, dv, dtype=q.dtype, device=dev) for _ in sets]
        S = torch.empty(B, H, dk, dv, device=dev)
        ws = torch.empty(mlstm.retention_workspace_bytes(B, H, T, dk, dv), dtype=torch.uint8, device=dev)
        byts, flops = retention_work(B, H, T, dk, dv)
        if want("retnet_msr_T2048"):
            r = timed(lambda i: mlstm.retention_chunkwise_fwd(*sets[i], out=outs[i], S_out=S, workspace=ws),
                      len(sets), args.variant_steps, args.variant_steps)
            out.append(dict(workload="retnet_msr_T2048", B=B, H=H, T=T, d_k=dk, d_v=dv, **r, bytes=byts,
                            flops=flops, tokens=B * T))
        # the same with the per-head group norm fused into the output write
        gw = torch.ones(H * dv, device=dev)
        gb = torch.zeros(H * dv, device=dev)
        if want("retnet_msr_T2048_groupnorm"):
            r = timed(lambda i: mlstm.retention_chunkwise_fwd(*sets[i], out=outs[i], S_out=S, workspace=ws,
                                                              groupnorm=(gw, gb, 1e-5)),
                      len(sets), args.variant_steps, args.variant_steps)
            out.append(dict(workload="retnet_msr_T2048_groupnorm", B=B, H=H, T=T, d_k=dk, d_v=dv, **r,
                            bytes=byts + 2 * H * dv * 4, flops=flops, tokens=B * T))
        del sets, outs, S, ws, gw, gb

    if want("retnet_msr_decode_B8"):
        # retention decode on the same workload: its first D tokens, one call
        # of retention_step each, state updated in place
        q, k, v = workload("retnet_msr_T2048")
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        D = min(128, T)
        toks = [tuple(t[:, :, s].contiguous().to(dev) for t in (q, k, v)) for s in range(D)]
        S = torch.zeros(B, H, dk, dv, device=dev)
        o = torch.empty(B, H, dv, dtype=q.dtype, device=dev)
        r = timed(lambda i: mlstm.retention_step(*toks[i], S, out=o), D, D, D, chunkwise=False)
        # the same D steps captured once in a HIP graph and replayed (what a
        # serving loop that captures its decode steps sees: no host enqueue per
        # step); GPU time per step over 5 replays
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(D):
                mlstm.retention_step(*toks[i], S, out=o)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        r["graph_ms_per_step"] = e0.elapsed_time(e1) / (5 * D)
        del graph
        byts = 2 * B * H * dk * dv * 4 + B * H * (2 * dk + 2 * dv) * 2
        out.append(dict(workload="retnet_msr_decode_B8", B=B, H=H, d_k=dk, d_v=dv, steps=D, **r, bytes=byts,
                        flops=B * H * 4 * dk * dv, tokens=B))
        del toks, S, o

    if want("xlstm7b_prefill_T8192_with_o", "xlstm7b_prefill_T8192_scalar_norm"):
        # the 7B prefill with an output gate o = sigmoid(o_pre) [B,H,T,d_v] read too
        x = workload("xlstm7b_prefill_T8192", with_o=True)
        B, H, T, dqk = x.q.shape
        dv = x.v.shape[-1]
        sets = [x.to(dev), x.to(dev)]
        hs = [torch.empty(B, H, T, dv, dtype=x.q.dtype, device=dev) for _ in sets]
        st = (torch.empty(B, H, 1, dqk, dv, device=dev), torch.empty(B, H, dqk, device=dev),
              torch.empty(B, H, device=dev))
        ws = torch.empty(mlstm.chunkwise_workspace_bytes(B, H, T, dqk, dv), dtype=torch.uint8, device=dev)

        def call_o(i):
            g = sets[i]
            mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, h=hs[i], state_out=st,
                                workspace=ws)

        if want("xlstm7b_prefill_T8192_with_o"):
            r = timed(call_o, len(sets), args.variant_steps, args.variant_steps)
            byts, flops = prefill_work(B, H, T, dqk, dv)
            byts += B * H * T * dv * 2
            out.append(dict(workload="xlstm7b_prefill_T8192_with_o", B=B, H=H, T=T, d_qk=dqk, d_v=dv, **r,
                            bytes=byts, flops=flops, tokens=B * T))

        # the same workload (no output gate) with the scalar normaliser reading
        st_s = (st[0], torch.empty(B, H, device=dev), st[2])

        def call_s(i):
            g = sets[i]
            mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, None, g.bias, h=hs[i], state_out=st_s, workspace=ws,
                                norm_mode="scalar")

        if want("xlstm7b_prefill_T8192_scalar_norm"):
            r = timed(call_s, len(sets), args.variant_steps, args.variant_steps)
            byts, flops = prefill_work(B, H, T, dqk, dv)
            out.append(dict(workload="xlstm7b_prefill_T8192_scalar_norm", B=B, H=H, T=T, d_qk=dqk, d_v=dv, **r,
                            bytes=byts - B * H * (dqk - 1) * 4, flops=flops, tokens=B * T))
        del sets, hs, st, st_s, ws

    if want("xlstm7b_prefill_T64_from_state"):
        # a short call: 64 tokens of the 7B head shape continuing from a
        # carried state (one superchunk, so one launch), state updated in place
        # into a second set of buffers
        x = workload("xlstm7b_prefill_T8192")
        T = 64
        B, H, _, dqk = x.q.shape
        dv = x.v.shape[-1]
        sl = [t[:, :, :T].contiguous().to(dev) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre)]
        g = torch.Generator().manual_seed(64)
        st0 = (torch.randn(B, H, 1, dqk, dv, generator=g).mul_(0.3).to(dev),
               torch.randn(B, H, dqk, generator=g).mul_(0.3).to(dev), torch.zeros(B, H, device=dev))
        st1 = tuple(torch.empty_like(t) for t in st0)
        h = torch.empty(B, H, T, dv, dtype=x.q.dtype, device=dev)
        ws = torch.empty(mlstm.chunkwise_workspace_bytes(B, H, T, dqk, dv), dtype=torch.uint8, device=dev)
        r = timed(lambda i: mlstm.chunkwise_fwd(*sl, None, None, state=st0, state_out=st1, h=h, workspace=ws),
                  1, args.variant_steps, args.variant_steps)
        byts, flops = prefill_work(B, H, T, dqk, dv)
        byts += B * H * (dqk * dv + dqk + 1) * 4  # the initial state read
        out.append(dict(workload="xlstm7b_prefill_T64_from_state", B=B, H=H, T=T, d_qk=dqk, d_v=dv, **r,
                        bytes=byts, flops=flops, tokens=B * T))
        del sl, st0, st1, h, ws

    if want("xlstm2_blockdiag_T65536", "xlstm2_blockdiag_T65536_block_norm"):
        # xLSTM-v2 block-diagonal: B=4, H=4, d=64, nb=2, T=65536 (541 MB per call)
        x = workload("xlstm2_blockdiag_T65536")
        B, H, T, dqk = x.q.shape
        dv = x.v.shape[-1]
        sets = [x.to(dev), x.to(dev)]
        hs = [torch.empty(B, H, T, dv, dtype=x.q.dtype, device=dev) for _ in sets]
        nb = x.num_blocks
        st = (torch.empty(B, H, nb, dqk // nb, dv // nb, device=dev), torch.empty(B, H, dqk, device=dev),
              torch.empty(B, H, device=dev))
        ws = torch.empty(mlstm.chunkwise_workspace_bytes(B, H, T, dqk, dv, nb), dtype=torch.uint8, device=dev)

        def call(i):
            g = sets[i]
            mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, num_blocks=nb, h=hs[i],
                                state_out=st, workspace=ws)

        byts, flops = prefill_work(B, H, T, dqk, dv)
        # block-diagonal: the state and its products are nb times smaller
        byts -= B * H * (dqk * dv - dqk * dv // nb) * 4
        flops -= B * H * T * 4 * (dqk * dv - dqk * dv // nb)
        if want("xlstm2_blockdiag_T65536"):
            r = timed(call, len(sets), args.variant_steps, args.variant_steps)
            out.append(dict(workload="xlstm2_blockdiag_T65536", B=B, H=H, T=T, d_qk=dqk, d_v=dv, num_blocks=nb, **r,
                            bytes=byts, flops=flops, tokens=B * T))

        # the same with one denominator per memory block
        def call_b(i):
            g = sets[i]
            mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, num_blocks=nb, h=hs[i],
                                state_out=st, workspace=ws, norm_mode="block")

        if want("xlstm2_blockdiag_T65536_block_norm"):
            r = timed(call_b, len(sets), args.variant_steps, args.variant_steps)
            out.append(dict(workload="xlstm2_blockdiag_T65536_block_norm", B=B, H=H, T=T, d_qk=dqk, d_v=dv,
                            num_blocks=nb, **r, bytes=byts, flops=flops, tokens=B * T))
    return out


def copy_calibration(torch, dev, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size (nbytes read, nbytes
    written per launch).  Its rocprofv3 FETCH_SIZE / WRITE_SIZE readings give
    the factors that turn those counters into HBM bytes for the kernels above."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return dict(bytes_read=nbytes, bytes_written=nbytes, ms=dt * 1e3, GBps=2 * nbytes / dt / 1e9)


def cpu_baseline(x, sample_tokens):
    """The fp64 oracle on the host cores: all 8 heads of the prefill workload
    (the same CPU tensors the GPU got) over its first ``sample_tokens`` tokens."""
    import oracle
    Ts = min(sample_tokens, x.q.shape[2])
    sl = lambda t: None if t is None else t[:, :, :Ts].contiguous()
    args = [sl(t) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre)]
    t0 = time.perf_counter()
    oracle.mlstm_fwd(*args)
    dt = time.perf_counter() - t0
    B, H = x.q.shape[:2]
    # the oracle runs one OpenMP thread per (batch, head): at most B*H of them
    threads = min(oracle.num_threads(), B * H)
    host = len(os.sched_getaffinity(0))
    return dict(value=B * Ts / dt, unit="tokens/s", cores=threads, host_cores=host, kind="oracle",
                sample="xlstm7b_prefill_T8192, B=%d, all %d heads, first %d of 8192 tokens, fp64, "
                       "%.1f s on %d threads (one per head) of %d host cores" % (B, H, Ts, dt, threads, host))


def variant_line(v):
    """One retention / block-diagonal / backward record: throughput of the
    whole call and the HBM and MFMA rooflines of its algorithmic work."""
    s = v["call_ms"] * 1e-3
    gbs = v["bytes"] / s / 1e9
    keep = {k: v[k] for k in v if k not in ("call_ms", "kernel_ms", "wall_ms", "bytes", "flops", "tokens")}
    traffic = workload_traffic(v["workload"])
    return dict(keep, value=v["tokens"] / s, unit="tokens/s", ms_per_call=v["call_ms"],
                wall_ms_per_call=v["wall_ms"], main_kernel_ms=v["kernel_ms"],
                roofline=dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                              traffic=traffic, kernel="whole call (all launches)",
                              mfma_frac=v["flops"] / s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                              algorithmic_bytes=v["bytes"], algorithmic_flops=v["flops"]))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant-steps", type=int, default=100,
                    help="timed calls of the retention and block-diagonal workloads (0: skip them)")
    ap.add_argument("--only", choices=("prefill", "decode", "copy", "variants", "backward"),
                    help="run one leg alone and print its raw figures (for profiler runs)")
    ap.add_argument("--variant", action="append",
                    help="with --only variants: run only this workload (repeatable; for counter runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the mLSTM heads shard across GPUs with no "
              "communication, so the per-GPU figure is the whole story; got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
    from linear_recurrent_sequence_mlstm_amd.workloads import workload

    dev = torch.device("cuda:0")
    if args.only:
        print("bench: only %s" % args.only, file=sys.stderr, flush=True)
        if args.only == "prefill":
            r = bench_prefill(torch, mlstm, prepare_prefill(torch, mlstm, workload("xlstm7b_prefill_T8192"), dev),
                              args, dev)
            r.pop("spec")
        elif args.only == "decode":
            r = bench_decode(torch, mlstm, workload, args, dev)
        elif args.only == "variants":
            r = dict(variants=bench_variants(torch, mlstm, workload, args, dev))
        elif args.only == "backward":
            r = dict(variants=bench_variants(torch, mlstm, workload, args, dev, only_backward=True))
        else:
            r = copy_calibration(torch, dev)
        print(json.dumps(dict(leg=args.only, **r)))
        return
    # The prefill's buffers and events are set up first and the decode leg (45
    # ms of continuous GPU work) runs right before the prefill leg, its events
    # read only afterwards, so that the prefill's warm-up and timed steps find
    # the GPU at its steady clocks: after a host-side pause of a few
    # milliseconds this GPU needs about 20 ms of work to return to them
    # (measured: pass 3 of the prefill takes about 15 % longer for its first 50
    # calls after a 1 s pause than after them).
    x = workload("xlstm7b_prefill_T8192")
    prep = prepare_prefill(torch, mlstm, x, dev)
    var = []
    if args.variant_steps > 0:
        print("bench: retention and block-diagonal workloads, %d calls each" % args.variant_steps,
              file=sys.stderr, flush=True)
        var = bench_variants(torch, mlstm, workload, args, dev)
    pf_events = prefill_events(torch, args.steps)
    print("bench: decode xlstm7b_decode_B256 steps=%d, then prefill xlstm7b_prefill_T8192 steps=%d warmup=%d"
          % (args.decode_steps, args.steps, args.warmup), file=sys.stderr, flush=True)
    dc_finish = bench_decode(torch, mlstm, workload, args, dev, finish_later=True)
    pf = bench_prefill(torch, mlstm, prep, args, dev, events=pf_events)
    dc = dc_finish()
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(x, args.cpu_sample_tokens)

    K = pf["K"]
    value = pf["tokens"] * K / pf["wall"]
    sha_cw = source_sha("chunkwise.hip", "common.h")
    sha_st = source_sha("step.hip", "common.h")
    # The headline roofline covers the whole prefill call (every launch of
    # it): algorithmic bytes and flops of one call over its GPU time per call.
    call_s = pf["step_ms"] * 1e-3
    roof = dict(bound="hbm", achieved=pf["bytes"] / call_s / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_from_profiles(PREFILL_KERNELS, sha_cw)
    roof["kernel"] = "whole prefill call (%s)" % ", ".join(PREFILL_KERNELS)
    roof["mfma_tflops"] = pf["flops"] / call_s / 1e12
    roof["mfma_frac"] = roof["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS
    roof["algorithmic_bytes"] = pf["bytes"]
    roof["algorithmic_flops"] = pf["flops"]
    roof["call_ms"] = pf["step_ms"]
    # the main (per-chunk output) kernel alone, timed by the library's events
    kern_s = pf["kern_ms"] * 1e-3
    roof["main_kernel"] = dict(kernel=PREFILL_KERNELS[-1], ms=pf["kern_ms"],
                               achieved_GBps=pf["bytes"] / kern_s / 1e9,
                               frac=pf["bytes"] / kern_s / 1e9 / HBM_PEAK_GBS,
                               mfma_frac=pf["flops"] / kern_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                               traffic=traffic_from_profiles((PREFILL_KERNELS[-1],), sha_cw))
    dk_s = dc["step_ms"] * 1e-3
    droof = dict(bound="hbm", achieved=dc["bytes"] / dk_s / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    droof["frac"] = droof["achieved"] / droof["peak"]
    droof["traffic"] = traffic_from_profiles(("step_kernel",), sha_st)
    droof["kernel"] = "step_kernel"
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": pf["wall"] / K * 1e3,
        "gpu_ms_per_step": pf["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "xlstm7b_prefill_T8192", "B": 1, "H": 8, "T": 8192, "d_qk": 256,
                   "d_v": 512, "chunk": 64, "state": "fp32", "input_sets_rotated": 4},
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": {
            "workload": "xlstm7b_decode_B256",
            "value": dc["bytes"] / dk_s / 1e9,
            "unit": "GB/s",
            "tokens_per_s": dc["B"] / dk_s,
            "ms_per_step": dc["step_ms"],
            "wall_ms_per_step": dc["wall"] / dc["S"] * 1e3,
            "steps": dc["S"],
            "roofline": droof,
        },
        "variants": [variant_line(v) for v in var],
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
