#!/usr/bin/env python
"""Benchmark of the gated delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one chunked prefill of the long-context workload: B=1, H=6,
d_k = d_v = 256, T = 65,536 tokens, bf16 q/k/v, fp32 gates and state, chunk
64, inputs resident in HBM, as one whole-prefill call with an execution
context created once beforehand (gdn_chunk_prefill_ctx: the library pipelines
segments of its three stages over the context's streams).  ``value`` is prefill tokens/s
of those steps.  The same work is then run stage by stage (per-chunk
preparation, the sequential state chain as one launch over all chunks, the
per-chunk outputs), each stage timed with HIP events on the stream it runs
on, for the breakdown and the roofline.
The decode workload (256 sequences x 6 heads, d = 256, 128 consecutive
single-token steps, fp32 state updated in place) is timed in the same run and
reported under "decode" (state GB/s).

Roofline: the dominant kernel of the step is the state chain.  Its achieved
rate is its algorithmic flops per launch over its average launch duration
(the one-launch form of the stage-by-stage run):
4 d_k d_v flops per token and head (Delta = U - W S^T, which the bf16 chain
forms as U - T' (K S^T), and the rank-C state update, 2 d_k d_v each), the
dense contraction it performs; peak is dense bf16 MFMA.  Whole-path figures use F_tok = H [6 d_k d_v + C (3 d_k + 2 d_v)
+ C^2 / 3] flops per token and the minimum HBM traffic (q, k, v, o in bf16,
g and beta in fp32).

cpu_baseline: the fp64 oracle (plain sequential recurrence, one thread per
(sequence, head) chain, threads = min(chains, host cores)) run on the host on
the same 64K-token inputs, timed around its computation only; plus one head's
chain on a single thread for a per-core figure.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (H=6,d=256,T=64K) + decode state GB/s; % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 (matrix cores; the vector rate is the same)

T, H, DK, DV, C = 65536, 6, 256, 256, 64
DEC_N = 256


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_chain_per_token():
    """State chain: Delta = U - W S^T and S <- decay S + K^T Delta, per token (all heads)."""
    return H * 4 * DK * DV


def flops_path_per_token():
    """Whole prefill path per token (all heads), the algorithmic count."""
    return H * (6 * DK * DV + C * (3 * DK + 2 * DV) + C * C / 3.0)


def prefill_min_bytes():
    """q, k, v, o in bf16, g and beta in fp32, initial and final fp32 state."""
    return T * H * (2 * DK + 2 * DV) * 2 + T * H * 8 + 2 * H * DK * DV * 4


def decode_bytes_per_step(N=DEC_N):
    # state read + write (fp32), q, k, v read and o written (bf16), g and beta (fp32)
    return 2 * N * H * DK * DV * 4 + N * H * (2 * DK + 2 * DV) * 2 + 2 * N * H * 4


def decode_bytes_per_step_dv(N, dv):
    """Decode bytes per step at value width dv: state read and written (fp32),
    q, k read and v, o (bf16), g and beta (fp32)."""
    return 2 * N * H * DK * dv * 4 + N * H * (2 * DK + 2 * dv) * 2 + 2 * N * H * 4


def kernel_sources_digest():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "hybrid_linear_attention_delta_amd", "csrc")
    for fn in sorted(os.listdir(d)):
        if fn.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(d, fn), "rb") as f:
                h.update(fn.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE,
    scaled by the copy-kernel calibration), valid only while the kernel sources
    are unchanged since the counters were taken; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("sources_digest") != kernel_sources_digest():
        return None
    ent = d.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def bench_prefill(torch, gdn, synth, steps, warmup, ctx):
    dev = torch.device("cuda:0")
    log(f"[bench] generating prefill inputs T={T} H={H} d={DK} bf16")
    inp = synth.prefill_inputs(T, H, DK, DV, "bf16", seed=synth.seed_for("prefill64k"))
    q = synth.to_torch(inp.q, dev, bf16=True)
    k = synth.to_torch(inp.k, dev, bf16=True)
    v = synth.to_torch(inp.v, dev, bf16=True)
    g = synth.to_torch(inp.g, dev)
    beta = synth.to_torch(inp.beta, dev)
    o = torch.empty((T, H, DV), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((1, H, DV, DK), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_size(T, 1, H, DK, DV, C), dtype=torch.uint8, device=dev)
    log(f"[bench] workspace {ws.numel() / 2**20:.0f} MiB")

    def run(st):
        gdn.chunk_prefill(q, k, v, g, beta, chunk=C, out=o, final_state=fs, workspace=ws, stages=st, ctx=ctx)

    # --- the step as a caller runs it: one whole-prefill call (the library
    #     pipelines its stages over streams internally)
    for _ in range(warmup):
        run(gdn.STAGE_ALL)
    torch.cuda.synchronize()
    log(f"[bench] prefill warmup done ({warmup} steps)")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        run(gdn.STAGE_ALL)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t0.elapsed_time(t1)

    # --- the same work stage by stage, each stage timed with events on the
    #     stream it runs on (the chain here is one launch over all chunks)
    stages = (gdn.STAGE_PREPARE, gdn.STAGE_PROPAGATE, gdn.STAGE_OUTPUT)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    for st in stages:
        run(st)
    torch.cuda.synchronize()
    for i in range(steps):
        for j, st in enumerate(stages):
            evs[i][j].record()
            run(st)
        evs[i][len(stages)].record()
    torch.cuda.synchronize()
    stage_ms = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(len(stages))]
    log(f"[bench] prefill {steps} steps: {total_ms / steps:.3f} ms/step; wall {wall / steps * 1e3:.3f} ms/step; "
        f"stage by stage: prepare {stage_ms[0]:.3f}, chain {stage_ms[1]:.3f}, output {stage_ms[2]:.3f} "
        f"(sum {sum(stage_ms):.3f})")

    # --- the same prefill with the gated RMSNorm read-out (App. A.3 Eq. 20)
    #     fused into its output stage
    z, w = synth.norm_inputs((T, H, DV), "bf16", synth.seed_for("prefill64k"))
    zt = synth.to_torch(z, dev, bf16=True)
    wt = synth.to_torch(w, dev)
    gated = lambda: gdn.chunk_prefill(q, k, v, g, beta, chunk=C, out=o, final_state=fs, workspace=ws, gate=zt,
                                      norm_weight=wt, ctx=ctx)
    for _ in range(max(1, warmup)):
        gated()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        gated()
    t1.record()
    torch.cuda.synchronize()
    gated_ms = t0.elapsed_time(t1) / steps
    log(f"[bench] gated prefill {steps} steps: {gated_ms:.3f} ms/step")

    # --- the whole-prefill call captured once in a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(gdn.STAGE_ALL)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    graph_ms = t0.elapsed_time(t1) / steps
    log(f"[bench] prefill replayed from a HIP graph: {graph_ms:.3f} ms/step")
    del graph  # release the graph (and its references to the context's streams) before the context
    torch.cuda.synchronize()
    return dict(ms_per_step=total_ms / steps, wall_ms_per_step=wall * 1e3 / steps, prepare_ms=stage_ms[0],
                chain_ms=stage_ms[1], output_ms=stage_ms[2], staged_ms=sum(stage_ms), gated_ms=gated_ms,
                graph_ms=graph_ms, inputs=inp)


def bench_decode(torch, gdn, synth, n_steps, warmup=3):
    dev = torch.device("cuda:0")
    seed = synth.seed_for("decode")
    log(f"[bench] generating decode inputs N={DEC_N} H={H} d={DK}, {n_steps} steps")
    state = torch.from_numpy(synth.decode_state(DEC_N, H, DK, DV, seed)).to(dev)
    per_step = []
    for s in range(n_steps):
        qn, kn, vn, gn, bn = synth.decode_step_inputs(DEC_N, H, DK, DV, "bf16", seed, s)
        per_step.append((synth.to_torch(qn, dev, bf16=True), synth.to_torch(kn, dev, bf16=True),
                         synth.to_torch(vn, dev, bf16=True), synth.to_torch(gn, dev), synth.to_torch(bn, dev)))
    o = torch.empty((DEC_N, H, DV), dtype=torch.bfloat16, device=dev)
    scratch = state.clone()
    for s in range(warmup):
        gdn.decode_step(*per_step[s % n_steps], scratch, out=o)
    del scratch
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    evs[0].record()
    for s in range(n_steps):
        gdn.decode_step(*per_step[s], state, out=o)
        evs[s + 1].record()
    torch.cuda.synchronize()
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(n_steps)]
    total = evs[0].elapsed_time(evs[-1])
    ms = total / n_steps
    times.sort()
    med = times[len(times) // 2]
    log(f"[bench] decode {n_steps} steps: mean {ms * 1e3:.1f} us/step, median {med * 1e3:.1f} us/step")
    # the same steps with the gated RMSNorm read-out (its second small kernel)
    z, w = synth.norm_inputs((DEC_N, H, DV), "bf16", seed)
    zt, wt = synth.to_torch(z, dev, bf16=True), synth.to_torch(w, dev)
    evs[0].record()
    for s in range(n_steps):
        gdn.decode_step(*per_step[s], state, out=o, gate=zt, norm_weight=wt)
    evs[1].record()
    torch.cuda.synchronize()
    gated = evs[0].elapsed_time(evs[1]) / n_steps
    log(f"[bench] gated decode {n_steps} steps: mean {gated * 1e3:.1f} us/step")
    # the same n_steps launches captured once in a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for s in range(n_steps):
                gdn.decode_step(*per_step[s], state, out=o)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    evs[0].record()
    graph.replay()
    evs[1].record()
    torch.cuda.synchronize()
    graphed = evs[0].elapsed_time(evs[1]) / n_steps
    log(f"[bench] decode {n_steps} steps in one HIP graph: {graphed * 1e3:.1f} us/step")
    del graph
    torch.cuda.synchronize()
    # d_v = 512 (the pages' value width): twice the state per sequence and head
    st5 = torch.from_numpy(synth.decode_state(DEC_N, H, DK, 2 * DV, seed)).to(dev)
    qn, kn, vn, gn, bn = synth.decode_step_inputs(DEC_N, H, DK, 2 * DV, "bf16", seed, 0)
    a5 = (synth.to_torch(qn, dev, bf16=True), synth.to_torch(kn, dev, bf16=True), synth.to_torch(vn, dev, bf16=True),
          synth.to_torch(gn, dev), synth.to_torch(bn, dev))
    o5 = torch.empty((DEC_N, H, 2 * DV), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        gdn.decode_step(*a5, st5, out=o5)
    torch.cuda.synchronize()
    evs[0].record()
    for _ in range(32):
        gdn.decode_step(*a5, st5, out=o5)
    evs[1].record()
    torch.cuda.synchronize()
    dv512 = evs[0].elapsed_time(evs[1]) / 32
    log(f"[bench] decode d_v=512: {dv512 * 1e3:.1f} us/step")
    del st5
    return dict(ms_per_step=ms, median_ms=med, gated_ms=gated, graph_ms=graphed, dv512_ms=dv512)


def bench_prefill_other(torch, gdn, synth, steps, warmup, ctx):
    """The other prefill workloads, timed as whole-prefill calls: 8K tokens
    (B=1, H=6, d=256, bf16), 64K tokens at d_v = 512, and the packed 2M-token
    batch (16 sequences, log-uniform lengths in [4K, 512K]) with a full-size
    workspace and with one bounded to 8 GiB (the chunks then run in windows)."""
    dev = torch.device("cuda:0")
    res = {}
    inp = synth.prefill_inputs(8192, H, DK, DV, "bf16", seed=synth.seed_for("prefill8k"))
    q, k, v = (synth.to_torch(x, dev, bf16=True) for x in (inp.q, inp.k, inp.v))
    g, beta = synth.to_torch(inp.g, dev), synth.to_torch(inp.beta, dev)
    cases = [("prefill_8k", (q, k, v, g, beta), None, None, None)]
    # d_v = 2 d_k = 512, the value width of the pages' GDN layer (64K tokens)
    inp5 = synth.prefill_inputs(T, H, DK, 2 * DV, "bf16", seed=synth.seed_for("prefill64k"))
    cases.append(("prefill_64k_dv512", tuple(synth.to_torch(x, dev, bf16=True) for x in (inp5.q, inp5.k, inp5.v))
                  + (synth.to_torch(inp5.g, dev), synth.to_torch(inp5.beta, dev)), None, None, None))
    del inp5
    lengths = synth.varlen_lengths(synth.seed_for("varlen2m"))
    log(f"[bench] generating the 2M-token packed batch (lengths {list(map(int, lengths))})")
    vq, vk, vv, vg, vb, cu = synth.varlen_torch_inputs(lengths, H, DK, DV, synth.seed_for("varlen2m"), dev)
    cu_host = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cases.append(("varlen_2m", (vq, vk, vv, vg, vb), cu_host, lengths, None))
    cases.append(("varlen_2m_workspace_8GiB", (vq, vk, vv, vg, vb), cu_host, lengths, 8 << 30))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    for name, (a, b, c, d, e), cuh, lens, ws_cap in cases:
        Tn, N, dvn = a.shape[0], (1 if cuh is None else len(lens)), c.shape[2]
        o = torch.empty((Tn, H, dvn), dtype=torch.bfloat16, device=dev)
        fs = torch.empty((N, H, dvn, DK), dtype=torch.float32, device=dev)
        need = gdn.prefill_workspace_size(Tn, N, H, DK, dvn, C)
        ws_bytes = need if ws_cap is None else min(need, ws_cap)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        cu_arg = None if cuh is None else torch.from_numpy(cuh)
        run = lambda: gdn.chunk_prefill(a, b, c, d, e, cu_seqlens=cu_arg, chunk=C, out=o, final_state=fs,
                                        workspace=ws, ctx=ctx)
        n_steps = steps if cuh is None else max(2, steps // 3)
        for _ in range(max(1, warmup)):
            run()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(n_steps):
            run()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / n_steps
        f_tok = H * (6 * DK * dvn + C * (3 * DK + 2 * dvn) + C * C / 3.0)
        ent = {"tokens": int(Tn), "d_v": int(dvn), "ms_per_step": ms, "tokens_per_s": Tn / (ms / 1e3),
               "workspace_GiB": ws_bytes / 2**30, "full_workspace_GiB": need / 2**30,
               "mfma_frac": f_tok * Tn / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
               "min_traffic_hbm_frac": Tn * H * ((2 * DK + 2 * dvn) * 2 + 8) / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
        if lens is not None:
            ent["lengths"] = [int(x) for x in lens]
        res[name] = ent
        log(f"[bench] {name}: {ms:.3f} ms/step, {ent['tokens_per_s'] / 1e6:.1f} M tokens/s")
        del o, fs, ws
    return res


def frontend_bytes(tokens):
    """Front end, algorithmic HBM bytes: the q, k, v projections read and the
    convolved q, k, v written (bf16), a and b read and g, beta written (fp32),
    the taps read once."""
    ctot = H * (2 * DK + DV)
    return 2 * tokens * ctot * 2 + 4 * tokens * H * 4 + ctot * 4 * 4


def bench_frontend(torch, gdn, synth, steps, warmup, ctx):
    """The front end (App. A.3: 4-tap causal conv + SiLU on q, k, v and the gate
    math) over the 64K-token workload, alone and followed by the prefill; and
    its decode form for the 256-sequence decode batch."""
    dev = torch.device("cuda:0")
    log(f"[bench] generating front-end inputs T={T} H={H} d={DK} bf16")
    f = synth.frontend_inputs(T, H, DK, DV, "bf16", seed=synth.seed_for("prefill64k"))
    xq = synth.to_torch(f.xq, dev, bf16=True).view(T, H, DK)
    xk = synth.to_torch(f.xk, dev, bf16=True).view(T, H, DK)
    xv = synth.to_torch(f.xv, dev, bf16=True).view(T, H, DV)
    w, a_, b_, al, db = (synth.to_torch(x, dev) for x in (f.conv_weight, f.a, f.b, f.A_log, f.dt_bias))
    o = torch.empty((T, H, DV), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((1, H, DV, DK), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_size(T, 1, H, DK, DV, C), dtype=torch.uint8, device=dev)
    fo = (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv),
          torch.empty((T, H), dtype=torch.float32, device=dev), torch.empty((T, H), dtype=torch.float32, device=dev))
    front = lambda: gdn.frontend_prefill(xq, xk, xv, w, a_, b_, al, db, return_conv_state=False, out=fo)

    def both():
        q, k, v, g, beta, _ = front()
        gdn.chunk_prefill(q, k, v, g, beta, chunk=C, out=o, final_state=fs, workspace=ws, ctx=ctx)

    fused = lambda: gdn.chunk_prefill_frontend(xq, xk, xv, w, a_, b_, al, db, return_conv_state=False, out=o,
                                               final_state=fs, workspace=ws, ctx=ctx)

    res = {}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    for name, fn in (("frontend", front), ("frontend_then_prefill", both), ("fused", fused)):
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        res[name] = t0.elapsed_time(t1) / steps
    log(f"[bench] front end {res['frontend'] * 1e3:.1f} us; front end + prefill {res['frontend_then_prefill']:.3f} ms; "
        f"front end folded into the prefill {res['fused']:.3f} ms")

    fd = synth.frontend_inputs(DEC_N, H, DK, DV, "bf16", seed=synth.seed_for("decode"), with_state=True,
                               N=DEC_N)
    st = synth.to_torch(fd.conv_state, dev, bf16=True)
    dq = synth.to_torch(fd.xq, dev, bf16=True).view(DEC_N, H, DK)
    dk_ = synth.to_torch(fd.xk, dev, bf16=True).view(DEC_N, H, DK)
    dv_ = synth.to_torch(fd.xv, dev, bf16=True).view(DEC_N, H, DV)
    dw, da, dbb, dal, ddb = (synth.to_torch(x, dev) for x in (fd.conv_weight, fd.a, fd.b, fd.A_log, fd.dt_bias))
    n_dec = 128
    do = (torch.empty_like(dq), torch.empty_like(dk_), torch.empty_like(dv_),
          torch.empty((DEC_N, H), dtype=torch.float32, device=dev),
          torch.empty((DEC_N, H), dtype=torch.float32, device=dev))
    gdn.frontend_decode(dq, dk_, dv_, dw, da, dbb, dal, ddb, st, out=do)  # checks the arguments once
    # then the C entry point itself, arguments marshalled once (as a serving loop
    # would): the per-call Python checks cost more than this small kernel
    lib = gdn.load_library()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [P(dq), P(dk_), P(dv_), P(dw), P(da), P(dbb), P(dal), P(ddb), P(st), DEC_N, H, DK, DV, gdn.GDN_BF16,
            *[P(t) for t in do], ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)]
    for _ in range(max(1, warmup)):
        assert lib.gdn_frontend_decode(*args) == 0
    torch.cuda.synchronize()
    t0.record()
    for _ in range(n_dec):
        lib.gdn_frontend_decode(*args)
    t1.record()
    torch.cuda.synchronize()
    res["decode_frontend"] = t0.elapsed_time(t1) / n_dec
    log(f"[bench] decode front end {res['decode_frontend'] * 1e3:.1f} us/step")
    return res


def flops_backward_per_token():
    """Chunked backward per token (all heads), algorithmic: the d_k d_v
    contractions (forward chain 2, reverse chain 3, per-chunk dQ, dK, dW 3, each
    2 d_k d_v flops), the C d terms (K K^T, Q K^T, W, dPG K, dPG^T Q, dT, T^T dW,
    dA-terms of dK: 18 C d_k; U, P^T dO, dP, dT, dV: 10 C d_v) and the C x C ones."""
    return H * (16 * DK * DV + 18 * C * DK + 10 * C * DV + 4 * C * C)


def bench_backward(torch, gdn, synth, inp, steps, warmup):
    """Gradients of the 64K-token prefill (gdn_chunk_prefill_backward): all
    launches are on the current stream, timed with events around whole calls."""
    dev = torch.device("cuda:0")
    t = lambda a, b=False: synth.to_torch(a, dev, bf16=b)
    q, k, v, g, beta = t(inp.q, True), t(inp.k, True), t(inp.v, True), t(inp.g), t(inp.beta)
    do, ds = synth.backward_cotangents(T, H, DK, DV, 1, "bf16", synth.seed_for("prefill64k"))
    do, ds = t(do, True), t(ds)
    ws = torch.empty(gdn.prefill_backward_workspace_size(T, 1, H, DK, DV), dtype=torch.uint8, device=dev)
    log(f"[bench] backward: workspace {ws.numel() / 2**30:.1f} GiB")
    run = lambda: gdn.chunk_prefill_backward(q, k, v, g, beta, do, dstate=ds, workspace=ws)
    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    log(f"[bench] backward {ms:.2f} ms per 64K-token step")
    return ms


def host_cores():
    """CPU cores this process may run on (its affinity set), and os.cpu_count()."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return usable, os.cpu_count() or usable


def cpu_baseline(inp, max_threads=16):
    """The fp64 oracle on the host, timed around its computation only.

    Leg 1: the whole 64K-token workload, one thread per (sequence, head) chain,
    threads = min(chains, usable cores, 16) (16 = one GPU's share of the host).
    Leg 2: one head's chain (the first) on one thread, for a per-core figure.
    fp64 work: 7 d_k d_v flops per token and head (the retrieval dot product,
    the decay-plus-write update and the read, 2 + 3 + 2 per state element)."""
    import oracle

    usable, count = host_cores()
    chains = H
    threads = max(1, min(chains, usable, max_threads))
    flop_tok_head = 7.0 * DK * DV
    log(f"[bench] cpu baseline: fp64 oracle on {T} tokens x {H} heads, {threads} threads "
        f"(usable cores {usable}, os.cpu_count {count})")
    tm = {}
    oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, bf16=True, n_threads=threads, timing=tm)
    dt = tm["seconds"]
    tm1 = {}
    oracle.prefill(inp.q[:, :1], inp.k[:, :1], inp.v[:, :1], inp.g[:, :1], inp.beta[:, :1], bf16=True, n_threads=1,
                   timing=tm1)
    dt1 = tm1["seconds"]
    log(f"[bench] cpu baseline {dt:.2f} s ({threads} threads); one head on one thread {dt1:.2f} s")
    return dict(value=T / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"full prefill workload: {T} tokens x {H} heads, d={DK}, fp64 sequential recurrence, "
                       f"{threads} threads (one per head chain), {dt:.2f} s of computation; per-core leg: head 0 "
                       f"alone on one thread, {dt1:.2f} s",
                nproc=usable, os_cpu_count=count, threads=threads, seconds=dt,
                gflops_fp64=flop_tok_head * T * H / dt / 1e9,
                single_thread={"tokens_per_s_per_core": T / (H * dt1), "seconds_one_head": dt1,
                               "gflops_fp64": flop_tok_head * T / dt1 / 1e9},
                flops_per_token_head=flop_tok_head)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the 8K and 2M-token prefill figures")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the mixer shards by head, state row or sequence without collectives). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from hybrid_linear_attention_delta_amd import gdn, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (cuda:0)", file=sys.stderr)
        sys.exit(2)
    gdn.load_library()
    ctx = gdn.Context()  # streams and events of the overlapped prefill, created once
    pre = bench_prefill(torch, gdn, synth, a.steps, a.warmup, ctx)
    dec = None if a.no_decode else bench_decode(torch, gdn, synth, a.decode_steps)
    fe = bench_frontend(torch, gdn, synth, a.steps, a.warmup, ctx)
    other = None if a.no_other else bench_prefill_other(torch, gdn, synth, a.steps, a.warmup, ctx)
    bwd_ms = None if a.no_backward else bench_backward(torch, gdn, synth, pre["inputs"], min(a.steps, 3), 1)
    torch.cuda.synchronize()
    ctx.close()  # every HIP object the library made is released before the process ends

    tok_s = T / (pre["ms_per_step"] / 1e3)
    chain_flops = flops_chain_per_token() * T
    chain_tflops = chain_flops / (pre["chain_ms"] / 1e3) / 1e12
    path_tflops = flops_path_per_token() * T / (pre["ms_per_step"] / 1e3) / 1e12
    path_gbps = prefill_min_bytes() / (pre["ms_per_step"] / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gdn_chunk_prefill B=1 H={H} d_k={DK} d_v={DV} T={T} chunk={C} bf16",
                   "global_batch": 1, "seq_len": T, "heads": H, "d_k": DK, "d_v": DV, "chunk": C,
                   "parallelism": "single-gpu"},
        "roofline": {
            "kernel": "chain_kr_kernel (sequential state chain, one launch over all chunks)",
            "bound": "mfma",
            "achieved": chain_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": chain_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic_from_profiles("chain_kr_kernel"),
            "avg_launch_ms": pre["chain_ms"],
            "algorithmic_flops_per_launch": chain_flops,
        },
        "prefill": {
            "tokens_per_s": tok_s,
            "prepare_ms": pre["prepare_ms"],
            "chain_ms": pre["chain_ms"],
            "output_ms": pre["output_ms"],
            "stage_by_stage_ms": pre["staged_ms"],
            "hip_graph_ms_per_step": pre["graph_ms"],
            "wall_ms_per_step": pre["wall_ms_per_step"],
            "path_tflops": path_tflops,
            "path_mfma_frac": path_tflops / PEAK_BF16_TFLOPS,
            "path_min_traffic_GBps": path_gbps,
            "path_hbm_frac": path_gbps / PEAK_HBM_GBPS,
            "algorithmic_flops_per_token": flops_path_per_token(),
            "traffic": {"intra_kernel": traffic_from_profiles("intra_kernel"),
                        "output_kernel": traffic_from_profiles("output_kernel")},
            "gated_rmsnorm": {"ms_per_step": pre["gated_ms"], "tokens_per_s": T / (pre["gated_ms"] / 1e3),
                              "overhead_ms": pre["gated_ms"] - pre["ms_per_step"]},
        },
    }
    if dec is not None:
        b = decode_bytes_per_step()
        gbps = b / (dec["ms_per_step"] / 1e3) / 1e9
        state_gbps = 2 * DEC_N * H * DK * DV * 4 / (dec["ms_per_step"] / 1e3) / 1e9
        out["decode"] = {
            "workload": f"gdn_decode_step N={DEC_N} H={H} d={DK} bf16 q/k/v, fp32 state, "
                        f"{a.decode_steps} steps",
            "ms_per_step": dec["ms_per_step"],
            "median_ms_per_step": dec["median_ms"],
            "gated_rmsnorm_ms_per_step": dec["gated_ms"],
            "hip_graph_ms_per_step": dec["graph_ms"],
            "dv512": {"ms_per_step": dec["dv512_ms"],
                      "hbm_frac": decode_bytes_per_step_dv(DEC_N, 2 * DV) / (dec["dv512_ms"] / 1e3) / 1e9
                      / PEAK_HBM_GBPS},
            "tokens_per_s": DEC_N / (dec["ms_per_step"] / 1e3),
            "state_GBps": state_gbps,
            "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                         "traffic": traffic_from_profiles("decode_kernel"),
                         "algorithmic_bytes_per_launch": b},
        }
    if other is not None:
        out["prefill"]["other_workloads"] = other
    fb = frontend_bytes(T)
    ctot = H * (2 * DK + DV)
    dec_fb = 2 * DEC_N * ctot * 2 + 2 * 3 * DEC_N * ctot * 2 + 4 * DEC_N * H * 4 + ctot * 16
    out["frontend"] = {
        "workload": f"gdn_frontend_prefill T={T} H={H} d={DK} bf16 (4-tap conv + SiLU on q, k, v; gates)",
        "ms_per_step": fe["frontend"],
        "frontend_then_prefill_ms": fe["frontend_then_prefill"],
        "frontend_then_prefill_tokens_per_s": T / (fe["frontend_then_prefill"] / 1e3),
        "fused_frontend_prefill_ms": fe["fused"],
        "fused_frontend_prefill_tokens_per_s": T / (fe["fused"] / 1e3),
        "fused_overhead_over_prefill_ms": fe["fused"] - pre["ms_per_step"],
        "roofline": {"kernel": "conv_silu_kernel", "bound": "hbm", "achieved": fb / (fe["frontend"] / 1e3) / 1e9,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": fb / (fe["frontend"] / 1e3) / 1e9 / PEAK_HBM_GBPS,
                     "traffic": traffic_from_profiles("conv_silu_kernel"), "algorithmic_bytes_per_launch": fb},
        "decode_frontend_ms_per_step": fe["decode_frontend"],
        "decode_frontend_GBps": dec_fb / (fe["decode_frontend"] / 1e3) / 1e9,
    }
    if bwd_ms is not None:
        bf = flops_backward_per_token() * T
        tf = bf / (bwd_ms / 1e3) / 1e12
        out["backward"] = {
            "workload": f"gdn_chunk_prefill_backward B=1 H={H} d_k={DK} d_v={DV} T={T} bf16 inputs, fp32 gradients",
            "ms_per_step": bwd_ms,
            "tokens_per_s": T / (bwd_ms / 1e3),
            "algorithmic_flops_per_token": flops_backward_per_token(),
            "roofline": {"kernel": "whole backward (fp32 contractions on the fp32 matrix cores)", "bound": "mfma",
                         "achieved": tf, "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_F32_TFLOPS},
        }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pre["inputs"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
