"""Benchmark: KDA chunkwise prefill (B=1, H=16, dk=dv=128, T=65536) and the
recurrent decode step (256 sequences x 16 heads, 1024 steps) on one MI355X.

One step = one kda_chunk_fwd over the whole 64K-token batch: every stage of
the prefill (cumulative decay, decayed Gram blocks, UT inverse, WY factors,
inter-chunk state propagation, output) runs inside that call.  Inputs are
drawn on the host, copied to HBM once, and are resident when timing starts.
Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-append] [--no-fused]
                    [--no-backward] [--no-cpu] [--calibrate-copy]

--calibrate-copy adds, before the timed region, one launch of the streaming
copy kernel (libkda_ceilings.so) of a known size (256 MiB read + 256 MiB
written): its FETCH_SIZE / WRITE_SIZE counters give the scale for the
operator's measured HBM traffic.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, vendor figure
# forward flops per token and head from the Kimi Linear review notes' complexity section,
# 6 d^2 + 3 C d + C^2 at d = 128, C = 64
PAGES_FLOPS_PER_TOKEN_HEAD = 6 * 128 * 128 + 3 * 64 * 128 + 64 * 64
METRIC = "KDA prefill tokens/s (H=16,d=128,T=64K) + decode step us/token, % roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_chunk_fwd_prefill_64k_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_alg_bytes(B, T, H, dk, dv, N, in_bytes=2, out_bytes=2, h0=True, hT=True, gate_width=None):
    """Algorithmic HBM bytes of one prefill: every input read once, every
    output written once, no intermediates.  gate_width: fp32 gate values per
    token and head (dk, or 1 for a scalar gate)."""
    th = B * T * H
    gw = dk if gate_width is None else gate_width
    per_th = (2 * dk + dv + 1) * in_bytes + gw * 4 + dv * out_bytes
    return th * per_th + (int(h0) + int(hT)) * N * H * dk * dv * 4


def decode_alg_bytes(N, H, dk, dv, in_bytes=2, out_bytes=2):
    nh = N * H
    return nh * (2 * dk * dv * 4 + (2 * dk + dv + 1) * in_bytes + dk * 4 + dv * out_bytes)


# sources no kernel of kda_chunk_fwd is built from (decode and append kernels, gradients, DPLR)
# the sources kda_chunk_fwd's kernels (segment table, prep, scans, combine) are built from
PREFILL_SOURCES = ("kda_prep.hip", "kda_scan.hip", "kda_segments.hip", "kda_mfma.h", "kda_device.h",
                   "kda_internal.h")


def source_digest():
    """sha256 over the HIP/C++ sources the prefill's kernels are built from: a
    stored traffic measurement is only reported while they are unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_52_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in PREFILL_SOURCES:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per kda_chunk_fwd call from the committed counter summary,
    or None when it was taken on different kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def settle(fn, ms=40.0):
    """Call fn until about ``ms`` of wall time has passed, synchronizing every few
    calls: the untimed warm-up of the secondary lines, by time rather than by
    count, so that the GPU has left its idle clocks (each line draws its inputs
    on the host first, and the GPU idles meanwhile) before their warm-up calls."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < 2 or (time.perf_counter() - t0) * 1e3 < ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_prefill(args, name="prefill_64k", calibrate=False, sweep=None, before=None, settle_ms=40.0):
    """Time kda_chunk_fwd on a named workload; ``prefill_64k_fused`` is the same
    problem handed over before the L2 norm and the gate activation, which the
    kernels then apply (the input transforms).  ``before`` runs once the inputs
    are on the GPU and before the warm-up calls: the main line measures the
    ceilings there, because a GPU that has been idle (here: while the host draws
    the inputs) raises its clocks over its first ~20 ms of load (64K prefill
    calls fall from 1.20 to 0.95 ms over the first 20), and the ceilings' copy
    and matrix-core loops are that much load."""
    import torch
    import gated_delta_rule_52_amd as kda
    from gated_delta_rule_52_amd.inputs import make_workload
    x = make_workload(name)
    tr = x.transforms()
    log(f"{name} drawn: B={x.B} T={x.T} H={x.H} dk={x.dk} dv={x.dv} transforms={tr}")
    dev = "cuda:0"
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    q, k, v, beta = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf)
    g, h0 = t(x.g, f32), t(x.h0, f32)
    hT = torch.empty_like(h0)
    o = torch.empty((x.B, x.T, x.H, x.dv), dtype=bf, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(q, v), dtype=torch.uint8, device=dev)
    step = lambda: kda.chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o,
                                 out_dtype=bf, workspace=ws, **tr)
    if before is not None:
        before()
    elif settle_ms:
        settle(step, settle_ms)
    if calibrate:
        # the streaming copy kernel of libkda_ceilings.so (not a runtime blit), so the counters see it
        lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_52_amd", "libkda_ceilings.so"))
        lib.kda_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                         ctypes.c_void_p]
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        assert lib.kda_ceiling_copy(a.data_ptr(), b.data_ptr(), 256 << 20, 0,
                                    torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        del a, b
        log("calibration copy (copy_kernel<false>): 268435456 B read, 268435456 B written")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the library launches on torch's current stream: events there bracket every kernel of a call
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    ms = float(ev[0].elapsed_time(ev[-1]) / args.steps)
    log(f"{'prefill' if name == 'prefill_64k' else name}: {ms:.3f} ms/step (events), median {np.median(per):.3f}, p10 {np.percentile(per, 10):.3f}, "
        f"p90 {np.percentile(per, 90):.3f}, wall {1e3 * wall / args.steps:.3f} ms/step")
    nbytes = prefill_alg_bytes(x.B, x.T, x.H, x.dk, x.dv, x.N)
    if sweep is not None:
        # the pages' operator sweep (batch 1, 16 heads, 2K..64K tokens): prefixes of the resident inputs
        for T in (2048, 4096, 8192, 16384, 32768):
            sl = lambda a: a[:, :T]
            o_t = o[:, :T]
            ws_t = torch.empty(kda.chunk_fwd_workspace_bytes(sl(q), v), dtype=torch.uint8, device=dev)
            call = lambda: kda.chunk_fwd(sl(q), sl(k), sl(v), sl(g), sl(beta), initial_state=h0, final_state=hT,
                                         o=o_t, out_dtype=bf, workspace=ws_t, **tr)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(10, 2 * args.steps * 65536 // T // 4)
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            sweep[T] = e0.elapsed_time(e1) / reps
            log(f"sweep T={T}: {sweep[T] * 1e3:.1f} us per call")
        sweep[x.T] = ms
    return x, ms, per, nbytes


def time_decode(args):
    """The decode workload, 1024 consecutive steps, two ways: in place (one
    state buffer of 256 MiB, as a serving cache updates it) and ping-pong
    (step s reads buffer s % 2 and writes the other: 512 MiB of state, twice
    the 256 MiB Infinity Cache, so the state streams from HBM)."""
    import torch
    from gated_delta_rule_52_amd import _lib
    from gated_delta_rule_52_amd.inputs import WORKLOADS, make_decode_state, decode_step_pool
    w = WORKLOADS["decode_256x16"]
    N, H, dk, dv, steps, pool = w["N"], w["H"], w["dk"], w["dv"], w["steps"], w["pool"]
    rng, S0 = make_decode_state(w["seed"], N, H, dk, dv, std=w["state_std"])
    P = decode_step_pool(rng, pool, N, H, dk, dv, in_dtype=w["in_dtype"], gscale=w["gscale"])
    dev = "cuda:0"
    bf, f32 = torch.bfloat16, torch.float32
    # every step reads its own inputs at its own offset
    idx = torch.arange(steps) % pool
    q = torch.from_numpy(P["q"]).to(dev).to(bf)[idx].contiguous()
    k = torch.from_numpy(P["k"]).to(dev).to(bf)[idx].contiguous()
    v = torch.from_numpy(P["v"]).to(dev).to(bf)[idx].contiguous()
    g = torch.from_numpy(P["g"]).to(dev)[idx].contiguous()
    beta = torch.from_numpy(P["beta"]).to(dev).to(bf)[idx].contiguous()
    S = [torch.from_numpy(S0).to(dev), torch.from_numpy(S0).to(dev)]
    o = torch.empty((steps, N, H, dv), dtype=bf, device=dev)
    lib = _lib.load()
    stream = torch.cuda.current_stream()

    def make_args(strm, ping_pong):
        keep = []
        for s in range(steps):
            a = _lib.RecurrentStepArgs()
            a.struct_size = ctypes.sizeof(_lib.RecurrentStepArgs)
            a.q, a.k, a.v = q[s].data_ptr(), k[s].data_ptr(), v[s].data_ptr()
            a.g, a.beta = g[s].data_ptr(), beta[s].data_ptr()
            if ping_pong:
                a.initial_state, a.final_state = S[s % 2].data_ptr(), S[(s + 1) % 2].data_ptr()
            else:
                a.initial_state = a.final_state = S[0].data_ptr()
            a.o = o[s].data_ptr()
            a.N, a.H, a.dk, a.dv, a.scale = N, H, dk, dv, 1.0
            a.in_dtype = a.out_dtype = _lib.KDA_DTYPE_BF16
            a.stream = strm.cuda_stream
            keep.append(a)
        return keep

    def run_all(args):
        for a in args:
            rc = lib.kda_recurrent_step(ctypes.byref(a))
            if rc:
                _lib.check(rc)

    res = {}
    for mode in ("ping_pong", "in_place"):
        refs = make_args(stream, mode == "ping_pong")
        run_all(refs)  # warm-up pass (advances the state; timing does not depend on values)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_all(refs)
        e1.record(stream)
        torch.cuda.synchronize()
        res[mode] = 1e3 * e0.elapsed_time(e1) / steps
        log(f"decode ({mode}): {res[mode]:.2f} us/step over {steps} steps")
    # the in-place steps captured once into a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(graph, stream=side):
        run_all(make_args(torch.cuda.current_stream(), False))
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us_graph = 1e3 * e0.elapsed_time(e1) / steps
    log(f"decode (in place) under a graph: {us_graph:.2f} us/step")
    return dict(N=N, H=H, dk=dk, dv=dv, steps=steps, us=res["ping_pong"], us_in_place=res["in_place"],
                us_graph=us_graph, nbytes=decode_alg_bytes(N, H, dk, dv))


def time_prefill_own(args, name, cold_flush_bytes=512 << 20):
    """kda_chunk_fwd on a named workload with its own recipe (its seed, its
    initial state or none, final states written, bf16 o), ms per call: warm
    (calls back to back) and cold (each call after writing a 512 MiB buffer,
    which evicts the inputs from the 256 MiB Infinity Cache)."""
    import torch
    import gated_delta_rule_52_amd as kda
    from gated_delta_rule_52_amd.inputs import make_workload
    x = make_workload(name)
    dev = "cuda:0"
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    q, k, v, beta, g = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf), t(x.g, f32)
    h0 = None if x.h0 is None else t(x.h0, f32)
    cu = None if x.cu_seqlens is None else t(x.cu_seqlens, torch.int32)
    hT = torch.empty((x.N, x.H, x.dk, x.dv), dtype=f32, device=dev)
    o = torch.empty((x.B, x.T, x.H, x.dv), dtype=bf, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(q, v, cu), dtype=torch.uint8, device=dev)
    call = lambda: kda.chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o, cu_seqlens=cu,
                                 out_dtype=bf, workspace=ws)
    stream = torch.cuda.current_stream()
    settle(call)
    for _ in range(max(args.warmup, 3)):
        call()
    torch.cuda.synchronize()
    reps = max(args.steps, 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) / reps
    flush = torch.empty(cold_flush_bytes // 4, dtype=f32, device=dev)
    cold = []
    for _ in range(reps):
        flush.fill_(1.0)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    nbytes = prefill_alg_bytes(1, x.B * x.T, x.H, x.dk, x.dv, x.N, h0=h0 is not None, hT=True)
    log(f"{name}: {x.B * x.T} tokens, warm {warm * 1e3:.1f} us, cold median {np.median(cold) * 1e3:.1f} us")
    return x, warm, float(np.median(cold)), nbytes


def append_alg_bytes(N, T, H, dk, dv, in_bytes=2, out_bytes=2):
    nh = N * H
    return nh * (2 * dk * dv * 4 + T * ((2 * dk + dv + 1) * in_bytes + dk * 4 + dv * out_bytes))


def time_append(args):
    """Short appends: 256 sequences x 16 heads each take 64 new tokens from a
    cached state; the fused recurrent path and the chunkwise path side by side."""
    import torch
    import gated_delta_rule_52_amd as kda
    from gated_delta_rule_52_amd.inputs import make_workload
    x = make_workload("append_256x16x64")
    dev = "cuda:0"
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    q, k, v, beta = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf)
    g, h0 = t(x.g, f32), t(x.h0, f32)
    hT = torch.empty_like(h0)
    o = torch.empty((x.B, x.T, x.H, x.dv), dtype=bf, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(q, v), dtype=torch.uint8, device=dev)
    paths = {
        "recurrent_fwd": lambda: kda.recurrent_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o,
                                                   out_dtype=bf),
        "recurrent_fwd_token_by_token": lambda: kda.recurrent_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT,
                                                                  o=o, out_dtype=bf, token_by_token=True),
        "chunk_fwd": lambda: kda.chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o,
                                           out_dtype=bf, workspace=ws),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in paths.items():
        settle(fn)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = 1e3 * e0.elapsed_time(e1) / 10
        log(f"append_256x16x64 {name}: {res[name]:.1f} us per call")
    return x, res, append_alg_bytes(x.B, x.T, x.H, x.dk, x.dv)


def time_append_grid():
    """Which path serves a short append faster: sequences x new tokens (16
    heads, d = 128, bf16, cached fp32 states), us per call of each."""
    import torch
    import gated_delta_rule_52_amd as kda
    from gated_delta_rule_52_amd.inputs import make_prefill
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt: torch.from_numpy(a).to("cuda:0").to(dt)
    stream = torch.cuda.current_stream()
    grid = {}
    for N in (1, 16, 256):
        for T in (1, 16, 64):
            x = make_prefill(7, N, T, 16, 128, 128, h0_std=0.02)
            q, k, v, beta = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf)
            g, h0 = t(x.g, f32), t(x.h0, f32)
            hT = torch.empty_like(h0)
            o = torch.empty((N, T, 16, 128), dtype=bf, device="cuda:0")
            ws = torch.empty(kda.chunk_fwd_workspace_bytes(q, v), dtype=torch.uint8, device="cuda:0")
            row = {}
            for name, fn in (("chunk_fwd", lambda: kda.chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT,
                                                                  o=o, out_dtype=bf, workspace=ws)),
                             ("recurrent_fwd", lambda: kda.recurrent_fwd(q, k, v, g, beta, initial_state=h0,
                                                                          final_state=hT, o=o, out_dtype=bf)),
                             ("token_by_token", lambda: kda.recurrent_fwd(q, k, v, g, beta, initial_state=h0,
                                                                           final_state=hT, o=o, out_dtype=bf,
                                                                           token_by_token=True))):
                settle(fn, 20.0)
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(20):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                row[name] = 1e3 * e0.elapsed_time(e1) / 20
            grid[f"{N}x{T}"] = row
            log(f"append grid N={N} T={T}: chunk_fwd {row['chunk_fwd']:.1f} us, recurrent_fwd {row['recurrent_fwd']:.1f} us "
                f"(token by token {row['token_by_token']:.1f} us)")
    return grid


FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (FMA = 2 flops)


def backward_alg_flops(tokens, H, dk, dv):
    """Algorithmic flops of the gradients (FMA = 2): per token and head one
    forward step to recover the state (S~ = alpha S, S~^T k, the rank-1
    write: 5 dk dv) and the reverse step (dS += q do^T, S_t do, dS^T k,
    dS u, S~ du, dS - k du^T, rowsum(S~ .* dS~), alpha dS~: 15 dk dv)."""
    return 20 * tokens * H * dk * dv


def backward_alg_bytes(tokens, H, dk, dv, N, in_bytes=2):
    """Inputs q, k, v, beta, grad_o (in_bytes), g (fp32), h0 and the
    final-state gradient read once; dq, dk, dv, dg, dbeta (fp32) and dh0
    written once."""
    th = tokens * H
    return th * ((2 * dk + 2 * dv + 1) * in_bytes + dk * 4 + (3 * dk + dv + 1) * 4) + 3 * N * H * dk * dv * 4


def time_backward(args, name="backward_64k", chunk=True):
    """Gradients of a named workload, ms per call: kda_chunk_bwd (the chunk
    path) or kda_recurrent_bwd (token by token)."""
    import torch
    import gated_delta_rule_52_amd as kda
    from gated_delta_rule_52_amd.inputs import make_output_grads, make_workload
    x = make_workload(name)
    do, dhT = make_output_grads(x, 106)
    dev = "cuda:0"
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    q, k, v, beta, d_o = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf), t(do, bf)
    g, h0, dht = t(x.g, f32), t(x.h0, f32), t(dhT, f32)
    wsb = kda.chunk_bwd_workspace_bytes(q, v) if chunk else kda.recurrent_bwd_workspace_bytes(q, v)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    dh0 = torch.empty_like(h0)
    grads = {n: torch.empty(sh, dtype=f32, device=dev) for n, sh in
             (("dq", q.shape), ("dk", q.shape), ("dv", v.shape), ("dg", q.shape), ("dbeta", beta.shape))}
    bwd = kda.chunk_bwd if chunk else kda.recurrent_bwd
    fn = lambda: bwd(q, k, v, g, beta, d_o, initial_state=h0, grad_final_state=dht,
                     grad_initial_state=dh0, workspace=ws, out=grads)
    settle(fn)
    for _ in range(max(args.warmup, 1)):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    n = max(3, min(args.steps, 10))
    per = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    ms = float(np.mean(per))
    log(f"{name} ({'chunk' if chunk else 'token'} path): {ms:.3f} ms per call")
    del ws, grads
    return x, ms, per


def cpu_backward_sample(x):
    """The fp64 oracle's gradients on the first 1024 tokens of sequence 0,
    all heads (OpenMP over heads): tokens (all heads) per second."""
    import oracle
    from gated_delta_rule_52_amd.inputs import make_output_grads
    do, dhT = make_output_grads(x, 106)
    L = 1024
    sl = lambda a: np.ascontiguousarray(a[:1, :L])
    threads = min(len(os.sched_getaffinity(0)), x.H)
    t0 = time.perf_counter()
    oracle.backward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), sl(do), h0=x.h0[:1].astype(np.float64),
                    d_final_state=dhT[:1].astype(np.float64), nthreads=threads)
    dt = time.perf_counter() - t0
    log(f"oracle backward: {dt:.2f} s on {threads} threads")
    return dict(value=L / dt, unit="tokens/s (all 16 heads)", cores=threads, kind="oracle",
                sample=f"first {L} tokens of sequence 0, {x.H} heads, {dt:.2f} s wall")


def time_dplr(args):
    """The general DPLR recurrence against KDA on the same token-level harness: 256
    sequences x 16 heads x 64 new tokens from cached states (bf16, d = 128), us per call."""
    import torch
    import gated_delta_rule_52_amd as kda
    from gated_delta_rule_52_amd.inputs import make_dplr, make_workload
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda z, dt: torch.from_numpy(z).to("cuda:0").to(dt)
    x = make_workload("append_256x16x64")
    d = make_dplr(8, x.B, x.T, x.H, x.dk, x.dv, h0_std=0.02)
    kq, kk, kv, kb, kg, kh = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf), t(x.g, f32), t(x.h0, f32)
    dq, dk_, dv_, da, db = (t(d[n], bf) for n in ("q", "k", "v", "a", "b"))
    dg, dh = t(d["g"], f32), t(d["h0"], f32)
    hT = torch.empty_like(kh)
    o = torch.empty((x.B, x.T, x.H, x.dv), dtype=bf, device="cuda:0")
    paths = {
        "kda_recurrent_fwd": lambda: kda.recurrent_fwd(kq, kk, kv, kg, kb, initial_state=kh, final_state=hT, o=o,
                                                       token_by_token=True),
        "dplr_recurrent_fwd": lambda: kda.dplr_recurrent_fwd(dq, dk_, dv_, dg, da, db, initial_state=dh,
                                                             final_state=hT, o=o),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in paths.items():
        settle(fn)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = 1e3 * e0.elapsed_time(e1) / 10
        log(f"dplr comparison {name}: {res[name]:.1f} us per call")
    return res


def time_dplr_chunk(args, x):
    """KDA against the general DPLR recurrence, both in chunkwise form on the same fp32 matrix-core harness
    (chunks of 32, same segment plan and combine) over the 64K prefill: B=1, T=65536, H=16, d=128, bf16
    inputs.  The DPLR call gets a = beta k and b = exp(g) * k (KDA's member of the family; the kernel does
    not know they are tied).  ms per call of each, and the ratio."""
    import torch
    import gated_delta_rule_52_amd as kda
    dev = "cuda:0"
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    q, k, v, beta, g, h0 = t(x.q, bf), t(x.k, bf), t(x.v, bf), t(x.beta, bf), t(x.g, f32), t(x.h0, f32)
    a = (beta.float()[..., None] * k.float()).to(bf)
    b = (torch.exp(g) * k.float()).to(bf)
    hT = torch.empty_like(h0)
    o = torch.empty((x.B, x.T, x.H, x.dv), dtype=bf, device=dev)
    ws_k = torch.empty(kda.chunk_fwd_workspace_bytes(q, v, chunk_size=32), dtype=torch.uint8, device=dev)
    paths = {
        "kda_chunk_fwd_c32_fp32_path": lambda: kda.chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT,
                                                             o=o, out_dtype=bf, workspace=ws_k, chunk_size=32),
        "dplr_chunk_fwd_c32": lambda: kda.dplr_chunk_fwd(q, a, v, g, a, b, initial_state=h0, final_state=hT, o=o,
                                                         out_dtype=bf),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in paths.items():
        settle(fn)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
        log(f"chunk harness {name}: {res[name]:.3f} ms per call")
    return res


def ceilings():
    """Measured ceilings from this build's own kernels (libkda_ceilings.so):
    a streaming copy of 1 GiB read + 1 GiB written per launch (plain and
    non-temporal loads/stores, best launch of either), and a bf16 matrix-core
    loop (8 independent 16x16x32 products per wave, 2,048 workgroups of 4
    waves, no memory traffic).  Returns (copy GB/s, MFMA TFLOP/s, details)."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_52_amd", "libkda_ceilings.so"))
    lib.kda_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.kda_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.kda_ceiling_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.kda_ceiling_mfma_flops.restype = ctypes.c_double
    stream = torch.cuda.current_stream()
    nbytes = 1 << 30
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    best = {}
    for nt in (0, 1):
        for _ in range(2):
            assert lib.kda_ceiling_copy(a.data_ptr(), b.data_ptr(), nbytes, nt, stream.cuda_stream) == 0
        t = float("inf")
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lib.kda_ceiling_copy(a.data_ptr(), b.data_ptr(), nbytes, nt, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t = min(t, e0.elapsed_time(e1))
        best["nontemporal" if nt else "plain"] = 2 * nbytes / (t * 1e-3) / 1e9
    torch.cuda.synchronize()
    assert bool(torch.equal(a[:1024], b[:1024])), "copy ceiling kernel did not copy"
    del a, b
    blocks, iters = 2048, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    lib.kda_ceiling_mfma(out.data_ptr(), blocks, 100, stream.cuda_stream)
    tm = float("inf")
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert lib.kda_ceiling_mfma(out.data_ptr(), blocks, iters, stream.cuda_stream) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        tm = min(tm, e0.elapsed_time(e1))
    tflops = lib.kda_ceiling_mfma_flops(blocks, iters) / (tm * 1e-3) / 1e12
    del out
    copy_gbs = max(best.values())
    log(f"ceilings: copy {best} GB/s, bf16 MFMA loop {tflops:.0f} TFLOP/s")
    return copy_gbs, tflops, dict(copy_gbs=best, copy_bytes_each_way=nbytes, mfma_tflops=tflops,
                                  mfma="v_mfma_f32_16x16x32_bf16, 8 independent chains per wave, "
                                       f"{blocks} workgroups x 4 waves x {iters} iterations")


def cpu_baseline(x):
    """The fp64 token-recurrence oracle on the host cores, over the whole
    prefill_64k workload (16 heads x 65,536 tokens: a few seconds)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    units = x.N * x.H
    threads = min(cores, units)
    t0 = time.perf_counter()
    oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0.astype(np.float64), nthreads=threads,
                   want_state=True)
    dt = time.perf_counter() - t0
    log(f"oracle: {dt:.2f} s on {threads} threads")
    return dict(value=x.B * x.T / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"whole prefill_64k workload ({x.H} heads x {x.T} tokens, fp64 token "
                       f"recurrence, OpenMP over heads), {dt:.2f} s wall")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode and append lines")
    ap.add_argument("--no-append", action="store_true", help="skip the append line")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the length sweep and the fused input-transform and scalar-gate lines")
    ap.add_argument("--no-backward", action="store_true", help="skip the gradients line")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the operator's heads and sequences shard with no exchange, see the design notes",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sweep = None if args.no_fused else {}
    ceil_res = []
    x, ms, per, nbytes = time_prefill(args, calibrate=args.calibrate_copy, sweep=sweep,
                                      before=lambda: ceil_res.append(ceilings()), settle_ms=0.0)
    copy_gbs, mfma_tflops, ceil = ceil_res[0]
    tok_s = x.B * x.T / (ms * 1e-3)
    ach = nbytes / (ms * 1e-3) / 1e9
    traffic = stored_traffic()
    rec = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_64k", "B": x.B, "T": x.T, "H": x.H, "dk": x.dk, "dv": x.dv,
                   "in_dtype": "bf16", "out_dtype": "bf16", "chunk": 64, "initial_state": True,
                   "final_state": True},
        "ms_median": float(np.median(per)), "ms_p10": float(np.percentile(per, 10)),
        "ms_p90": float(np.percentile(per, 90)),
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                     "measured_copy_gbs": copy_gbs, "frac_of_measured_copy": ach / copy_gbs,
                     "alg_bytes_per_launch": nbytes,
                     "pages_flops_per_launch": PAGES_FLOPS_PER_TOKEN_HEAD * x.B * x.T * x.H,
                     "mfma_frac_of_bf16_peak": PAGES_FLOPS_PER_TOKEN_HEAD * x.B * x.T * x.H / (ms * 1e-3) / 1e12
                                               / BF16_MFMA_PEAK_TFLOPS,
                     "kernel": "kda_chunk_fwd: one call = prep, exact-path pass, local scan (segment tails, "
                               "then whole segments whose tail transition is not zero), combine, output scan "
                               "(timed together on the library's stream)"},
    }
    rec["ceilings"] = ceil
    if not args.no_decode:
        d = time_decode(args)
        dach = d["nbytes"] / (d["us"] * 1e-6) / 1e9
        dach_ip = d["nbytes"] / (d["us_in_place"] * 1e-6) / 1e9
        rec["decode"] = {
            "workload": "decode_256x16", "state_buffers": "ping-pong: step s reads buffer s%2, writes the other "
                                                          "(512 MiB of state, beyond the 256 MiB Infinity Cache)",
            "us_per_step": d["us"], "us_per_token_step": d["us"], "us_per_token_amortized": d["us"] / d["N"],
            "tokens_per_s": d["N"] / (d["us"] * 1e-6), "steps": d["steps"],
            "roofline": {"bound": "hbm", "achieved": dach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dach / HBM_PEAK_GBS, "alg_bytes_per_launch": d["nbytes"],
                         "measured_copy_gbs": copy_gbs, "frac_of_measured_copy": dach / copy_gbs},
            "in_place": {"us_per_step": d["us_in_place"], "us_per_step_graph": d["us_graph"],
                         "note": "one 256 MiB state buffer updated in place: the Infinity Cache can serve part of it",
                         "achieved_gbs": dach_ip, "frac": dach_ip / HBM_PEAK_GBS},
        }
    for key, wl in (("prefill_4k", "prefill_4k"), ("varlen", "varlen_8seq")):
        xo, warm, cold, obytes = time_prefill_own(args, wl)
        toks = xo.B * xo.T
        rec[key] = {
            "workload": wl, "tokens": toks, "H": xo.H, "N": xo.N, "initial_state": xo.h0 is not None,
            "ms_per_call_warm": warm, "ms_per_call_cold": cold,
            "tokens_per_s_warm": toks / (warm * 1e-3), "tokens_per_s_cold": toks / (cold * 1e-3),
            "roofline": {"bound": "hbm", "alg_bytes_per_launch": obytes, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "achieved_cold": obytes / (cold * 1e-3) / 1e9,
                         "frac_cold": obytes / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "achieved_warm": obytes / (warm * 1e-3) / 1e9,
                         "frac_warm": obytes / (warm * 1e-3) / 1e9 / HBM_PEAK_GBS},
        }
        if xo.cu_seqlens is not None:
            rec[key]["seqlens"] = np.diff(xo.cu_seqlens).tolist()
        del xo
    if not (args.no_decode or args.no_append):
        xa, ra, abytes = time_append(args)
        best = min(ra, key=ra.get)
        aach = abytes / (ra[best] * 1e-6) / 1e9
        rec["append"] = {
            "workload": "append_256x16x64", "N": xa.B, "T": xa.T, "H": xa.H,
            "us_per_call": {k: v for k, v in ra.items()}, "path": best,
            "tokens_per_s": xa.B * xa.T / (ra[best] * 1e-6),
            "roofline": {"bound": "hbm", "achieved": aach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": aach / HBM_PEAK_GBS, "alg_bytes_per_launch": abytes},
        }
    if sweep:
        rec["sweep"] = {
            "workload": "prefixes of prefill_64k (B=1, H=16, dk=dv=128, bf16, h0 and hT)",
            "ms_per_call": {str(T): t for T, t in sorted(sweep.items())},
            "tokens_per_s": {str(T): T / (t * 1e-3) for T, t in sorted(sweep.items())},
            "frac_of_hbm_peak": {str(T): prefill_alg_bytes(1, T, x.H, x.dk, x.dv, 1) / (t * 1e-3) / 1e9 / HBM_PEAK_GBS
                                 for T, t in sorted(sweep.items())},
        }
    if not args.no_fused:
        xf, msf, perf, fbytes = time_prefill(args, "prefill_64k_fused")
        fach = fbytes / (msf * 1e-3) / 1e9
        rec["fused"] = {
            "workload": "prefill_64k_fused", "transforms": xf.transforms(),
            "ms_per_step": msf, "ms_median": float(np.median(perf)),
            "tokens_per_s": xf.B * xf.T / (msf * 1e-3),
            "roofline": {"bound": "hbm", "achieved": fach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": fach / HBM_PEAK_GBS, "alg_bytes_per_launch": fbytes},
        }
        xs, mss, pers, _ = time_prefill(args, "prefill_64k_scalar_gate")
        sbytes = prefill_alg_bytes(xs.B, xs.T, xs.H, xs.dk, xs.dv, xs.N, gate_width=1)
        sach = sbytes / (mss * 1e-3) / 1e9
        rec["scalar_gate"] = {
            "workload": "prefill_64k_scalar_gate", "ms_per_step": mss, "ms_median": float(np.median(pers)),
            "tokens_per_s": xs.B * xs.T / (mss * 1e-3), "vs_channel_gate": ms / mss,
            "roofline": {"bound": "hbm", "achieved": sach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": sach / HBM_PEAK_GBS, "alg_bytes_per_launch": sbytes},
        }
    if not (args.no_decode or args.no_append):
        rd = time_dplr(args)
        rec["dplr"] = {
            "workload": "256 sequences x 16 heads x 64 new tokens, dk=dv=128, bf16, cached states; token by token",
            "us_per_call": rd, "dplr_over_kda": rd["dplr_recurrent_fwd"] / rd["kda_recurrent_fwd"],
        }
        rc = time_dplr_chunk(args, x)
        rec["dplr_chunk"] = {
            "workload": "prefill_64k inputs (B=1, T=65536, H=16, dk=dv=128, bf16, h0), chunkwise, fp32 matrix-core "
                        "harness with chunks of 32; DPLR gets a = beta k, b = exp(g) k",
            "ms_per_call": rc, "dplr_over_kda": rc["dplr_chunk_fwd_c32"] / rc["kda_chunk_fwd_c32_fp32_path"],
            "pages_ratio": 59.22 / 29.83,
        }
        rec["append_grid"] = {
            "workload": "N sequences x T new tokens, 16 heads, dk=dv=128, bf16, cached states (key 'NxT')",
            "us_per_call": time_append_grid(),
        }
    if not args.no_backward:
        for key, wl in (("backward", "backward_64k"), ("backward_batch", "backward_16x4096x16")):
            xb, msb, perb = time_backward(args, wl, chunk=True)
            _, mst, pert = time_backward(args, wl, chunk=False)
            toks = xb.B * xb.T
            flops = backward_alg_flops(toks, xb.H, xb.dk, xb.dv)
            bbytes = backward_alg_bytes(toks, xb.H, xb.dk, xb.dv, xb.N)
            tf = flops / (msb * 1e-3) / 1e12
            rec[key] = {
                "workload": wl, "B": xb.B, "T": xb.T, "H": xb.H, "dk": xb.dk, "dv": xb.dv,
                "in_dtype": "bf16", "grad_dtype": "fp32", "path": "kda_chunk_bwd",
                "ms_per_call": msb, "ms_median": float(np.median(perb)),
                "tokens_per_s": toks / (msb * 1e-3),
                "token_path": {"entry": "kda_recurrent_bwd", "ms_per_call": mst, "ms_median": float(np.median(pert)),
                               "tokens_per_s": toks / (mst * 1e-3), "chunk_speedup": mst / msb},
                "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": tf / FP32_VECTOR_PEAK_TFLOPS, "alg_flops_per_launch": flops,
                             "flops_basis": "the token recurrence's gradient flops (20 dk dv per token and head); "
                                            "peak: fp32 matrix cores, on which the chunk-local kernel runs",
                             "hbm_alg_bytes_per_launch": bbytes,
                             "hbm_frac": bbytes / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "kernel": "one kda_chunk_bwd call: segment table, prep, local pass, combine, forward "
                                       "replay, reverse packs, reverse local pass, reverse combine, reverse replay, "
                                       "chunk gradients"},
            }
            if key == "backward" and not args.no_cpu:
                rec[key]["cpu_baseline"] = cpu_backward_sample(xb)
            del xb
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
