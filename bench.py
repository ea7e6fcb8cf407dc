#!/usr/bin/env python3
"""Throughput of the SSD forward scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                    [--no-layer]

Profiling helpers (see profiles/):
    python bench.py --profile-loop K      run each kernel K times, plus a
                                          1 GiB device copy for calibration
    python bench.py --summarize-trace DIR --out FILE
    python bench.py --summarize-counters DIR_FETCH DIR_WRITE --out-dir profiles
    python bench.py --summarize-sq DIR --out-dir profiles
    python bench.py --state-passing-long  sequential vs segmented state passing
                                          at the long-context shape

A step is one ssd_forward call over the Mamba-2-2.7B-shaped workload (chunk
cumsum, chunk state, state passing and chunk scan): batch 4, seqlen 8192, 80
heads, P = 64, N = 128, one B/C group, chunk 256, bf16 x/B/C, fp32 dt/A/D and
state, random initial state.  Inputs are resident in HBM before timing starts;
about 0.3 s of untimed forward calls let the GPU clocks ramp before the W
warm-up steps and the K timed ones.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (its
algorithmic bytes per launch over its average launch time, measured here with
HIP events on the stream it runs on), per-kernel figures, the decode step
(batch 256, 64 steps; and at batch 1 and 4 issued call by call against one
HIP graph of the 64 calls), the zero-order-hold forward, the kernels of the block
around the scan (short convolution + step, gate) at the same shape, and the
fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = "SSD fwd tokens/s at B=4,L=8K,H=80,P=64,N=128 bf16; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
KERNEL_SOURCES = {
    "chunk_cumsum": "chunk_cumsum.hip",
    "chunk_state": "chunk_state.hip",
    "chunk_state_cumsum": "chunk_state.hip",
    "state_passing": "state_passing.hip",
    "chunk_scan": "chunk_scan.hip",
    "state_scan": "state_scan.hip",
    "chunk_state_runs": "chunk_state.hip",
    "run_passing": "state_passing.hip",
    "chunk_scan_runs": "chunk_scan.hip",
    "ssm_step": "ssm_step.hip",
    "layer_in": "layer.hip",
    "layer_dt": "layer.hip",
    "layer_out": "layer.hip",
}
LAYER_K = 4                     # short-convolution width of the block around the scan


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------- byte models
def forward_model(b, L, H, P, N, G, Q, K=0):
    """Algorithmic HBM bytes and flops of each kernel: every input read once,
    every output written once (workspace intermediates included, S, Hin, T
    and Hr in bf16).
    state_scan does what chunk_state + state_passing do without S.  With a
    run length K > 0, also the two-level path: chunk_state_runs writes one T
    per chunk (and lam, rdec), run_passing reads the T ending each run and
    writes one Hr per run, chunk_scan_runs reads the T of every chunk past a
    run's first and each run's Hr once."""
    nc = -(-L // Q)
    tok = b * L
    x = tok * H * P * 2
    bc = tok * G * N * 2
    dt = tok * H * 4
    rows = b * H * nc * Q * 4               # one of cs / dtc
    st = b * H * P * N * 4                  # init or final
    S = b * H * nc * P * N * 2                # bf16, like Hin
    Hin = b * H * nc * P * N * 2
    bytes_ = {
        "chunk_cumsum": dt + 2 * rows,
        "chunk_state": x + bc + 2 * rows + S,
        "chunk_state_cumsum": x + bc + dt + 2 * rows + S,
        "state_passing": S + b * H * nc * 4 + st + Hin + st,
        "chunk_scan": x + 2 * bc + 2 * rows + Hin + x,
        "state_scan": x + bc + 2 * rows + st + Hin + st,
    }
    if K > 0:
        nruns = -(-nc // K)
        pn = P * N * 2
        bytes_.update({
            "chunk_state_runs": x + bc + dt + 2 * rows + S + b * H * nc * 4 + b * H * nruns * 4,
            "run_passing": b * H * nruns * pn + b * H * nruns * 4 + st + b * H * nruns * pn + st,
            "chunk_scan_runs": x + 2 * bc + 2 * rows + b * H * (nc - nruns) * pn + b * H * nruns * pn +
                               b * H * nc * 4 + x,
        })
    th = tok * H
    flops = {
        "chunk_cumsum": 2 * th,
        "chunk_state": 2 * P * N * th,                               # sum_j w_j x_j B_j^T
        "chunk_state_cumsum": 2 * P * N * th + 2 * th,
        "state_passing": 2 * b * H * nc * P * N,
        "chunk_scan": ((Q + 1) * P + 2 * N * P) * th + (Q + 1) * N * tok * G,  # causal-exact
        "state_scan": 2 * P * N * th + 2 * b * H * nc * P * N,
    }
    if K > 0:
        flops.update({
            "chunk_state_runs": flops["chunk_state_cumsum"] + 2 * b * H * nc * P * N,
            "run_passing": 2 * b * H * (-(-nc // K)) * P * N,
            "chunk_scan_runs": flops["chunk_scan"] + 2 * b * H * nc * P * N,
        })
    return bytes_, flops


def layer_model(b, L, H, P, N, G, K):
    """Algorithmic HBM bytes of the kernels around the scan (bf16 storage):
    the convolution launch reads xbc (and the filter) and writes x, B, C, and
    its extra blocks read dt_raw (and dt_bias) and write dt; the gate reads y
    and z and writes out.  (layer_dt: the step kernel the per-element path
    launches on its own.)"""
    tok = b * L
    cd = H * P + 2 * G * N
    dt = 2 * tok * H * 4 + H * 4
    return {"layer_in": 2 * tok * cd * 2 + cd * (K + 1) * 4 + dt,
            "layer_dt": dt,
            "layer_out": 3 * tok * H * P * 2}


def compulsory_bytes(b, L, H, P, N, G):
    tok = b * L
    return tok * H * P * 2 * 2 + tok * G * N * 2 * 2 + tok * H * 4 + 2 * b * H * P * N * 4


def source_hash(kernel: str) -> str:
    p = ROOT / "mamba_ssd_scan_02_amd" / "csrc" / KERNEL_SOURCES[kernel]
    h = hashlib.sha256(p.read_bytes())
    for inc in ("device_common.h", "lds_pipe.h"):   # device code every kernel includes
        h.update((ROOT / "mamba_ssd_scan_02_amd" / "csrc" / inc).read_bytes())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per dispatch from the committed rocprofv3 counter summary for
    this kernel and workload, or None if there is none or the kernel source
    changed since the counters were taken."""
    path = ROOT / "profiles" / f"{kernel}_{workload}_counters.txt"
    if not path.exists():
        return None
    text = path.read_text()
    m_hash = re.search(r"^source_sha256_16:\s*(\w+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_dispatch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(kernel):
        return None
    return float(m_bytes.group(1))


def trace_average(kernel: str, workload: str):
    """(average dispatch duration in us, file) of ``kernel`` in the committed
    rocprofv3 kernel-trace summary of this workload's forward, or None."""
    path = ROOT / "profiles" / f"ssd_forward_{workload}_kernel_trace.txt"
    if not path.exists():
        return None
    for line in path.read_text().splitlines():
        parts = line.split()
        if len(parts) >= 3 and parts[0] == kernel:
            try:
                return float(parts[2]), str(path.relative_to(ROOT))
            except ValueError:
                return None
    return None


# -------------------------------------------------------------------- timing
SETTLE_S = 0.3


def settle(fn, seconds=SETTLE_S):
    """Run fn untimed for about ``seconds`` of wall time so that the GPU's
    clocks have ramped before anything is timed (without it the first tens
    of steps run up to 8% slower)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def time_forward(ssd, g, y, fin, ws, chunk, steps, warmup, zoh=False):
    import torch

    def step():
        ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk, g["init"], y=y,
                        final_state=fin, workspace=ws, zoh=zoh)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def forward_kernels(dims, K=0):
    """The kernels ssd_forward runs at these sizes, by the names of the stage
    calls that launch the same kernels: with a run length K > 0 (what
    ssd_forward_run_chunks reports) the two-level path (chunk states over
    runs, the chain over runs, the chunk scan forming the entering states);
    else chunk state with the cumsum inside (ssd_chunk_cumsum_state, one
    launch where a group's head count is even), state passing and
    chunk_scan."""
    b, L, H, P, N, G, Q = dims
    if K > 0:
        return ["chunk_state_runs", "run_passing", "chunk_scan_runs"]
    fused = P == 64 and N == 128 and Q in (64, 128, 256) and (H // G) % 2 == 0
    return (["chunk_state_cumsum"] if fused else ["chunk_cumsum", "chunk_state"]) + \
        ["state_passing", "chunk_scan"]


def time_stages(ssd, g, y, fin, dims, steps, K=0):
    """Average duration of each kernel, from HIP events recorded on the
    stream the stage calls are launched on (torch's current stream): first
    the forward's own kernels in the forward's order (chunk state with the
    cumsum inside, state passing, chunk scan -- each launched by the stage
    call that runs the same kernel), repeated with nothing else in between,
    so each one follows what it follows in the forward; then, in a loop of
    their own, the stand-alone cumsum and chunk state and the one-pass state
    stage.  Buffers of their own, not the forward's workspace."""
    import ctypes
    import torch
    lib = ssd.load()
    b, L, H, P, N, G, Q = dims
    nc = -(-L // Q)
    dev = g["x"].device
    cs_t = torch.empty((b, H, nc, Q), dtype=torch.float32, device=dev)
    dtc_t = torch.empty_like(cs_t)
    S_t = torch.empty((b, H, nc, P, N), dtype=torch.bfloat16, device=dev)
    Hin_t = torch.empty((b, H, nc, P, N), dtype=torch.bfloat16, device=dev)
    cs, dtc, S, Hin = (ctypes.c_void_p(t.data_ptr()) for t in (cs_t, dtc_t, S_t, Hin_t))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    names = ["chunk_state_cumsum", "state_passing", "chunk_scan", "chunk_cumsum", "chunk_state",
             "state_scan"]
    groups = [(0, 1, 2), (3, 4, 5)]
    if K > 0:   # the forward's two-level path first; the per-chunk trio as a stage group
        nruns = -(-nc // K)
        T_t = torch.empty((b, H, nc, P, N), dtype=torch.bfloat16, device=dev)
        Hr_t = torch.empty((b, H, nruns, P, N), dtype=torch.bfloat16, device=dev)
        lam_t = torch.empty((b, H, nc), dtype=torch.float32, device=dev)
        rdec_t = torch.empty((b, H, nruns), dtype=torch.float32, device=dev)
        T, Hr, lam, rdec = (ctypes.c_void_p(t.data_ptr()) for t in (T_t, Hr_t, lam_t, rdec_t))
        names += ["chunk_state_runs", "run_passing", "chunk_scan_runs"]
        groups = [(6, 7, 8), (0, 1, 2), (3, 4, 5)]
    calls = [
        lambda: lib.ssd_chunk_cumsum_state(b, L, H, P, N, G, Q, 1, p(g["x"]), p(g["B"]), p(g["dt"]),
                                           p(g["A"]), cs, dtc, S, stream),
        lambda: lib.ssd_state_passing(b, L, H, P, N, Q, 1, S, cs, p(g["init"]), Hin, p(fin), stream),
        lambda: lib.ssd_chunk_scan(b, L, H, P, N, G, Q, 1, p(g["x"]), p(g["B"]), p(g["C"]),
                                   cs, dtc, Hin, p(g["D"]), p(y), stream),
        lambda: lib.ssd_chunk_cumsum(b, L, H, Q, p(g["dt"]), p(g["A"]), cs, dtc, stream),
        lambda: lib.ssd_chunk_state(b, L, H, P, N, G, Q, 1, p(g["x"]), p(g["B"]), cs, dtc, S, stream),
        lambda: lib.ssd_state_scan(b, L, H, P, N, G, Q, 1, p(g["x"]), p(g["B"]), cs, dtc,
                                   p(g["init"]), Hin, p(fin), stream),
    ]
    if K > 0:
        calls += [
            lambda: lib.ssd_chunk_state_runs(b, L, H, P, N, G, Q, 1, K, p(g["x"]), p(g["B"]),
                                             p(g["dt"]), p(g["A"]), cs, dtc, T, lam, rdec, stream),
            lambda: lib.ssd_run_passing(b, L, H, P, N, Q, 1, K, T, rdec, p(g["init"]), Hr, p(fin),
                                        stream),
            lambda: lib.ssd_chunk_scan_runs(b, L, H, P, N, G, Q, 1, K, p(g["x"]), p(g["B"]),
                                            p(g["C"]), cs, dtc, T, Hr, lam, p(g["D"]), p(y), stream),
        ]
    for f in calls:            # warm
        assert f() == 0
    torch.cuda.synchronize()
    out = {}
    # the forward's three kernels on their own, back to back: what each finds
    # in the caches is what it finds inside ssd_forward; then each other group
    # of stage kernels in a loop of its own
    for group in groups:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(group) + 1)]
              for _ in range(steps)]
        for k in range(steps):
            ev[k][0].record()
            for j, i in enumerate(group):
                if calls[i]() != 0:
                    raise RuntimeError(f"{names[i]} failed")
                ev[k][j + 1].record()
        torch.cuda.synchronize()
        for j, i in enumerate(group):   # microseconds
            out[names[i]] = sum(ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(steps)) / steps * 1e3
    return out


def bench_decode(ssd, steps_warm=3):
    import torch
    from mamba_ssd_scan_02_amd.workloads import DECODE_B256 as spec
    from mamba_ssd_scan_02_amd.workloads import make_decode_static, make_decode_step
    st = make_decode_static(spec)
    state = st["state"].cuda()
    A, D = st["A"].cuda(), st["D"].cuda()
    ins = [{k: v.cuda() for k, v in make_decode_step(spec, t).items()} for t in range(spec.steps)]
    ys = [torch.empty_like(i["x"]) for i in ins]
    for t in range(steps_warm):
        ssd.ssm_step(state, ins[t]["x"], ins[t]["dt"], A, ins[t]["B"], ins[t]["C"], D, y_t=ys[t])
    torch.cuda.synchronize()
    state.copy_(st["state"].cuda())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(spec.steps):
        ssd.ssm_step(state, ins[t]["x"], ins[t]["dt"], A, ins[t]["B"], ins[t]["C"], D, y_t=ys[t])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / spec.steps
    b, H, P, N, G = spec.batch, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    byts = b * H * P * N * 4 * 2 + b * H * P * 2 * 2 + b * H * 4 + 2 * b * G * N * 2 + 2 * H * 4
    gbs = byts / (us * 1e-6) / 1e9
    return {
        "workload": spec.name, "tokens_per_s": b / (us * 1e-6), "us_per_step": us,
        "bytes_per_step": byts, "achieved_GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
        "traffic": counter_traffic("ssm_step", spec.name),
    }


def bench_decode_graph(ssd, batches=(1, 4), reps=5):
    """Decode at small batch, where each step is a few microseconds of GPU
    work: the 64 steps issued one binding call at a time (host-bound) against
    the same 64 calls captured once in a HIP graph and replayed."""
    import torch
    from mamba_ssd_scan_02_amd.workloads import DECODE_B256, make_decode_static, make_decode_step
    out = []
    for batch in batches:
        spec = DECODE_B256.with_(batch=batch)
        st = make_decode_static(spec)
        A, D = st["A"].cuda(), st["D"].cuda()
        state = st["state"].cuda()
        ins = [{k: v.cuda() for k, v in make_decode_step(spec, t).items()} for t in range(spec.steps)]
        ys = [torch.empty_like(i["x"]) for i in ins]

        def run():
            for i, yt in zip(ins, ys):
                ssd.ssm_step(state, i["x"], i["dt"], A, i["B"], i["C"], D, y_t=yt)

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) * 1e3 / (reps * spec.steps)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * spec.steps)
        out.append({"batch": batch, "eager_us_per_step": round(eager, 2), "graph_us_per_step": round(us, 2)})
    return out


def bench_layer(ssd, spec, steps=20, block=True):
    """ssd_layer_in (convolution + step kernels) and ssd_layer_out at the
    forward workload's shape, filter width LAYER_K, timed with HIP events on
    the stream they run on."""
    import torch
    from mamba_ssd_scan_02_amd.workloads import make_layer_inputs
    b, L, H, P, N, G = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    li = {k: v.cuda() for k, v in make_layer_inputs(spec, LAYER_K).items() if v is not None}
    x = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    Bm = torch.empty((b, L, G, N), dtype=torch.bfloat16, device="cuda")
    Cm = torch.empty_like(Bm)
    dt = torch.empty((b, L, H), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    run_in = lambda: ssd.layer_in(li["xbc"], li["conv_w"], li["conv_b"], li["dt_raw"],
                                  li["dt_bias"], H, P, G, N, x=x, B=Bm, C=Cm, dt=dt)
    run_out = lambda: ssd.layer_out(x, li["z"], out=out)
    res = {}
    mb = layer_model(b, L, H, P, N, G, LAYER_K)
    for name, fn, byts in (("layer_in", run_in, mb["layer_in"]),
                           ("layer_out", run_out, mb["layer_out"])):
        settle(fn, 0.2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        gbs = byts / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "alg_bytes": byts, "GBps": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    res["kernel_width"] = LAYER_K
    if not block:
        return res
    # the whole block: layer_in -> ssd_forward -> layer_out (in place)
    A, D, init = li["A"], li["D"], li.get("init")
    y = torch.empty_like(x)
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(ssd.workspace_bytes(b, L, H, P, N, G, spec.chunk, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def block():
        run_in()
        ssd.ssd_forward(x, dt, A, Bm, Cm, D, spec.chunk, init, y=y, final_state=fin, workspace=ws)
        ssd.layer_out(y, li["z"], out=y)

    # the same block with the gate inside the chunk scan's store
    # (ssd_forward_gated): layer_in -> ssd_forward_gated
    def block_gated():
        run_in()
        ssd.ssd_forward(x, dt, A, Bm, Cm, D, spec.chunk, init, y=y, final_state=fin, workspace=ws,
                        z=li["z"])

    for name, fn in (("block", block), ("block_gated", block_gated)):
        settle(fn, 0.1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        res[name] = {"us": round(us, 2), "tokens_per_s": round(b * L / (us * 1e-6), 1)}
    return res


def bench_state_passing_long(nsegs=(8, 32, 128), steps=10):
    """State passing at the long-context shape (1 x 32 chains of 4,096 chunks):
    the sequential kernel against the segmented associative scan.  S and the
    decays are drawn on the device (only their shapes matter for timing)."""
    import ctypes
    import torch
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import LONG_1M as spec
    b, L, H, P, N, Q = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.chunk
    nc = -(-L // Q)
    lib = ssd.load()
    gen = torch.Generator(device="cuda").manual_seed(spec.seed)
    dt = torch.nn.functional.softplus(torch.randn(b, L, H, device="cuda", generator=gen) + spec.dt_shift)
    A = -torch.exp(torch.rand(H, device="cuda", generator=gen) * spec.a_hi)
    cs, _ = ssd.chunk_cumsum(dt, A, Q)
    del dt
    S = torch.randn(b, H, nc, P, N, device="cuda", generator=gen).to(torch.bfloat16)
    Hin = torch.empty(b, H, nc, P, N, dtype=torch.bfloat16, device="cuda")
    fin = torch.empty(b, H, P, N, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    byts = S.numel() * 2 + Hin.numel() * 2 + fin.numel() * 4

    def timed(f):
        assert f() == 0
        settle(f, 0.1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        return {"us": round(us, 1), "hbm_frac_one_pass": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    out = {"workload": f"state passing, {b * H} chains x {nc} chunks (P {P}, N {N})",
           "one_pass_bytes": byts,
           "sequential": timed(lambda: lib.ssd_state_passing(b, L, H, P, N, Q, 1, p(S), p(cs), None,
                                                             p(Hin), p(fin), st))}
    for ns in nsegs:
        need = lib.ssd_state_passing_seg_workspace_bytes(b, H, P, N, ns)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out[f"segmented_{ns}"] = timed(lambda: lib.ssd_state_passing_seg(
            b, L, H, P, N, Q, ns, 1, p(S), p(cs), None, p(Hin), p(fin), p(ws), need, st))
        del ws
    return out


def host_cpu():
    """(CPU model name, physical core count) of this host from /proc/cpuinfo
    (distinct (physical id, core id) pairs), or (None, None)."""
    try:
        text = Path("/proc/cpuinfo").read_text()
    except OSError:
        return None, None
    model, cores, phys, core = None, set(), None, None
    for line in text.splitlines() + [""]:
        if ":" in line:
            k, v = (t.strip() for t in line.split(":", 1))
            if k == "model name" and model is None:
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id":
                core = v
        elif not line.strip():
            if core is not None:
                cores.add((phys, core))
            phys = core = None
    return model, (len(cores) or None)


def cpu_baseline(inp, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same workload: whole
    sequences of (batch, head) pairs, in batches of one pair per core,
    cycling over the pairs until the time budget is spent."""
    import oracle
    b, L, H = inp["x"].shape[0], inp["x"].shape[1], inp["x"].shape[2]
    cores = oracle.threads()
    pairs = [(i, h) for i in range(b) for h in range(H)]
    done, t_total, k = 0, 0.0, 0
    while t_total < budget_s:
        chunk = [pairs[(k + i) % len(pairs)] for i in range(min(cores, len(pairs)))]
        t0 = time.perf_counter()
        oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init"],
                       bh=chunk)
        t_total += time.perf_counter() - t0
        done += len(chunk)
        k = (k + len(chunk)) % len(pairs)
    tokens_equiv = done * L / H
    model, physical = host_cpu()
    return {"value": tokens_equiv / t_total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "physical_cores": physical, "logical_cpus": os.cpu_count(),
            "sample": f"{done} (batch, head) sequences of {L} tokens of the same workload, cycling "
                      f"over its {len(pairs)} pairs (= {tokens_equiv:.0f} full-width tokens), "
                      f"in {t_total:.1f} s"}


# ----------------------------------------------------------------- profiling
COPY_BYTES = 1 << 30


def profile_loop(k: int):
    """Each kernel of the forward and decode paths k times, then a plain
    device-to-device copy of COPY_BYTES (the counter calibration)."""
    import torch

    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_2P7B as spec
    from mamba_ssd_scan_02_amd.workloads import make_forward_inputs
    dims = (spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups,
            spec.chunk)
    b, L, H, P, N, G, Q = dims
    inp = make_forward_inputs(spec)
    g = {kk: v.cuda() for kk, v in inp.items()}
    y = torch.empty_like(g["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(ssd.workspace_bytes(b, L, H, P, N, G, Q, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    for _ in range(k):   # the forward itself, so the trace holds its kernels as it runs them
        ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], Q, g["init"], y=y,
                        final_state=fin, workspace=ws)
    time_stages(ssd, g, y, fin, dims, k, ssd.forward_run_chunks(*dims, torch.bfloat16))
    from mamba_ssd_scan_02_amd.workloads import DECODE_B256 as dspec
    from mamba_ssd_scan_02_amd.workloads import make_decode_static, make_decode_step
    st = make_decode_static(dspec)
    state = st["state"].cuda()
    A, D = st["A"].cuda(), st["D"].cuda()
    s0 = {kk: v.cuda() for kk, v in make_decode_step(dspec, 0).items()}
    for _ in range(k):
        ssd.ssm_step(state, s0["x"], s0["dt"], A, s0["B"], s0["C"], D)
    del g, y, ws
    bench_layer(ssd, spec, steps=k, block=False)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(k):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[profile-loop] done ({k} iterations)")


def _short_kernel(name: str) -> str:
    if "chunk_state_runs_kernel" in name:
        return "chunk_state_runs"     # chunk states over runs (two-level path)
    if "run_passing_kernel" in name:
        return "run_passing"          # the chain over runs
    if "chunk_scan_paired_kernel<true, true>" in name:
        return "chunk_scan_runs_gated"   # the same with the block's gate in its store
    if "chunk_scan_paired_kernel<false, true>" in name:
        return "chunk_scan_gated"
    if "chunk_scan_paired_kernel<true" in name:
        return "chunk_scan_runs"      # chunk scan forming the entering states
    if "chunk_state" in name and ", true>" in name:
        return "chunk_state_cumsum"   # chunk state with the cumsum inside
    if "state_walk" in name:
        return "state_scan"           # what ssd_state_scan launches for chunk 128 / 256
    for k in KERNEL_SOURCES:
        if k in name:
            return k
    if "copyBuffer" in name or "copy" in name.lower():
        return "copy"
    return name.split("(")[0][-40:]


def summarize_trace(d: str, out: str, cmd: str):
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not f:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(f[0])))
    # medians from the per-dispatch trace beside the stats, when present
    med = {}
    t = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if t:
        durs = {}
        for r in csv.DictReader(open(t[0])):
            durs.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in durs.items():
            v.sort()
            n = len(v)
            med[k] = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    lines = ["# rocprofv3 kernel trace summary (per-kernel dispatch durations)",
             f"command: {cmd}", "",
             f"{'kernel':24s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} "
             f"{'max_us':>10s} {'total_%':>8s}"]
    for r in rows:
        avg = float(r["AverageNs"]) / 1e3
        m = med.get(r["Name"])
        mtxt = f"{m:10.2f}" if m is not None else f"{'-':>10s}"
        lines.append(f"{_short_kernel(r['Name']):24s} {int(r['Calls']):6d} {avg:10.2f} {mtxt} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):8.2f}")
    lines.append("")
    lines.append("full kernel names:")
    for r in rows:
        lines.append(f"  {_short_kernel(r['Name'])}: {r['Name'][:160]}")
    Path(out).write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(d_fetch: str, d_write: str, out_dir: str, cmd_fetch: str, cmd_write: str,
                       xcheck=None, cmd_rd: str = "", cmd_wr: str = ""):
    """Per-kernel HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by the ratio known bytes / counter value of the
    calibration copy (COPY_BYTES read and written).  With ``xcheck`` = (dir of
    a TCC_EA0_RDREQ{,_32B,_64B,_128B} pass, dir of a TCC_EA0_WRREQ{,_64B}
    pass), the same bytes are also counted request by request at their
    sizes, which needs no calibration: FETCH_SIZE counts each read request
    that is not 32 bytes as 64 bytes, while the reads here are 128-byte
    requests -- the copy's factor of 2."""
    import csv
    import glob
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_2P7B, DECODE_B256

    def load(dd, counter):
        f = sorted(glob.glob(os.path.join(dd, "**", "*counter_collection.csv"), recursive=True))
        if not f:
            raise SystemExit(f"no counter_collection.csv under {dd}")
        acc = {}
        copies = []
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] != counter:
                continue
            k = _short_kernel(r["Kernel_Name"])
            if k == "copy":
                copies.append((int(r["Grid_Size"]), float(r["Counter_Value"])))
            else:
                acc.setdefault(k, []).append(float(r["Counter_Value"]))
        if copies:   # the calibration copy is the largest one
            gmax = max(gs for gs, _ in copies)
            acc["copy"] = [v for gs, v in copies if gs == gmax]
        return acc

    fetch = load(d_fetch, "FETCH_SIZE")
    write = load(d_write, "WRITE_SIZE")
    xr = xw = None
    if xcheck:
        rq = {c: load(xcheck[0], c) for c in ("TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B",
                                               "TCC_EA0_RDREQ_128B")}
        wq = {c: load(xcheck[1], c) for c in ("TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B")}
        avg = lambda v: sum(v) / len(v)
        xr = {k: 32 * avg(rq["TCC_EA0_RDREQ_32B"][k]) + 64 * avg(rq["TCC_EA0_RDREQ_64B"][k]) +
              128 * avg(rq["TCC_EA0_RDREQ_128B"][k]) for k in rq["TCC_EA0_RDREQ_128B"]}
        xw = {k: 64 * avg(wq["TCC_EA0_WRREQ_64B"][k]) +
              32 * (avg(wq["TCC_EA0_WRREQ"][k]) - avg(wq["TCC_EA0_WRREQ_64B"][k]))
              for k in wq["TCC_EA0_WRREQ"]}
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("calibration copy missing from the counters")
    cf = COPY_BYTES / (sum(fetch["copy"]) / len(fetch["copy"]) * 1024)
    cw = COPY_BYTES / (sum(write["copy"]) / len(write["copy"]) * 1024)
    b, L, H, P, N, G, Q = (MAMBA2_2P7B.batch, MAMBA2_2P7B.seqlen, MAMBA2_2P7B.nheads,
                           MAMBA2_2P7B.headdim, MAMBA2_2P7B.dstate, MAMBA2_2P7B.ngroups,
                           MAMBA2_2P7B.chunk)
    import mamba_ssd_scan_02_amd as ssd
    import torch
    alg, _ = forward_model(b, L, H, P, N, G, Q,
                           ssd.forward_run_chunks(b, L, H, P, N, G, Q, torch.bfloat16))
    alg.update(layer_model(b, L, H, P, N, G, LAYER_K))
    db = DECODE_B256
    alg["ssm_step"] = (db.batch * db.nheads * db.headdim * db.dstate * 4 * 2 +
                       db.batch * db.nheads * db.headdim * 2 * 2 + db.batch * db.nheads * 4 +
                       2 * db.batch * db.ngroups * db.dstate * 2 + 2 * db.nheads * 4)
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        fk = sum(fetch[k]) / len(fetch[k]) * 1024 * cf
        wk = sum(write[k]) / len(write[k]) * 1024 * cw
        wl = DECODE_B256.name if k == "ssm_step" else MAMBA2_2P7B.name
        text = "\n".join([
            f"# HBM traffic of {k} on {wl} (rocprofv3 counters, calibrated)",
            f"command_fetch: {cmd_fetch}",
            f"command_write: {cmd_write}",
            f"calibration: a {COPY_BYTES}-byte device copy reads FETCH_SIZE x {cf:.4f} and writes "
            f"WRITE_SIZE x {cw:.4f} of its counter values (KiB per dispatch)",
            f"dispatches: {len(fetch[k])}",
            f"fetch_bytes_per_dispatch: {fk:.6g}",
            f"write_bytes_per_dispatch: {wk:.6g}",
            f"hbm_bytes_per_dispatch: {fk + wk:.6g}",
            f"algorithmic_bytes_per_dispatch: {alg[k]}",
            f"traffic_over_algorithmic: {(fk + wk) / alg[k]:.4f}",
        ] + ([
            f"command_read_requests: {cmd_rd}",
            f"command_write_requests: {cmd_wr}",
            "read_bytes_by_request_size: 32 x TCC_EA0_RDREQ_32B + 64 x TCC_EA0_RDREQ_64B + "
            "128 x TCC_EA0_RDREQ_128B (no calibration)",
            f"xcheck_copy_read_bytes: {xr['copy']:.6g} (copy reads {COPY_BYTES})",
            f"xcheck_read_bytes_per_dispatch: {xr[k]:.6g}",
            "write_bytes_by_request_size: 64 x TCC_EA0_WRREQ_64B + 32 x the rest",
            f"xcheck_copy_write_bytes: {xw['copy']:.6g} (copy writes {COPY_BYTES})",
            f"xcheck_write_bytes_per_dispatch: {xw[k]:.6g}",
        ] if xr is not None and k in xr and k in xw and "copy" in xr and "copy" in xw else []) + [
            f"source_sha256_16: {source_hash(k)}",
        ]) + "\n"
        outp = Path(out_dir) / f"{k}_{wl}_counters.txt"
        outp.write_text(text)
        print(text)


SQ_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
               "SQ_VALU_MFMA_BUSY_CYCLES"]


def summarize_sq(d: str, out_dir: str, cmd: str):
    """Per-kernel issue profile from one rocprofv3 --pmc pass over SQ_COUNTERS:
    averages per dispatch, and the wait / VALU / LDS / VMEM shares of the
    waves' cycles (as the counters report them, summed over the device)."""
    import csv
    import glob
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_2P7B, DECODE_B256
    f = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    acc = {}
    for r in csv.DictReader(open(f[0])):
        k = _short_kernel(r["Kernel_Name"])
        if k not in KERNEL_SOURCES:
            continue
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for k, cnt in acc.items():
        avg = {c: sum(v) / len(v) for c, v in cnt.items()}
        wc = avg.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        wl = DECODE_B256.name if k == "ssm_step" else MAMBA2_2P7B.name
        lines = [f"# issue profile of {k} on {wl} (rocprofv3 SQ counters, per dispatch)",
                 f"command: {cmd}",
                 f"dispatches: {len(next(iter(cnt.values())))}"]
        for c in SQ_COUNTERS:
            if c in avg:
                lines.append(f"{c}: {avg[c]:.6g}")
        for c, label in (("SQ_WAIT_ANY", "waiting"), ("SQ_WAIT_INST_ANY", "waiting to issue"),
                         ("SQ_ACTIVE_INST_VALU", "issuing VALU"), ("SQ_ACTIVE_INST_LDS", "issuing LDS"),
                         ("SQ_ACTIVE_INST_VMEM", "issuing VMEM")):
            if c in avg:
                lines.append(f"share_of_wave_cycles_{label.replace(' ', '_')}: {avg[c] / wc:.4f}")
        Path(out_dir, f"{k}_{wl}_issue.txt").write_text("\n".join(lines) + "\n")
        print("\n".join(lines))


# ---------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 130M-shaped and the one-million-token forwards printed beside "
                         "the headline")
    ap.add_argument("--workload", default="mamba2_2p7b_b4_l8192_h80_p64_n128",
                    choices=["mamba2_2p7b_b4_l8192_h80_p64_n128", "mamba2_130m_b8_l2048_h24_p64_n128",
                             "long_b1_l1048576_h32_p64_n128_g8"],
                    help="forward workload (the default is the headline one; the others print "
                         "the same line for the 130M-shaped layer and for one 1M-token sequence, "
                         "the latter without the block around the scan and the oracle baseline, "
                         "whose host-side inputs or fp64 work do not fit a short run)")
    ap.add_argument("--state-passing-long", action="store_true",
                    help="only compare sequential and segmented state passing at the "
                         "long-context shape")
    ap.add_argument("--profile-loop", type=int, default=0)
    ap.add_argument("--summarize-trace", default=None)
    ap.add_argument("--summarize-counters", nargs=2, default=None)
    ap.add_argument("--summarize-sq", default=None)
    ap.add_argument("--out", default=None)
    ap.add_argument("--out-dir", default="profiles")
    ap.add_argument("--cmd", default="", help="command recorded in a summary")
    ap.add_argument("--cmd2", default="", help="second command recorded in a summary")
    ap.add_argument("--xcheck", nargs=2, default=None,
                    help="with --summarize-counters: dirs of the TCC_EA0_RDREQ* and TCC_EA0_WRREQ* "
                         "passes (bytes counted per request size)")
    ap.add_argument("--cmd3", default="", help="read-request command recorded in a summary")
    ap.add_argument("--cmd4", default="", help="write-request command recorded in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.cmd)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.out_dir, args.cmd)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.out_dir,
                           args.cmd, args.cmd2, args.xcheck, args.cmd3, args.cmd4)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import FORWARD_SPECS, make_forward_inputs
    spec = FORWARD_SPECS[args.workload]
    if spec.seqlen > 65536:
        args.no_layer = args.no_cpu_baseline = True

    ssd.load()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    if args.profile_loop:
        profile_loop(args.profile_loop)
        return
    if args.state_passing_long:
        print(json.dumps(bench_state_passing_long()), flush=True)
        return
    dims = (spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups,
            spec.chunk)
    b, L, H, P, N, G, Q = dims
    log(f"[bench] generating {spec.name}")
    inp = make_forward_inputs(spec)
    g = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y = torch.empty_like(g["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(ssd.workspace_bytes(b, L, H, P, N, G, Q, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    headline = spec.name == "mamba2_2p7b_b4_l8192_h80_p64_n128"

    log(f"[bench] forward: {args.warmup} warmup + {args.steps} timed steps")
    ms, wall = time_forward(ssd, g, y, fin, ws, Q, args.steps, args.warmup)
    tokens_per_s = b * L / (ms * 1e-3)
    log(f"[bench] forward {ms * 1e3:.1f} us/step, {tokens_per_s:.4g} tokens/s")

    log("[bench] per-kernel event timing")
    K = ssd.forward_run_chunks(*dims, torch.bfloat16)
    k_us = time_stages(ssd, g, y, fin, dims, max(args.steps, 10), K)
    kbytes, kflops = forward_model(*dims, K)
    path = forward_kernels(dims, K)
    kernels = {}
    for n, us in k_us.items():
        gbs = kbytes[n] / (us * 1e-6) / 1e9
        tf = kflops[n] / (us * 1e-6) / 1e12
        kernels[n] = {"us": round(us, 2), "alg_bytes": kbytes[n], "GBps": round(gbs, 1),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "alg_flops": kflops[n],
                      "TFLOPs": round(tf, 2), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                      "in_forward": n in path}
    dom = max(path, key=lambda n: k_us[n])
    d_us = k_us[dom]
    achieved = kbytes[dom] / (d_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(dom, spec.name), "kernel": dom,
                "alg_bytes_per_launch": kbytes[dom], "avg_launch_us": round(d_us, 2),
                "timing": "HIP events on the launching stream, this run"}
    tr = trace_average(dom, spec.name)
    if tr is not None:
        roofline["trace_avg_us"], roofline["trace_file"] = tr
        roofline["trace_frac"] = round(kbytes[dom] / (tr[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    comp = compulsory_bytes(b, L, H, P, N, G)
    flops_total = sum(kflops[n] for n in path)

    out = {
        "metric": METRIC if headline else f"SSD fwd tokens/s at {spec.name}",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; x,dt,B,C,D,A,init drawn from the workload's distributions)",
        "config": {"workload": spec.name, "batch": b, "seqlen": L, "nheads": H, "headdim": P,
                   "dstate": N, "ngroups": G, "chunk": Q},
        "roofline": roofline,
        "path": {"hbm_frac_of_compulsory_bytes": round(comp / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac_algorithmic_flops": round(flops_total / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                 "compulsory_bytes": comp, "forward_kernels": path, "run_chunks": K,
                 "forward_kernel_bytes": sum(kbytes[n] for n in path),
                 "forward_kernel_event_sum_us": round(sum(k_us[n] for n in path), 2),
                 "algorithmic_flops": flops_total, "wall_s_timed_region": round(wall, 4)},
        "kernels": kernels,
    }
    if headline and not args.no_extra:
        from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M as s2
        log(f"[bench] {s2.name} forward")
        inp2 = make_forward_inputs(s2)
        g2 = {k: (v.cuda() if v is not None else None) for k, v in inp2.items()}
        y2 = torch.empty_like(g2["x"])
        f2 = torch.empty((s2.batch, s2.nheads, s2.headdim, s2.dstate), dtype=torch.float32,
                         device="cuda")
        ws2 = torch.empty(ssd.workspace_bytes(s2.batch, s2.seqlen, s2.nheads, s2.headdim, s2.dstate,
                                              s2.ngroups, s2.chunk, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        ms2, _ = time_forward(ssd, g2, y2, f2, ws2, s2.chunk, args.steps, args.warmup)
        dims2 = (s2.batch, s2.seqlen, s2.nheads, s2.headdim, s2.dstate, s2.ngroups, s2.chunk)
        out["forward_130m"] = {"workload": s2.name, "us_per_step": round(ms2 * 1e3, 2),
                               "tokens_per_s": round(s2.batch * s2.seqlen / (ms2 * 1e-3), 1),
                               "forward_kernels": forward_kernels(
                                   dims2, ssd.forward_run_chunks(*dims2, torch.bfloat16))}
        del g2, y2, f2, ws2
        # one sequence of 1,048,576 tokens (8 groups of 4 heads): few steps,
        # its seeded inputs take most of this leg's time to draw on the host
        from mamba_ssd_scan_02_amd.workloads import LONG_1M as s4
        log(f"[bench] {s4.name} forward")
        inp4 = make_forward_inputs(s4)
        g4 = {k: (v.cuda() if v is not None else None) for k, v in inp4.items()}
        del inp4
        y4 = torch.empty_like(g4["x"])
        f4 = torch.empty((s4.batch, s4.nheads, s4.headdim, s4.dstate), dtype=torch.float32,
                         device="cuda")
        ws4 = torch.empty(ssd.workspace_bytes(s4.batch, s4.seqlen, s4.nheads, s4.headdim, s4.dstate,
                                              s4.ngroups, s4.chunk, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        ms4, _ = time_forward(ssd, g4, y4, f4, ws4, s4.chunk, 5, 2)
        dims4 = (s4.batch, s4.seqlen, s4.nheads, s4.headdim, s4.dstate, s4.ngroups, s4.chunk)
        out["forward_long"] = {"workload": s4.name, "us_per_step": round(ms4 * 1e3, 2),
                               "tokens_per_s": round(s4.batch * s4.seqlen / (ms4 * 1e-3), 1),
                               "steps": 5, "forward_kernels": forward_kernels(
                                   dims4, ssd.forward_run_chunks(*dims4, torch.bfloat16))}
        del g4, y4, f4, ws4
    log("[bench] zero-order-hold forward")
    ms_zoh, _ = time_forward(ssd, g, y, fin, ws, Q, args.steps, args.warmup, zoh=True)
    out["forward_zoh"] = {"us_per_step": round(ms_zoh * 1e3, 2),
                          "tokens_per_s": round(b * L / (ms_zoh * 1e-3), 1)}
    if not args.no_decode:
        log("[bench] decode")
        out["decode"] = bench_decode(ssd)
        out["decode_small_batch"] = bench_decode_graph(ssd)
    if not args.no_layer:
        log("[bench] layer around the scan")
        out["layer"] = bench_layer(ssd, spec)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
