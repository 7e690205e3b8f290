"""Benchmark of the Mamba-3 SSM layer core on one MI355X.

One step = one mamba3_ssm_chunked_fwd (scans, RoPE, intra-chunk MFMA work,
chunk states and the inter-chunk pass: the whole prefill path) over the
1.5B-scale MIMO workload: batch 8, L=4096, H=64, P=64, N=64, R=4, chunk 64,
bf16 io, fp32 state, synthetic inputs drawn on the device.  Inputs are resident
in HBM before the timed region starts.

Printed: one JSON line with the prefill throughput (tokens/s), the roofline of
the walker kernel (HIP events on its stream), the decode workload (batch 256,
1024 consecutive one-token steps, fp32 state in HBM) with its achieved
bandwidth, the rope rotation, and the fp64 CPU oracle timed on a bounded
sample of the same prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only prefill|decode|rope]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
BF16_DENSE_TFLOPS = 2516.6       # MI355X dense bf16 MFMA


def prefill_bytes_per_token_head(w, s_io=2):
    """Algorithmic bytes: x, B, C read once, y written once, dt/A/lam fp32, theta fp32 (N/2 per token)."""
    return s_io * w.rank * (2 * w.headdim + 2 * w.dstate) + 12 + 2 * w.dstate


def subwalk_applies(w):
    """The sub-chunk walker's sizes (mirrors subwalk_supported in csrc/chunk_subwalk.hip)."""
    if w.io != "bf16" or w.headdim != 64:
        return False
    if w.dstate == 64:
        return w.chunk in (16, 32, 64) and w.rank in (1, 2, 4)  # shorter chunks walked at the sub-chunk length
    return w.dstate == 128 and w.chunk in (16, 32, 64) and w.rank in (2, 4)


def walked_chunk(w):
    """Chunk length the library walks with: the sub-chunk walker walks 32-token
    (N = 64; 64-token for R = 1) or 16-token (N = 128) pieces of the requested
    chunk (a shorter requested chunk at its own length)."""
    if subwalk_applies(w):
        return (64 if w.rank == 1 else 32) if w.dstate == 64 else 16
    return w.chunk


def walker_kernel(w):
    if subwalk_applies(w):
        return f"subchunk_walk_kernel<{w.dstate},{w.rank}>"
    if w.io == "bf16" and w.dstate <= 64 and w.headdim <= 64:
        return f"chunk_walk_fast_kernel<{w.dstate},{w.headdim},{w.rank}>"
    return f"chunk_walk_kernel<{w.io},{w.dstate},{w.headdim},8>"


def prefill_flops_per_token_head(w, causal, at_configured_chunk=False):
    """MFMA work of the chunked algorithm at the walked chunk length Q (what
    the matrix cores execute), or at the workload's configured chunk (the
    fixed algorithmic count of the chunked form with that chunk): scores and
    masked scores x X within the chunk (Q R x Q R, causal or dense), the
    inter-chunk output C H' and the chunk state (w B)^T X."""
    Q = w.chunk if at_configured_chunk else walked_chunk(w)
    R, N, P = w.rank, w.dstate, w.headdim
    if causal:
        return R * R * (N + P) * (Q + 1) + 4 * R * N * P
    return 2 * Q * R * R * (N + P) + 4 * R * N * P


def decode_bytes_per_step(w, s_io=2):
    BH, N, P, R = w.batch * w.nheads, w.dstate, w.headdim, w.rank
    state = 2 * BH * N * P * 4
    inputs = BH * (R * P + 2 * R * N) * s_io + BH * (R * N + R * P) * s_io  # x, B, C + prev_B, prev_x
    scal = BH * (3 * 4 + (N // 2) * 4)
    y = BH * R * P * s_io
    return state + inputs + scal + y


def rope_bytes_per_token_head(w, s_io=2):
    return 4 * w.rank * w.dstate * s_io + 4 + 2 * w.dstate


def timed(fn, steps, warmup, torch):
    """Run fn warmup+steps times; returns (wall ms/step, event ms/step on the current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, e0.elapsed_time(e1) / steps


def step_percentiles(fn, steps, torch):
    """p10 / p50 / p90 of single-step times (HIP events around each step)."""
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    pick = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return pick(0.1), pick(0.5), pick(0.9)


def settle(fn, torch, seconds=0.3):
    """Untimed calls for a fixed stretch of wall time, whatever the warm-up
    count: the first launches after the inputs are drawn run slower while the
    clocks settle, and a short warm-up would fold that into the timed mean."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def bench_prefill(ops, inputs, w, steps, warmup, torch):
    d = inputs.torch_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, io=w.io,
                            seed=inputs.seed_of(w.name))
    y = torch.empty_like(d["x"])
    hf = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), device="cuda", dtype=torch.float32)
    fn = lambda: ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], chunk=w.chunk,
                                 y=y, h_final=hf)
    settle(fn, torch)
    wall, ev = timed(fn, steps, warmup, torch)
    pct = step_percentiles(fn, steps, torch)
    th = w.batch * w.seqlen * w.nheads
    bytes_ = th * prefill_bytes_per_token_head(w)
    dense = th * prefill_flops_per_token_head(w, False)
    causal = th * prefill_flops_per_token_head(w, True)
    dense_cfg = th * prefill_flops_per_token_head(w, False, at_configured_chunk=True)
    del d, y, hf
    torch.cuda.empty_cache()
    return dict(ms=ev, wall_ms=wall, tokens_per_s=w.tokens / (ev * 1e-3), bytes=bytes_,
                gbps=bytes_ / (ev * 1e-3) / 1e9, tflops_dense=dense / (ev * 1e-3) / 1e12,
                tflops_dense_cfg=dense_cfg / (ev * 1e-3) / 1e12,
                tflops_causal=causal / (ev * 1e-3) / 1e12, p10_p50_p90=pct)


def bench_decode(ops, inputs, w, torch, reps=3):
    """1024 consecutive one-token steps (step t passes step t-1's raw B and x as
    prev), captured once in a HIP graph so that Python launch overhead does not
    starve the GPU; each replay is timed with HIP events on the capture stream."""
    steps = w.decode_steps
    d = inputs.torch_inputs(w.batch, steps, w.nheads, w.headdim, w.dstate, w.rank, io=w.io,
                            seed=inputs.seed_of(w.name), with_h0=True)
    sm = {k: d[k].transpose(0, 1).contiguous() for k in ("x", "B", "C", "dt", "A", "lam", "theta")}
    h0 = d["h0"]
    del d
    torch.cuda.empty_cache()
    state = h0.clone()
    y = torch.empty(sm["x"].shape[1:], dtype=sm["x"].dtype, device="cuda")

    def run_all():
        for t in range(steps):
            pb = sm["B"][t - 1] if t > 0 else None
            px = sm["x"][t - 1] if t > 0 else None
            ops.decode_step(state, sm["x"][t], sm["B"][t], sm["C"][t], sm["dt"][t], sm["A"][t], sm["lam"][t],
                            sm["theta"][t], pb, px, y=y)

    run_all()  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    per_step = []
    for _ in range(reps):
        state.copy_(h0)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        per_step.append(e0.elapsed_time(e1) / steps)
    per_step = sorted(per_step)[len(per_step) // 2]
    b = decode_bytes_per_step(w)
    del sm, state, y, h0, g
    torch.cuda.empty_cache()
    return dict(steps=steps, ms_per_step=per_step, steps_per_s=1e3 / per_step, bytes_per_step=b,
                gbps=b / (per_step * 1e-3) / 1e9)


def verify_bytes_per_call(w, k, s_io=2):
    """k tokens on a decode state: the state read and written once, the
    previous token's B and x once, and per token x, B, C, dt, A, lam, theta, y."""
    BH, N, P, R = w.batch * w.nheads, w.dstate, w.headdim, w.rank
    state = 2 * BH * N * P * 4
    prev = BH * (R * N + R * P) * s_io
    per_token = BH * ((R * P + 2 * R * N) * s_io + 3 * 4 + (N // 2) * 4 + R * P * s_io)
    return state + prev + k * per_token


def bench_verify(ops, inputs, w, k, steps, warmup, torch):
    """k tokens per call on the decode state (chunked_fwd with h0 = h_final =
    the state, prev given): the short-sequence path, and the chunk walk forced
    for comparison."""
    d = inputs.torch_inputs(w.batch, k, w.nheads, w.headdim, w.dstate, w.rank, io=w.io,
                            seed=inputs.seed_of(w.name) + k, with_h0=True)
    d["prev_B"], d["prev_x"] = d["B"][:, 0].contiguous(), d["x"][:, 0].contiguous()  # any token of the same draw
    state = d["h0"].clone()
    y = torch.empty_like(d["x"])
    res = {}
    for name, walk, tok in (("default", False, False), ("token_path", False, True), ("chunk_walk", True, False)):
        fn = lambda: ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=state,
                                     prev_B=d["prev_B"], prev_x=d["prev_x"], chunk=w.chunk, chunk_walk=walk,
                                     token_path=tok, y=y, h_final=state)
        settle(fn, torch, 0.1)
        wall, ev = timed(fn, steps, warmup, torch)
        res[name] = ev
    b = verify_bytes_per_call(w, k)
    del d, state, y
    torch.cuda.empty_cache()
    ms = res["default"]
    return dict(k=k, ms_per_call=ms, tokens_per_s=w.batch * k / (ms * 1e-3), bytes_per_call=b,
                gbps=b / (ms * 1e-3) / 1e9, token_path_ms=res["token_path"], chunk_walk_ms=res["chunk_walk"])


def bwd_chunk(w):
    """Tokens per chunk of the backward walk: 16, or 8 when N or P is 128
    and R = 4."""
    return 8 if (w.dstate > 64 or w.headdim > 64) and w.rank == 4 else 16


def backward_flops_per_token_head(w):
    """Dense MFMA flops of the backward per token-head, as (checkpoint walk,
    reverse walk): per chunk of Q = 16 tokens (8 when N or P is 128 and
    R = 4; V = Q R rows) the checkpoint walk's
    state product W^T X and the reverse walk's nine products (G, dGM, two for
    dX, two for dC~, two for dB~ and dH_in), each 2 M N K. With bf16 io all of
    them run on bf16 MFMAs, the checkpoint product twice (bf16 hi and lo parts
    of W)."""
    Q = bwd_chunk(w)
    V, N, P = Q * w.rank, w.dstate, w.headdim
    ckpt = 2 * (N * P * V)
    walk = 2 * (V * V * N + V * V * P + V * P * V + V * P * N + V * N * V + V * N * P + V * N * V + V * N * P
                + N * P * V)
    return ckpt / Q, walk / Q


def backward_bytes_per_token_head(w, s_io=2):
    """Algorithmic HBM bytes: x, B, C, dy, dt, A, lam, theta read; dx, dB,
    dC, ddt, dA, dlam, dtheta written; the chunk-start states written once
    and read once."""
    R, N, P = w.rank, w.dstate, w.headdim
    io_in = s_io * R * (2 * P + 2 * N) + 12 + 2 * N
    io_out = s_io * R * (P + 2 * N) + 12 + 2 * N
    states = 2 * N * P * 4 / bwd_chunk(w)
    return io_in + io_out + states


def bench_backward(ops, inputs, w, steps, warmup, torch):
    """mamba3_ssm_chunked_bwd on the prefill workload with dy ~ N(0, 1)."""
    d = inputs.torch_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, io=w.io,
                            seed=inputs.seed_of(w.name) + 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(inputs.seed_of(w.name) + 2)
    dy = torch.randn(d["x"].shape, generator=g, device="cuda", dtype=torch.float32).to(d["x"].dtype)
    dims = ops.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, w.chunk, ops._io_code(d["x"]))
    ws = torch.empty(ops.chunked_bwd_workspace_size(dims), device="cuda", dtype=torch.uint8)
    fn = lambda: ops.chunked_bwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], dy, chunk=w.chunk,
                                 want_dh0=False, workspace=ws)
    wall, ev = timed(fn, steps, warmup, torch)
    th = w.batch * w.seqlen * w.nheads
    ck_fl, walk_fl = (th * f for f in backward_flops_per_token_head(w))
    flops = ck_fl + walk_fl
    bytes_ = th * backward_bytes_per_token_head(w)
    # time floors: the issued products at the dense bf16 MFMA peak, the bytes at the HBM peak
    mfma_floor_ms = (2 * ck_fl + walk_fl) / (BF16_DENSE_TFLOPS * 1e12) * 1e3
    hbm_floor_ms = bytes_ / (HBM_PEAK_GBPS * 1e9) * 1e3
    del d, dy, ws
    torch.cuda.empty_cache()
    return dict(ms=ev, tokens_per_s=w.tokens / (ev * 1e-3), tflops=flops / (ev * 1e-3) / 1e12, flops=flops,
                gbps=bytes_ / (ev * 1e-3) / 1e9, bytes=bytes_, mfma_floor_ms=mfma_floor_ms, hbm_floor_ms=hbm_floor_ms)


def bench_prologue(ops, inputs, steps, warmup, torch):
    """mamba3_bc_prologue at the 1.5B shapes: flops of the projection (2 M F D,
    M = B L tokens, F = 2 H R N features) and bytes of u, W, dt, theta read
    and B_rot, C_rot written (the angle pre-pass writes and re-reads 4 bytes
    per token, head and pair on top)."""
    c = inputs.PROLOGUE
    b, L, H, R, N, D = c["batch"], c["seqlen"], c["nheads"], c["rank"], c["dstate"], c["d_model"]
    d = inputs.prologue_torch(b, L, H, N, R, D, seed=inputs.PROLOGUE_SEED)
    dims = ops.make_dims(b, L, H, 16, N, R, 16, ops.M3_BF16)
    ws = torch.empty(ops.bc_prologue_workspace_size(dims), device="cuda", dtype=torch.uint8)
    Bo = torch.empty((b, L, H, R, N), device="cuda", dtype=torch.bfloat16)
    Co = torch.empty_like(Bo)
    fn = lambda: ops.bc_prologue(d["u"], d["W"], d["dt"], d["theta"], H, R, N, gain=d["gain"], bias=d["bias"],
                                 B_rot=Bo, C_rot=Co, want_final=False, workspace=ws)
    wall, ev = timed(fn, steps, warmup, torch)
    M, F = b * L, 2 * H * R * N
    flops = 2.0 * M * F * D
    bytes_ = 2 * M * D + 2 * F * D + 8 * F + M * H * (4 + 4 * N // 2) + 2 * M * F
    del d, ws, Bo, Co
    torch.cuda.empty_cache()
    return dict(ms=ev, flops=flops, tflops=flops / (ev * 1e-3) / 1e12, bytes=bytes_, gbps=bytes_ / (ev * 1e-3) / 1e9,
                tokens_per_s=M / (ev * 1e-3), shape=dict(batch=b, seqlen=L, nheads=H, rank=R, dstate=N, d_model=D))


def bench_rope(ops, inputs, w, steps, warmup, torch):
    d = inputs.torch_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, io=w.io,
                            seed=inputs.seed_of(w.name))
    Br, Cr = torch.empty_like(d["B"]), torch.empty_like(d["C"])
    fn = lambda: ops.rope_bc(d["B"], d["C"], d["dt"], d["theta"], B_rot=Br, C_rot=Cr)
    wall, ev = timed(fn, steps, warmup, torch)
    th = w.batch * w.seqlen * w.nheads
    b = th * rope_bytes_per_token_head(w)
    del d, Br, Cr
    torch.cuda.empty_cache()
    return dict(ms=ev, gbps=b / (ev * 1e-3) / 1e9, bytes=b)


def host_cores():
    """(logical CPUs this process may run on, physical cores of the host)."""
    try:
        logical = len(os.sched_getaffinity(0))
    except AttributeError:
        logical = os.cpu_count() or 1
    phys = set()
    try:
        pid = cid = None
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("physical id"):
                pid = ln.split(":")[1].strip()
            elif ln.startswith("core id"):
                cid = ln.split(":")[1].strip()
            elif not ln.strip() and cid is not None:
                phys.add((pid, cid))
                pid = cid = None
        if cid is not None:
            phys.add((pid, cid))
    except OSError:
        pass
    return logical, (len(phys) or None)


def cpu_baseline(inputs, w, budget_s=8.0, decode=False):
    """The fp64 oracle (as it stands) on a bounded sample of the workload: a set
    of (b,h) slices over the full sequence (for decode: the workload's 1024
    consecutive steps, which the oracle's token-by-token recurrence is), one
    host thread per slice, timed over repeated calls for about budget_s.  The
    rate is scaled to the whole workload: tokens/s for prefill, steps/s (all
    B*H slices advanced by one token) for decode."""
    import oracle
    logical, physical = host_cores()
    cores = min(logical, int(os.environ.get("OMP_NUM_THREADS", logical)))
    total = w.batch * w.nheads
    L = w.decode_steps if decode else w.seqlen
    nsl = min(total, cores)
    t = inputs.torch_inputs(nsl, L, 1, w.headdim, w.dstate, w.rank, io=w.io, seed=6, device="cpu",
                            with_h0=decode)
    s = {k: v.float().numpy() for k, v in t.items()}
    reps, el = 0, 0.0
    while el < budget_s:
        t0 = time.perf_counter()
        oracle.forward(s["x"], s["B"], s["C"], s["dt"], s["A"], s["lam"], s["theta"], h0=s.get("h0"),
                       nthreads=nsl)
        el += time.perf_counter() - t0
        reps += 1
    slice_tokens_per_s = reps * nsl * L / el
    out = dict(unit="steps/s" if decode else "tokens/s", cores=nsl, kind="oracle",
               logical_cpus=logical, physical_cores=physical)
    if decode:
        out["value"] = slice_tokens_per_s / total
        out["sample"] = (f"{nsl} of the {total} (b,h) slices x {L} consecutive steps of {w.name}, {reps} call(s) in "
                         f"{el:.1f} s on {nsl} threads; steps/s = slice-steps/s / {total} slices")
    else:
        out["value"] = slice_tokens_per_s / w.nheads
        out["sample"] = (f"{nsl} of the {total} (b,h) slices x L={L} of {w.name}, {reps} call(s) in {el:.1f} s on "
                         f"{nsl} threads; tokens/s = token-heads/s / H={w.nheads}")
    out["value"] = round(out["value"], 3)
    return out


def bench_copy(torch, nbytes=1 << 30, reps=3):
    """A plain device copy of known size: the reference for scaling the FETCH_SIZE
    and WRITE_SIZE counters to bytes (run under rocprofv3 --pmc)."""
    src = torch.randn(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return dict(bytes_read=nbytes, bytes_written=nbytes, ms=ms, gbps=2 * nbytes / (ms * 1e-3) / 1e9)


def bench_floor(torch, w, reps=10):
    """Memory floors of this GPU for the prefill walker's traffic (the probes
    of libm3_floor.so move the same bytes with no arithmetic): the walker's own
    access pattern (one block per (b,h), two per compute unit; and two adjacent
    heads per block), the same bytes as contiguous streams (3:1 and 1:1
    read:write), and an in-place read-modify-write below and above the 256 MB
    memory-side cache (the decode state's traffic).  GB/s counts the bytes
    each probe is given to move.  Also the achievable bf16 MFMA rate of
    16x16x32 and 32x32x16 products with no memory traffic."""
    import ctypes
    from state_space_sequence_03_amd import build
    lib = ctypes.CDLL(build.FLOOR_LIB)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.m3f_stream.argtypes = [ci, vp, vp, vp, vp, i64, ci, vp]
    lib.m3f_walk.argtypes = [vp] * 8 + [i64, i64, i64, ci, ci, ci, ci, vp]
    lib.m3f_rmw.argtypes = [vp, i64, ci, vp]
    b, L, H, P, N, R = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank
    assert (P, N, R) == (64, 64, 4)
    u8 = torch.uint8
    x, Bt, Ct, y = (torch.zeros(b * L * H * R * P * 2, dtype=u8, device="cuda") for _ in range(4))
    th = torch.zeros(b * L * H * N // 2 * 4, dtype=u8, device="cuda")
    dt, A, lam = (torch.zeros(b * L * H * 4, dtype=u8, device="cuda") for _ in range(3))
    s = torch.cuda.current_stream()
    sp = ctypes.c_void_p(s.cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def t_ms(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    walk_bytes = b * L * H * prefill_bytes_per_token_head(w)
    out = {}
    for name, hpb, lds in (("walker_pattern_2_blocks_per_cu", 1, 80 * 1024), ("walker_pattern_2_heads_per_block", 2, 160 * 1024),
                           ("walker_pattern_8_blocks_per_cu", 1, 0)):
        fn = lambda: lib.m3f_walk(ptr(x), ptr(Bt), ptr(Ct), ptr(th), ptr(dt), ptr(A), ptr(lam), ptr(y), b, L, H, 64, 4,
                                  hpb, lds, sp)
        assert fn() == 0
        ms = t_ms(fn)
        out[name] = dict(ms=round(ms, 4), GBps=round(walk_bytes / (ms * 1e-3) / 1e9, 1))
    # the SISO walker's pattern (R = 1: rows of 128 B, 64-token sub-chunks) on the siso_bf16 bytes
    import dataclasses
    ws = dataclasses.replace(w, rank=1, name="siso_bf16")
    siso_bytes = b * L * H * prefill_bytes_per_token_head(ws)
    for name, hpb in (("siso_walker_pattern_2_blocks_per_cu", 1), ("siso_walker_pattern_2_heads_per_block", 2)):
        fn = lambda: lib.m3f_walk(ptr(x), ptr(Bt), ptr(Ct), ptr(th), ptr(dt), ptr(A), ptr(lam), ptr(y), b, L, H, 64, 1,
                                  hpb, 80 * 1024, sp)
        assert fn() == 0
        ms = t_ms(fn)
        out[name] = dict(ms=round(ms, 4), GBps=round(siso_bytes / (ms * 1e-3) / 1e9, 1))
    n16 = x.numel() // 16
    for name, nr in (("stream_3_read_1_write", 3), ("stream_1_read_1_write", 1)):
        for blocks in (2048, 8192):
            fn = lambda: lib.m3f_stream(nr, ptr(x), ptr(Bt), ptr(Ct), ptr(y), n16, blocks, sp)
            ms = t_ms(fn)
            out[f"{name}_{blocks}_blocks"] = dict(ms=round(ms, 4), GBps=round((nr + 1) * x.numel() / (ms * 1e-3) / 1e9, 1))
    del x, Bt, Ct, y, th, dt, A, lam
    torch.cuda.empty_cache()
    # the long-context walker's pattern (N = 128, R = 4, 16-token sub-chunks) on the long_mimo_bf16 bytes, as
    # the library walks it: 512 walkers (32 heads x 16 segments of 4,096 tokens), here a batch of 16 sequences
    # of 4,096 tokens (the same rows and strides within a segment)
    from state_space_sequence_03_amd import inputs as inputs_mod
    wl = inputs_mod.WORKLOADS["long_mimo_bf16"]
    lb, lL, lH, lN = 16, wl.seqlen // 16, wl.nheads, wl.dstate
    ntok = lb * lL * lH
    lx, ly = (torch.zeros(ntok * R * P * 2, dtype=u8, device="cuda") for _ in range(2))
    lB, lC = (torch.zeros(ntok * R * lN * 2, dtype=u8, device="cuda") for _ in range(2))
    lth = torch.zeros(ntok * lN // 2 * 4, dtype=u8, device="cuda")
    ldt, lA, llam = (torch.zeros(ntok * 4, dtype=u8, device="cuda") for _ in range(3))
    fn = lambda: lib.m3f_walk(ptr(lx), ptr(lB), ptr(lC), ptr(lth), ptr(ldt), ptr(lA), ptr(llam), ptr(ly), lb, lL, lH,
                              lN, 4, 1, 80 * 1024, sp)
    assert fn() == 0
    ms = t_ms(fn)
    out["long_walker_pattern_2_blocks_per_cu"] = dict(
        ms=round(ms, 4), GBps=round(ntok * prefill_bytes_per_token_head(wl) / (ms * 1e-3) / 1e9, 1))
    del lx, ly, lB, lC, lth, ldt, lA, llam
    torch.cuda.empty_cache()
    for name, nbytes in (("rmw_268MB", 268435456), ("rmw_2GB", 2 << 30)):
        buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
        fn = lambda: lib.m3f_rmw(ptr(buf), nbytes // 16, 4096, sp)
        ms = t_ms(fn)
        out[name] = dict(ms=round(ms, 4), GBps=round(2 * nbytes / (ms * 1e-3) / 1e9, 1))
        del buf
    torch.cuda.empty_cache()
    # the achievable bf16 MFMA rate: 8 independent chains per wave, operands in
    # registers, 512 blocks of 4 waves (two waves per SIMD)
    lib.m3f_mfma.argtypes = [ci, ci, ci, ci, vp, vp]
    blocks, iters = 512, 4096
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    for name, kind, fpm in (("mfma_loop_16x16x32_bf16", 0, 16384), ("mfma_loop_32x32x16_bf16", 1, 32768)):
        fn = lambda: lib.m3f_mfma(kind, iters, blocks, 0, ptr(sink), sp)
        assert fn() == 0
        ms = t_ms(fn)
        tf = blocks * 4 * 8 * iters * fpm / (ms * 1e-3) / 1e12
        out[name] = dict(ms=round(ms, 4), TFLOPs=round(tf, 1), frac_of_peak=round(tf / BF16_DENSE_TFLOPS, 4))
    del sink
    return out


def bench_gemm_reference(torch, inputs, reps=10):
    """Context for the B/C prologue: the vendor library's plain bf16 GEMM
    (torch.matmul, i.e. hipBLASLt) of the prologue's projection shape, with no
    normalisation, rotation or fused stores.  Not part of any path."""
    c = inputs.PROLOGUE
    M, F, D = c["batch"] * c["seqlen"], 2 * c["nheads"] * c["rank"] * c["dstate"], c["d_model"]
    u = torch.randn(M, D, device="cuda", dtype=torch.bfloat16)
    W = torch.randn(F, D, device="cuda", dtype=torch.bfloat16)
    fn = lambda: torch.matmul(W, u.t())
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del u, W
    torch.cuda.empty_cache()
    return {"library_gemm_prologue_shape": dict(M=M, F=F, D=D, ms=round(ms, 4),
                                                TFLOPs=round(2.0 * M * F * D / (ms * 1e-3) / 1e12, 1))}


def bench_decode_batches(ops, inputs, torch, batches=(256, 1024), steps=32):
    """The library's decode step at the decode workload's head shape with the
    fp32 state below (batch 256: 268 MB) and far above (batch 1024: 1.07 GB)
    the 256 MB memory-side cache: 32 consecutive steps in one HIP graph,
    median of 5 replays, algorithmic bytes per step / time."""
    from types import SimpleNamespace
    out = {}
    for batch in batches:
        d = inputs.torch_inputs(batch, steps, 64, 64, 64, 4, io="bf16", seed=5, with_h0=True)
        sm = {k: d[k].transpose(0, 1).contiguous() for k in ("x", "B", "C", "dt", "A", "lam", "theta")}
        st = d["h0"].clone()
        y = torch.empty(sm["x"].shape[1:], dtype=torch.bfloat16, device="cuda")

        def run():
            for t in range(steps):
                ops.decode_step(st, sm["x"][t], sm["B"][t], sm["C"][t], sm["dt"][t], sm["A"][t], sm["lam"][t],
                                sm["theta"][t], sm["B"][t - 1] if t else None, sm["x"][t - 1] if t else None, y=y)

        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / steps)
        ms = sorted(ts)[len(ts) // 2]
        b = decode_bytes_per_step(SimpleNamespace(batch=batch, nheads=64, dstate=64, headdim=64, rank=4))
        out[f"decode_batch_{batch}"] = dict(state_MB=round(batch * 64 * 64 * 64 * 4 / 1e6, 1), ms_per_step=round(ms, 5),
                                            GBps=round(b / (ms * 1e-3) / 1e9, 1))
        del d, sm, st, y, g
        torch.cuda.empty_cache()
    return out


# Counter summaries under profiles/ (FETCH_SIZE and WRITE_SIZE per dispatch,
# each scaled by what the same counter reads for a plain copy of known size),
# valid while the kernel's sources hash to the value recorded in them.
_CS = "state_space_sequence_03_amd/csrc/"
WALKER_SOURCES = tuple(_CS + f for f in ("chunk_subwalk.hip", "m3_common.hpp", "m3_lanes.hpp", "m3_order.hpp"))
# counter summary of the dominant kernel per workload, and the sources that kernel is built from
TRAFFIC = {
    "mimo_bf16": ("profiles/subchunk_walk_kernel_64_4__mimo_bf16__hbm_traffic.md", WALKER_SOURCES),
    "siso_bf16": ("profiles/subchunk_walk_kernel_64_1__siso_bf16__hbm_traffic.md", WALKER_SOURCES),
    "long_mimo_bf16": ("profiles/subchunk_walk_kernel_128_4__long_mimo_bf16__hbm_traffic.md", WALKER_SOURCES),
    "decode": ("profiles/decode_step_kernel_64_64_4__decode_mimo_bf16__hbm_traffic.md",
               tuple(_CS + f for f in ("decode.hip", "m3_common.hpp", "m3_lanes.hpp"))),
}


def source_sha256(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# sources bc_prologue_kernel is built from, and the summary of its measured graphics clock
PROLOGUE_SOURCES = tuple(_CS + f for f in ("prologue.hip", "m3_common.hpp", "m3_lanes.hpp", "m3_launch.hpp"))
CLOCK_SUMMARY = "profiles/gpu_clock__per_kernel.md"
ENGINE_CLOCK_GHZ = 2.4  # the engine clock the published peaks are quoted at


# SQ counter summary of the dominant prefill kernel per workload (SQ_INSTS_MFMA per dispatch)
SQ_SUMMARY = {
    "mimo_bf16": "profiles/subchunk_walk_kernel_64_4__mimo_bf16__sq_counters.md",
    "siso_bf16": "profiles/subchunk_walk_kernel_64_1__siso_bf16__sq_counters.md",
    "long_mimo_bf16": "profiles/subchunk_walk_kernel_128_4__long_mimo_bf16__sq_counters.md",
}


def summary_values(path, sources):
    """The '- key: value' lines of a committed counter summary, or None when it
    is missing or was taken on other sources."""
    path = os.path.join(ROOT, path)
    if not os.path.exists(path):
        return None
    vals = dict(re.findall(r"^- (\w+): ([0-9a-fA-F.e+-]+)\s*$", open(path).read(), re.M))
    if vals.get("source_sha256") != source_sha256(sources):
        return None
    return vals


def issued_mfma_flops(name):
    """MFMA flops one dispatch of the workload's walker issues, from the
    SQ_INSTS_MFMA counter of its committed summary (None if stale)."""
    vals = summary_values(SQ_SUMMARY[name], WALKER_SOURCES) if name in SQ_SUMMARY else None
    try:
        return float(vals["mfma_insts_per_dispatch"]) * float(vals["flop_per_mfma"]) if vals else None
    except (KeyError, ValueError):
        return None


def prologue_clock_ghz():
    """Average graphics clock of bc_prologue_kernel from its committed
    GRBM_COUNT summary (None if missing or taken on other sources)."""
    vals = summary_values(CLOCK_SUMMARY, PROLOGUE_SOURCES)
    try:
        return float(vals["prologue_clock_ghz"]) if vals else None
    except (KeyError, ValueError):
        return None


def measured_traffic(which="mimo_bf16"):
    """HBM bytes per dispatch of a kernel from its committed counter summary,
    or None when the summary is missing or was taken on other sources."""
    summary, sources = TRAFFIC[which]
    path = os.path.join(ROOT, summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    vals = dict(re.findall(r"^- (\w+): ([0-9a-fA-F.e+-]+)\s*$", text, re.M))
    try:
        sha = vals.get("source_sha256", vals.get("walker_source_sha256"))
        if sha != source_sha256(sources):
            return None
        return (float(vals["fetch_kib_per_dispatch"]) * float(vals["fetch_scale"])
                + float(vals["write_kib_per_dispatch"]) * float(vals["write_scale"])) * 1024.0
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "verify", "backward", "rope", "prologue", "copy", "floor", "all"],
                    default="all")
    ap.add_argument("--verify-k", type=int, default=8, help="tokens per call of the verify workload")
    ap.add_argument("--workload", default="mimo_bf16", choices=["mimo_bf16", "siso_bf16", "long_mimo_bf16"],
                    help="prefill workload timed by --only prefill (profiling); the headline line uses mimo_bf16")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the (b,h) slices of this "
              "workload shard over batch x heads with no communication", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.only == "copy":
        print(json.dumps({"copy": bench_copy(torch)}), flush=True)
        return
    if args.only == "floor":
        from state_space_sequence_03_amd import inputs
        from state_space_sequence_03_amd import ops
        fl = bench_floor(torch, inputs.WORKLOADS["mimo_bf16"])
        fl.update(bench_decode_batches(ops, inputs, torch))
        fl.update(bench_gemm_reference(torch, inputs))
        print(json.dumps({"floor": fl}), flush=True)
        return
    from state_space_sequence_03_amd import ops, inputs
    ops.lib()
    W = inputs.WORKLOADS
    w = W["mimo_bf16"] if args.only != "prefill" else W[args.workload]
    out = {}
    if args.only in ("prefill", "all"):
        print(f"[bench] prefill {w.name}: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
        pf = bench_prefill(ops, inputs, w, args.steps, args.warmup, torch)
        out["prefill"] = pf
    if args.only in ("decode", "all"):
        wd = W["decode_mimo_bf16"]
        print(f"[bench] decode {wd.name}: {wd.decode_steps} steps", file=sys.stderr, flush=True)
        out["decode"] = bench_decode(ops, inputs, wd, torch)
    if args.only in ("verify", "all"):
        wd = W["decode_mimo_bf16"]
        print(f"[bench] verify: {args.verify_k} tokens per call on {wd.name} shapes", file=sys.stderr, flush=True)
        out["verify"] = bench_verify(ops, inputs, wd, args.verify_k, args.steps, args.warmup, torch)
    if args.only in ("backward", "all"):
        print(f"[bench] backward on {w.name}", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(ops, inputs, w, max(3, args.steps // 4), 2, torch)
    if args.only in ("prologue", "all"):
        print("[bench] bc_prologue at the 1.5B shapes", file=sys.stderr, flush=True)
        out["prologue"] = bench_prologue(ops, inputs, max(3, args.steps // 2), 2, torch)
    if args.only in ("rope", "all"):
        print(f"[bench] rope_bc on {w.name} shapes", file=sys.stderr, flush=True)
        out["rope"] = bench_rope(ops, inputs, w, max(3, args.steps // 4), 2, torch)
    if args.only == "all":
        for name in ("siso_bf16", "long_mimo_bf16"):
            print(f"[bench] prefill {name} (context)", file=sys.stderr, flush=True)
            out[name] = bench_prefill(ops, inputs, W[name], 5, 2, torch)
        import dataclasses
        print("[bench] prefill mimo_bf16 at chunk 16 = N/R (context)", file=sys.stderr, flush=True)
        out["chunk16"] = bench_prefill(ops, inputs, dataclasses.replace(W["mimo_bf16"], chunk=16), 5, 2, torch)
        print("[bench] backward long_mimo_bf16 (context)", file=sys.stderr, flush=True)
        out["backward_long"] = bench_backward(ops, inputs, W["long_mimo_bf16"], 3, 1, torch)

    line = {"metric": "SSM prefill tokens/s + %MFMA peak (R=4); decode steps/s + HBM GB/s",
            "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{w.name} prefill: batch {w.batch}, L={w.seqlen}, H={w.nheads}, P={w.headdim}, "
                                   f"N={w.dstate}, R={w.rank}, chunk {w.chunk} (walked as {walked_chunk(w)}-token "
                                   f"chunks), {w.io} io, fp32 state",
                       "global_batch": w.batch, "seq_len": w.seqlen,
                       "parallelism": "single GPU"}}
    if "prefill" in out:
        pf = out["prefill"]
        line["value"] = round(pf["tokens_per_s"], 1)
        line["ms_per_step"] = round(pf["ms"], 4)
        traffic = measured_traffic(w.name) if w.name in TRAFFIC else None
        line["roofline"] = {"bound": "hbm", "achieved": round(pf["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(pf["gbps"] / HBM_PEAK_GBPS, 4),
                            "traffic": None if traffic is None else round(traffic),
                            "kernel": walker_kernel(w),
                            "bytes_per_launch": pf["bytes"]}
        line["ms_p10_p50_p90"] = [round(v, 4) for v in pf["p10_p50_p90"]]
        line["mfma"] = {"tflops_dense": round(pf["tflops_dense"], 1), "tflops_causal": round(pf["tflops_causal"], 1),
                        "frac_dense": round(pf["tflops_dense"] / BF16_DENSE_TFLOPS, 4),
                        "tflops_dense_at_configured_chunk": round(pf["tflops_dense_cfg"], 1),
                        "frac_dense_at_configured_chunk": round(pf["tflops_dense_cfg"] / BF16_DENSE_TFLOPS, 4),
                        "frac_causal": round(pf["tflops_causal"] / BF16_DENSE_TFLOPS, 4), "peak_tflops": BF16_DENSE_TFLOPS}
        fl = issued_mfma_flops(w.name)
        if fl is not None:  # what the matrix cores executed: SQ_INSTS_MFMA of the committed profile, this run's time
            line["mfma"]["tflops_issued_counters"] = round(fl / (pf["ms"] * 1e-3) / 1e12, 1)
            line["mfma"]["frac_issued_counters"] = round(fl / (pf["ms"] * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 4)
    if "decode" in out:
        dc = out["decode"]
        line["decode"] = {"workload": "decode_mimo_bf16: batch 256, H=64, P=64, N=64, R=4, fp32 state, 1024 steps "
                                      "(one HIP graph of 1024 launches, median of 3 replays)",
                          "steps_per_s": round(dc["steps_per_s"], 1), "ms_per_step": round(dc["ms_per_step"], 5),
                          "achieved_GBps": round(dc["gbps"], 1), "peak_GBps": HBM_PEAK_GBPS,
                          "frac": round(dc["gbps"] / HBM_PEAK_GBPS, 4), "bytes_per_step": dc["bytes_per_step"]}
        tr = measured_traffic("decode")
        line["decode"]["traffic"] = None if tr is None else round(tr)
        if tr is not None:  # DRAM-side rate from the counters (MALL hits excluded)
            line["decode"]["traffic_GBps"] = round(tr / (dc["ms_per_step"] * 1e-3) / 1e9, 1)
    if "verify" in out:
        vf = out["verify"]
        line["verify"] = {"workload": f"verify_mimo_bf16: decode shapes (batch 256, H=64, P=64, N=64, R=4), "
                                      f"k={vf['k']} tokens per chunked_fwd call on the fp32 state in place "
                                      f"(the library's short path: one chunk on bf16 MFMAs)",
                          "ms_per_call": round(vf["ms_per_call"], 5), "tokens_per_s": round(vf["tokens_per_s"], 1),
                          "achieved_GBps": round(vf["gbps"], 1), "frac": round(vf["gbps"] / HBM_PEAK_GBPS, 4),
                          "bytes_per_call": vf["bytes_per_call"],
                          "token_path_ms_per_call": round(vf["token_path_ms"], 5),
                          "chunk_walk_ms_per_call": round(vf["chunk_walk_ms"], 5)}
    def backward_entry(bw, workload):
        return {"workload": workload, "ms": round(bw["ms"], 4), "tokens_per_s": round(bw["tokens_per_s"], 1),
                "bound": "hbm" if bw["hbm_floor_ms"] >= bw["mfma_floor_ms"] else "mfma",
                "achieved_GBps": round(bw["gbps"], 1), "peak_GBps": HBM_PEAK_GBPS,
                "frac": round(max(bw["hbm_floor_ms"], bw["mfma_floor_ms"]) / bw["ms"], 4),
                "bytes_per_call": round(bw["bytes"]), "achieved_TFLOPs": round(bw["tflops"], 1),
                "flops_per_call": bw["flops"], "hbm_floor_ms": round(bw["hbm_floor_ms"], 4),
                "mfma_floor_ms": round(bw["mfma_floor_ms"], 4)}

    if "backward" in out:
        line["backward"] = backward_entry(out["backward"],
                                          f"{w.name} backward (mamba3_ssm_chunked_bwd, dy ~ N(0,1); bf16 MFMA "
                                          f"operands with fp32 accumulation, the checkpoint walk's in hi + lo parts)")
    if "backward_long" in out:
        line["backward_long_mimo_bf16"] = backward_entry(
            out["backward_long"], "long_mimo_bf16 backward: batch 1, L=65536, H=32, P=64, N=128, R=4, 8-token "
                                  "chunks, each sequence walked as segments (library default)")
    if "prologue" in out:
        pr = out["prologue"]
        sh = pr["shape"]
        line["bc_prologue"] = {
            "workload": f"mamba3_bc_prologue: batch {sh['batch']}, L={sh['seqlen']}, d_model={sh['d_model']} -> "
                        f"B, C of H={sh['nheads']}, R={sh['rank']}, N={sh['dstate']} (projection, RMS norm, "
                        f"bias, rotation; bf16 MFMA, fp32 accumulation)",
            "ms": round(pr["ms"], 4), "tokens_per_s": round(pr["tokens_per_s"], 1), "bound": "mfma",
            "achieved_TFLOPs": round(pr["tflops"], 1), "peak_TFLOPs": BF16_DENSE_TFLOPS,
            "frac": round(pr["tflops"] / BF16_DENSE_TFLOPS, 4), "flops_per_call": pr["flops"],
            "bytes_per_call": pr["bytes"], "achieved_GBps": round(pr["gbps"], 1)}
        clk = prologue_clock_ghz()
        # the same peak at the clock the kernel was measured to run at (GRBM_COUNT
        # over its dispatches, committed summary); frac above is against 2.4 GHz
        line["bc_prologue"]["clock_GHz_counters"] = clk
        line["bc_prologue"]["frac_at_measured_clock"] = (
            round(pr["tflops"] / (BF16_DENSE_TFLOPS * clk / ENGINE_CLOCK_GHZ), 4) if clk else None)
    if "rope" in out:
        line["rope_bc"] = {"ms": round(out["rope"]["ms"], 4), "achieved_GBps": round(out["rope"]["gbps"], 1),
                           "frac": round(out["rope"]["gbps"] / HBM_PEAK_GBPS, 4)}
    for name in ("siso_bf16", "long_mimo_bf16"):
        if name in out:
            o = out[name]
            tr = measured_traffic(name)
            line[name] = {"tokens_per_s": round(o["tokens_per_s"], 1), "ms": round(o["ms"], 4),
                          "achieved_GBps": round(o["gbps"], 1), "frac_hbm": round(o["gbps"] / HBM_PEAK_GBPS, 4),
                          "kernel": walker_kernel(W[name]), "traffic": None if tr is None else round(tr)}
    if "chunk16" in out:
        o = out["chunk16"]
        line["mimo_bf16_chunk16"] = {"workload": "mimo_bf16 prefill requested with chunk 16 (= N/R, the pages' "
                                                 "suggestion; walked as 32-token chunks)",
                                     "ms": round(o["ms"], 4), "tokens_per_s": round(o["tokens_per_s"], 1),
                                     "frac_hbm": round(o["gbps"] / HBM_PEAK_GBPS, 4)}
    if not args.no_cpu and "prefill" in out:
        print(f"[bench] cpu baseline (oracle) on {w.name}", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inputs, w)
        if args.only == "all":
            for name in ("siso_bf16", "long_mimo_bf16"):
                print(f"[bench] cpu baseline (oracle) on {name}", file=sys.stderr, flush=True)
                line[name]["cpu_baseline"] = cpu_baseline(inputs, W[name], budget_s=5.0)
            print("[bench] cpu baseline (oracle) on decode_mimo_bf16", file=sys.stderr, flush=True)
            line["decode"]["cpu_baseline"] = cpu_baseline(inputs, W["decode_mimo_bf16"], budget_s=5.0, decode=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
