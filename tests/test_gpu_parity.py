"""Parity of the HIP path with the fp64 CPU oracle (needs an MI355X).

Every case feeds the same seeded inputs to both sides and compares element by
element.  Error metric: for each (b, h) slice, max|gpu - ref| / max|ref|,
maximised over slices.  Bounds: 1e-4 for fp32 io, 2e-2 for bf16 io (fp32
accumulation), 1e-3 between chunked and token-by-token final states.
"""
import math
import zlib

import numpy as np
import pytest

import oracle
from state_space_sequence_03_amd.inputs import numpy_inputs, torch_inputs, WORKLOADS, seed_of
from state_space_sequence_03_amd.ops import M3_TOKEN_PATH_MAX_L

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_03_amd import ops as o
    o.lib()
    return o


def to_dev(inp, io):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        out[k] = t.to(dt) if k in ("x", "B", "C", "prev_B", "prev_x") else t.float()
    return out


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def slice_err(gpu, ref, bh_axes):
    """max over (b,h) slices of max|gpu-ref| / max|ref| within the slice."""
    g = np.moveaxis(gpu, bh_axes, (0, 1))
    r = np.moveaxis(ref, bh_axes, (0, 1))
    worst = 0.0
    for i in range(g.shape[0]):
        for j in range(g.shape[1]):
            den = np.max(np.abs(r[i, j]))
            if den == 0:
                den = 1.0
            worst = max(worst, float(np.max(np.abs(g[i, j] - r[i, j])) / den))
    return worst


def run_fwd(ops, d, chunk, **kw):
    y, hf = ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"],
                            h0=d.get("h0"), prev_B=d.get("prev_B"), prev_x=d.get("prev_x"), chunk=chunk, **kw)
    torch.cuda.synchronize()
    return y, hf


def oracle_fwd(inp):
    return oracle.forward(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["lam"], inp["theta"],
                          h0=inp.get("h0"), prev_B=inp.get("prev_B"), prev_x=inp.get("prev_x"))


def check_fwd(ops, inp, io, chunk, tol=None, **kw):
    tol = TOL[io] if tol is None else tol
    d = to_dev(inp, io)
    y, hf = run_fwd(ops, d, chunk, **kw)
    yo, ho = oracle_fwd(inp)
    ey = slice_err(host(y), yo, (0, 2))
    eh = slice_err(host(hf), ho, (0, 1))
    say(f"   y err {ey:.3e}  h_final err {eh:.3e}  (tol {tol}, final state {min(tol, 1e-3)})")
    assert ey < tol and eh < min(tol, 1e-3)
    return y, hf


# ---------------------------------------------------------------- chunked forward
FWD_CASES = [
    # io,    b, L,   H, P,  N,  R, Q,  h0,    prev
    ("f32", 1, 256, 2, 16, 16, 1, 32, False, False),   # the tiny SISO fp32 workload
    ("f32", 2, 77, 3, 32, 32, 2, 16, True, True),
    ("f32", 1, 130, 2, 16, 64, 1, 64, True, False),
    ("f32", 2, 50, 1, 64, 16, 4, 16, False, True),
    ("f32", 1, 97, 2, 64, 64, 2, 32, True, True),
    ("bf16", 2, 300, 3, 64, 64, 1, 64, True, True),
    ("bf16", 1, 200, 2, 64, 64, 4, 64, True, True),
    ("bf16", 1, 130, 2, 64, 128, 4, 64, True, True),
    ("bf16", 2, 95, 2, 32, 16, 2, 32, False, True),
    ("bf16", 1, 129, 2, 128, 32, 2, 64, True, False),
    ("bf16", 2, 70, 2, 64, 64, 4, 16, True, True),
    ("bf16", 1, 5, 2, 16, 16, 1, 16, True, True),
    ("bf16", 1, 64, 1, 128, 64, 4, 32, False, False),
    ("bf16", 1, 33, 2, 16, 128, 1, 16, True, True),
    # the 32-token walker (bf16, N = P = 64, Q 32 or 64): every rank, ragged
    # tails, a single-token tail, and sequences shorter than one sub-chunk
    ("bf16", 2, 161, 2, 64, 64, 2, 32, True, False),
    ("bf16", 1, 97, 3, 64, 64, 4, 32, False, True),
    ("bf16", 1, 31, 2, 64, 64, 2, 64, True, True),
    ("bf16", 1, 33, 1, 64, 64, 1, 32, False, False),
    ("bf16", 3, 64, 2, 64, 64, 4, 64, True, True),
    # R = 1: 64-token sub-chunks, two adjacent tokens per staging thread (a
    # tail ending inside a thread's pair, a single-token second sub-chunk,
    # requested chunks of 16 and 32 walked at 64)
    ("bf16", 1, 127, 2, 64, 64, 1, 64, True, True),
    ("bf16", 2, 65, 1, 64, 64, 1, 16, False, True),
    ("bf16", 1, 200, 3, 64, 64, 1, 32, True, False),
    # the sub-chunk walker at N = 128 (16-token sub-chunks)
    ("bf16", 2, 75, 2, 64, 128, 2, 16, True, True),
    ("bf16", 1, 40, 3, 64, 128, 4, 32, False, True),
    ("bf16", 1, 15, 1, 64, 128, 4, 64, True, False),
    # tiles that do not fit the LDS at the requested chunk: the general walker
    # walks the chunk as shorter pieces (fp32 at the 1.5B MIMO head shape,
    # bf16 with N = P = 128 at R = 4, fp32 N = P = 128 walked as 8 tokens)
    ("f32", 1, 150, 2, 64, 64, 4, 64, True, True),
    ("bf16", 1, 150, 2, 128, 128, 4, 64, True, True),
    ("f32", 1, 70, 1, 128, 128, 4, 16, True, True),
    ("f32", 2, 90, 1, 64, 128, 2, 64, False, True),
    ("f32", 1, 67, 2, 128, 128, 1, 64, True, False),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_chunked_matches_oracle(ops, case):
    io, b, L, H, P, N, R, Q, h0, prev = case
    say(f"chunked_fwd {case}")
    inp = numpy_inputs(b, L, H, P, N, R, io=io, seed=zlib.crc32(repr(case).encode()) % 10000, with_h0=h0, with_prev=prev)
    check_fwd(ops, inp, io, Q)
    if L <= M3_TOKEN_PATH_MAX_L:  # short: both paths
        say("   forced chunk walk, forced token path")
        check_fwd(ops, inp, io, Q, chunk_walk=True)
        check_fwd(ops, inp, io, Q, token_path=True)


# short sequences (at most M3_TOKEN_PATH_MAX_L tokens) run token by token with
# the state on chip; each case also runs through the chunk walk
TOKEN_CASES = [
    # io,    b, L,  H, P,   N,   R, h0,    prev
    ("f32", 3, 1, 5, 16, 16, 1, True, True),
    ("f32", 2, 7, 3, 64, 64, 4, True, False),
    ("f32", 1, 16, 2, 128, 128, 2, False, True),
    ("f32", 2, 4, 2, 32, 16, 1, False, False),
    ("bf16", 4, 8, 8, 64, 64, 4, True, True),     # decode shapes, 8 tokens per call
    ("bf16", 2, 3, 4, 32, 128, 1, False, False),
    ("bf16", 1, 16, 3, 128, 32, 2, True, True),
    ("bf16", 2, 2, 2, 16, 64, 4, True, True),
    ("bf16", 1, 11, 2, 64, 128, 4, True, True),   # long-context head shape
    # the one-chunk MFMA path (bf16, P = 64, N = 64 or 128): every rank, 1 to 16 tokens
    ("bf16", 2, 1, 3, 64, 64, 1, True, True),
    ("bf16", 1, 16, 2, 64, 64, 2, True, False),
    ("bf16", 3, 5, 2, 64, 128, 2, False, True),
    ("bf16", 1, 16, 1, 64, 128, 4, True, True),
    ("bf16", 2, 13, 2, 64, 64, 4, False, False),
    ("bf16", 1, 7, 2, 64, 128, 1, True, True),
]


@pytest.mark.parametrize("case", TOKEN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_short_sequence_token_path(ops, case):
    io, b, L, H, P, N, R, h0, prev = case
    say(f"token path {case}")
    inp = numpy_inputs(b, L, H, P, N, R, io=io, seed=zlib.crc32(repr(case).encode()) % 10000, with_h0=h0, with_prev=prev)
    y_t, h_t = check_fwd(ops, inp, io, 16, token_path=True)
    y_w, h_w = check_fwd(ops, inp, io, 16, chunk_walk=True)
    check_fwd(ops, inp, io, 16)  # the library's own choice
    assert slice_err(host(h_t), host(h_w), (0, 1)) < 1e-3


def test_verify_step_in_place(ops):
    """k tokens per call on a decode state: h_final aliases h0 (updated in
    place) and equals k one-token steps; y matches the oracle."""
    b, L, H, P, N, R = 4, 8, 8, 64, 64, 4
    inp = numpy_inputs(b, L, H, P, N, R, io="bf16", seed=21, with_h0=True, with_prev=True)
    d = to_dev(inp, "bf16")
    say("verify step in place")
    state = d["h0"].clone()
    y, hf = ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=state,
                            prev_B=d["prev_B"], prev_x=d["prev_x"], chunk=16, h_final=state, token_path=True)
    torch.cuda.synchronize()
    assert hf.data_ptr() == state.data_ptr()
    yo, ho = oracle_fwd(inp)
    assert slice_err(host(y), yo, (0, 2)) < TOL["bf16"]
    assert slice_err(host(state), ho, (0, 1)) < TOL["bf16"]
    st = d["h0"].clone()
    pb, px = d["prev_B"], d["prev_x"]
    for t in range(L):
        ops.decode_step(st, d["x"][:, t].contiguous(), d["B"][:, t].contiguous(), d["C"][:, t].contiguous(),
                        d["dt"][:, t].contiguous(), d["A"][:, t].contiguous(), d["lam"][:, t].contiguous(),
                        d["theta"][:, t].contiguous(), pb, px)
        pb, px = d["B"][:, t].contiguous(), d["x"][:, t].contiguous()
    torch.cuda.synchronize()
    assert slice_err(host(st), host(state), (0, 1)) < 1e-5


@pytest.mark.parametrize("N", [64, 128])
def test_verify_one_chunk_in_place(ops, N):
    """k = 8 tokens on a decode state by the library's default short path (one
    chunk on MFMAs), h_final aliasing h0: y against the oracle, the state
    against the oracle and against 8 one-token steps (the chunked-vs-sequential
    bound)."""
    b, L, H, P, R = 4, 8, 8, 64, 4
    inp = numpy_inputs(b, L, H, P, N, R, io="bf16", seed=22 + N, with_h0=True, with_prev=True)
    d = to_dev(inp, "bf16")
    say(f"verify one chunk in place N{N}")
    state = d["h0"].clone()
    y, hf = ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=state,
                            prev_B=d["prev_B"], prev_x=d["prev_x"], chunk=16, h_final=state)
    torch.cuda.synchronize()
    assert hf.data_ptr() == state.data_ptr()
    yo, ho = oracle_fwd(inp)
    ey, eh = slice_err(host(y), yo, (0, 2)), slice_err(host(state), ho, (0, 1))
    say(f"   y err {ey:.3e} state err {eh:.3e}")
    assert ey < TOL["bf16"] and eh < 1e-3
    st = d["h0"].clone()
    pb, px = d["prev_B"], d["prev_x"]
    for t in range(L):
        ops.decode_step(st, d["x"][:, t].contiguous(), d["B"][:, t].contiguous(), d["C"][:, t].contiguous(),
                        d["dt"][:, t].contiguous(), d["A"][:, t].contiguous(), d["lam"][:, t].contiguous(),
                        d["theta"][:, t].contiguous(), pb, px)
        pb, px = d["B"][:, t].contiguous(), d["x"][:, t].contiguous()
    torch.cuda.synchronize()
    assert slice_err(host(st), host(state), (0, 1)) < 1e-3


@pytest.mark.parametrize("io,N,P,R,Q", [("f32", 16, 32, 2, 32), ("bf16", 64, 64, 4, 64), ("bf16", 128, 64, 4, 64)])
def test_slow_decay_stress(ops, io, N, P, R, Q):
    """A in [-1e-2, 0] (A = 0 included): memory reaches across many chunks, so
    the inter-chunk pass carries most of y.  h0 != 0, prev given, ragged L."""
    say(f"slow decay {io} N{N} P{P} R{R} Q{Q}")
    inp = numpy_inputs(2, 1000, 2, P, N, R, io=io, seed=77, with_h0=True, with_prev=True,
                       a_range=(-30.0, math.log(1e-2)))
    inp["A"][0, 500:, 0] = 0.0
    # keep the state bounded: small steps
    inp["dt"] *= 0.2
    check_fwd(ops, inp, io, Q)


def test_parity_sequence_on_gpu(ops):
    """The hand-set parity example (tests/golden/parity_bits.txt) through the
    chunked kernel: x = 0, so every output comes from the state carried across
    chunks and rotated by pi for each 1."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "parity_bits.txt")
    lines = [ln.strip() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    bits = [int(c) for c in lines[0]]
    expect = np.array([float(v) for v in lines[1].split()])
    L, N, P = len(bits), 16, 16
    z = lambda *s: np.zeros(s, np.float32)
    inp = dict(x=z(1, L, 1, 1, P), B=z(1, L, 1, 1, N), C=z(1, L, 1, 1, N),
               dt=np.ones((1, L, 1), np.float32), A=z(1, L, 1), lam=np.full((1, L, 1), 0.5, np.float32),
               theta=z(1, L, 1, N // 2), h0=z(1, 1, N, P))
    inp["theta"][0, :, 0, 0] = np.pi * np.asarray(bits, np.float32)
    inp["C"][..., 0] = 1.0
    inp["h0"][0, 0, 0, 0] = 1.0
    say("parity sequence fp32 chunk 16")
    y, hf = run_fwd(ops, to_dev(inp, "f32"), 16)
    got = host(y)[0, :, 0, 0, 0]
    assert np.max(np.abs(got - expect)) < 1e-4


def test_chunk_size_invariance(ops):
    inp = numpy_inputs(1, 333, 2, 64, 64, 2, io="bf16", seed=5, with_h0=True, with_prev=True)
    d = to_dev(inp, "bf16")
    outs = []
    for Q in (16, 32, 64):
        say(f"chunk invariance Q={Q}")
        outs.append(run_fwd(ops, d, Q))
    yo, ho = oracle_fwd(inp)
    for y, hf in outs:
        assert slice_err(host(y), yo, (0, 2)) < TOL["bf16"]
        assert slice_err(host(hf), ho, (0, 1)) < 1e-3
    assert slice_err(host(outs[0][1]), host(outs[2][1]), (0, 1)) < 1e-3


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunked_vs_decode_iterated(ops, io):
    """Final state of the chunked form vs the one-token kernel iterated L times."""
    b, L, H, P, N, R = 2, 150, 2, 32, 32, 2
    inp = numpy_inputs(b, L, H, P, N, R, io=io, seed=11, with_h0=True, with_prev=True)
    d = to_dev(inp, io)
    say(f"chunked vs decode {io}")
    y, hf = run_fwd(ops, d, 32)
    st = d["h0"].clone()
    pb, px = d["prev_B"], d["prev_x"]
    ys = []
    for t in range(L):
        yt = ops.decode_step(st, d["x"][:, t].contiguous(), d["B"][:, t].contiguous(), d["C"][:, t].contiguous(),
                             d["dt"][:, t].contiguous(), d["A"][:, t].contiguous(), d["lam"][:, t].contiguous(),
                             d["theta"][:, t].contiguous(), pb, px)
        ys.append(yt)
        pb, px = d["B"][:, t].contiguous(), d["x"][:, t].contiguous()
    torch.cuda.synchronize()
    assert slice_err(host(st), host(hf), (0, 1)) < 1e-3
    yd = torch.stack(ys, 1)
    assert slice_err(host(yd), host(y), (0, 2)) < TOL[io]


def test_continuation_two_calls(ops):
    """Two chunked calls with (h_final, last raw B and x) carried == one call."""
    inp = numpy_inputs(2, 260, 2, 64, 64, 4, io="bf16", seed=12, with_h0=True, with_prev=True)
    d = to_dev(inp, "bf16")
    say("continuation")
    y_all, h_all = run_fwd(ops, d, 64)
    L1 = 100  # not a chunk multiple
    part = lambda s: {k: (v[:, s].contiguous() if k in ("x", "B", "C", "dt", "A", "lam", "theta") else v)
                      for k, v in d.items()}
    y1, h1 = run_fwd(ops, part(slice(0, L1)), 64)
    d2 = part(slice(L1, 260))
    d2["h0"] = h1
    d2["prev_B"] = d["B"][:, L1 - 1].contiguous()
    d2["prev_x"] = d["x"][:, L1 - 1].contiguous()
    y2, h2 = run_fwd(ops, d2, 64)
    assert slice_err(host(torch.cat([y1, y2], 1)), host(y_all), (0, 2)) < 1e-2
    assert slice_err(host(h2), host(h_all), (0, 1)) < 1e-3


def test_empty_and_single_token(ops):
    inp = numpy_inputs(1, 1, 2, 16, 16, 1, io="f32", seed=3, with_h0=True, with_prev=True)
    say("single token")
    check_fwd(ops, inp, "f32", 16)
    say("empty sequence")
    d = to_dev(numpy_inputs(1, 0, 2, 16, 16, 1, io="f32", seed=3, with_h0=True), "f32")
    y, hf = run_fwd(ops, d, 16)
    assert torch.equal(hf, d["h0"])
    # the same call with an aliased h_final is a no-op
    y, hf2 = ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"],
                             chunk=16, h_final=d["h0"])
    torch.cuda.synchronize()


def test_canary_and_determinism(ops):
    inp = numpy_inputs(2, 190, 3, 64, 64, 4, io="bf16", seed=21, with_h0=True, with_prev=True)
    d = to_dev(inp, "bf16")
    n = d["x"].numel()
    pad = 4096
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = buf[pad:pad + n].view(d["x"].shape)
    hbuf = torch.full((d["h0"].numel() + 2 * pad,), float("nan"), device="cuda")
    hf = hbuf[pad:pad + d["h0"].numel()].view(d["h0"].shape)
    say("canary")
    ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"],
                    prev_B=d["prev_B"], prev_x=d["prev_x"], chunk=64, y=y, h_final=hf)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[pad + n:].float()).all()
    assert torch.isnan(hbuf[:pad]).all() and torch.isnan(hbuf[pad + d["h0"].numel():]).all()
    assert not torch.isnan(y.float()).any() and not torch.isnan(hf).any()
    ref = (y.clone(), hf.clone())
    for _ in range(2):
        y2, h2 = run_fwd(ops, d, 64)
        assert torch.equal(y2, ref[0]) and torch.equal(h2, ref[1])


# ---------------------------------------------------------------- decode step
DEC_CASES = [("f32", 3, 2, 16, 16, 1), ("f32", 2, 3, 64, 64, 4), ("f32", 1, 2, 32, 128, 2),
             ("bf16", 4, 2, 64, 64, 4), ("bf16", 2, 2, 128, 64, 1), ("bf16", 2, 1, 16, 128, 4)]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_matches_oracle(ops, case):
    io, b, H, P, N, R = case
    say(f"decode {case}")
    steps = 12
    inp = numpy_inputs(b, steps, H, P, N, R, io=io, seed=31, with_h0=True, with_prev=True)
    d = to_dev(inp, io)
    st = d["h0"].clone()
    pb, px = d["prev_B"], d["prev_x"]
    ys = []
    for t in range(steps):
        cut = lambda k: d[k][:, t].contiguous()
        ys.append(ops.decode_step(st, cut("x"), cut("B"), cut("C"), cut("dt"), cut("A"), cut("lam"), cut("theta"),
                                  pb, px))
        pb, px = cut("B"), cut("x")
    torch.cuda.synchronize()
    yo, ho = oracle_fwd(inp)
    ey = slice_err(host(torch.stack(ys, 1)), yo, (0, 2))
    eh = slice_err(host(st), ho, (0, 1))
    say(f"   y err {ey:.3e} state err {eh:.3e}")
    assert ey < TOL[io] and eh < TOL[io]


def test_decode_first_token_without_prev(ops):
    inp = numpy_inputs(2, 1, 2, 64, 64, 4, io="bf16", seed=32, with_h0=True)
    d = to_dev(inp, "bf16")
    st = d["h0"].clone()
    say("decode without prev")
    y = ops.decode_step(st, d["x"][:, 0].contiguous(), d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(),
                        d["dt"][:, 0].contiguous(), d["A"][:, 0].contiguous(), d["lam"][:, 0].contiguous(),
                        d["theta"][:, 0].contiguous())
    torch.cuda.synchronize()
    yo, ho = oracle_fwd(inp)
    assert slice_err(host(y)[:, None], yo, (0, 2)) < 2e-2 and slice_err(host(st), ho, (0, 1)) < 1e-4


# ---------------------------------------------------------------- rope
@pytest.mark.parametrize("io,L,N,R,ang", [("f32", 1, 16, 1, False), ("f32", 63, 64, 2, True), ("bf16", 64, 128, 4, True),
                                          ("bf16", 65, 32, 1, False), ("bf16", 300, 64, 4, True), ("f32", 1000, 16, 4, True)])
def test_rope_matches_oracle(ops, io, L, N, R, ang):
    say(f"rope {io} L{L} N{N} R{R}")
    inp = numpy_inputs(2, L, 3, 16, N, R, io=io, seed=41)
    a0 = np.random.default_rng(4).uniform(-3, 3, (2, 3, N // 2)).astype(np.float32) if ang else None
    d = to_dev(inp, io)
    Br, Cr, af = ops.rope_bc(d["B"], d["C"], d["dt"], d["theta"],
                             torch.from_numpy(a0).cuda() if ang else None)
    torch.cuda.synchronize()
    Bo, Co, ao = oracle.rope_bc(inp["B"], inp["C"], inp["dt"], inp["theta"], a0)
    tol = TOL[io] if io == "bf16" else 2e-4
    assert slice_err(host(Br), Bo, (0, 2)) < tol and slice_err(host(Cr), Co, (0, 2)) < tol
    assert np.max(np.abs(host(af) - ao)) < 1e-4 * max(1.0, np.max(np.abs(ao)))


# ---------------------------------------------------------------- full-size workloads, sampled slices
def sampled_pairs(batch, nheads, n, seed):
    """n distinct (b, h) pairs: the first and the last pair of the grid (the
    highest block indices) and n - 2 more drawn with a fixed seed."""
    rng = np.random.default_rng(seed)
    pairs = [(0, 0), (batch - 1, nheads - 1)]
    while len(pairs) < min(n, batch * nheads):
        p = (int(rng.integers(batch)), int(rng.integers(nheads)))
        if p not in pairs:
            pairs.append(p)
    return pairs


def sample_slices(d, pairs, keys_bl=("x", "B", "C", "dt", "A", "lam", "theta")):
    """Host fp64 copies of the (b,h) slices named in pairs, stacked along the
    batch axis with one head each (so the oracle runs them on parallel threads)."""
    s = {}
    for k in keys_bl:
        s[k] = np.concatenate([host(d[k][bi:bi + 1, :, hi:hi + 1]) for bi, hi in pairs], 0)
    if "h0" in d:
        s["h0"] = np.concatenate([host(d["h0"][bi:bi + 1, hi:hi + 1]) for bi, hi in pairs], 0)
    return s


@pytest.mark.parametrize("name", ["siso_bf16", "mimo_bf16", "long_mimo_bf16"])
def test_full_workload_sampled(ops, name):
    w = WORKLOADS[name]
    say(f"full workload {name}: generating")
    d = torch_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, io=w.io, seed=seed_of(name))
    say(f"full workload {name}: chunked_fwd")
    y, hf = run_fwd(ops, d, w.chunk)
    pairs = sampled_pairs(w.batch, w.nheads, 4 if name == "long_mimo_bf16" else 8, seed=0)
    say(f"full workload {name}: oracle on slices {pairs}")
    yo, ho = oracle_fwd(sample_slices(d, pairs))
    for i, (bi, hi) in enumerate(pairs):
        ey = slice_err(host(y[bi:bi + 1, :, hi:hi + 1]), yo[i:i + 1], (0, 2))
        eh = slice_err(host(hf[bi:bi + 1, hi:hi + 1]), ho[i:i + 1], (0, 1))
        say(f"   slice {(bi, hi)}: y {ey:.3e} h {eh:.3e}")
        assert ey < TOL["bf16"] and eh < 1e-3


def test_full_decode_workload_sampled(ops):
    """Batch 256, H=64, P=N=64, R=4, fp32 state ~N(0,1), 1024 consecutive steps."""
    w = WORKLOADS["decode_mimo_bf16"]
    steps = w.decode_steps
    say("full decode workload: generating")
    d = torch_inputs(w.batch, steps, w.nheads, w.headdim, w.dstate, w.rank, io="bf16", seed=seed_of(w.name),
                     with_h0=True)
    # per-step inputs laid out (steps, B, H, ...) so each step is contiguous
    step_major = {k: d[k].transpose(0, 1).contiguous() for k in ("x", "B", "C", "dt", "A", "lam", "theta")}
    st = d["h0"].clone()
    ys = torch.empty((steps,) + step_major["x"].shape[1:], dtype=torch.bfloat16, device="cuda")
    say("full decode workload: 1024 steps")
    for t in range(steps):
        pb = step_major["B"][t - 1] if t > 0 else None
        px = step_major["x"][t - 1] if t > 0 else None
        ops.decode_step(st, step_major["x"][t], step_major["B"][t], step_major["C"][t], step_major["dt"][t],
                        step_major["A"][t], step_major["lam"][t], step_major["theta"][t], pb, px, y=ys[t])
    torch.cuda.synchronize()
    pairs = sampled_pairs(w.batch, w.nheads, 8, seed=1)
    say(f"full decode workload: oracle on slices {pairs}")
    yo, ho = oracle_fwd(sample_slices(d, pairs))
    for i, (bi, hi) in enumerate(pairs):
        ey = slice_err(host(ys[:, bi:bi + 1, hi:hi + 1]).transpose(1, 0, 2, 3, 4), yo[i:i + 1], (0, 2))
        eh = slice_err(host(st[bi:bi + 1, hi:hi + 1]), ho[i:i + 1], (0, 1))
        say(f"   slice {(bi, hi)}: y {ey:.3e} state {eh:.3e}")
        assert ey < TOL["bf16"] and eh < 1e-3


# ---------------------------------------------------------------- sequence segments
# segments=0: the library's own plan (B*H = 2 here, so it cuts the sequence)
@pytest.mark.parametrize("segs,slow,N,P,R", [(2, False, 64, 64, 4), (3, True, 64, 64, 4), (5, True, 128, 64, 4),
                                             (16, False, 128, 64, 4), (4, True, 32, 16, 4),
                                             # the general walker and the generic fix-up (N or P = 128)
                                             (3, True, 64, 128, 2), (0, True, 64, 128, 2),
                                             (4, True, 128, 64, 1), (0, True, 128, 64, 1),
                                             (3, True, 128, 128, 4), (0, False, 128, 128, 4),
                                             (3, True, 64, 64, 1), (0, False, 64, 64, 1)])
def test_segments_match_single_walk_and_oracle(ops, segs, slow, N, P, R):
    """Segments walked from zero + segment scan + fix-up == one sequential walk.
    With slow decay (A near 0) every chunk of every segment needs the fix-up."""
    say(f"segments S={segs} slow={slow} N{N} P{P} R{R}")
    kw = dict(a_range=(-30.0, math.log(1e-2))) if slow else {}
    inp = numpy_inputs(1, 1000, 2, P, N, R, io="bf16", seed=90 + segs + 7 * R, with_h0=True, with_prev=True, **kw)
    if slow:
        inp["dt"] *= 0.2
    d = to_dev(inp, "bf16")
    if segs == 0:
        dims = ops.make_dims(1, 1000, 2, P, N, R, 64, ops.M3_BF16)
        assert ops.chunked_fwd_workspace_size(dims) > 0  # the default plan walks segments
    y1, h1 = run_fwd(ops, d, 64, segments=1)
    ys, hs = run_fwd(ops, d, 64, segments=segs)
    yo, ho = oracle_fwd(inp)
    e_y = slice_err(host(ys), yo, (0, 2))
    e_h = slice_err(host(hs), ho, (0, 1))
    say(f"   vs oracle: y {e_y:.3e} h {e_h:.3e}; vs single walk: y {slice_err(host(ys), host(y1), (0, 2)):.3e}")
    assert e_y < TOL["bf16"] and e_h < 1e-3
    assert slice_err(host(hs), host(h1), (0, 1)) < 1e-3


def test_segments_workspace_and_fp32_rejected(ops):
    w = WORKLOADS["long_mimo_bf16"]
    dims = ops.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, w.chunk, ops.M3_BF16)
    assert ops.chunked_fwd_workspace_size(dims) > 0
    w2 = WORKLOADS["mimo_bf16"]
    dims2 = ops.make_dims(w2.batch, w2.seqlen, w2.nheads, w2.headdim, w2.dstate, w2.rank, w2.chunk, ops.M3_BF16)
    assert ops.chunked_fwd_workspace_size(dims2) == 0
    inp = to_dev(numpy_inputs(1, 200, 2, 16, 16, 1, io="f32", seed=3), "f32")
    with pytest.raises(ops.Mamba3Error):
        run_fwd(ops, inp, 32, segments=2)


def test_decode_graph_replays_match_eager(ops):
    """Decode steps captured in a HIP graph: every replay (with eager work and
    synchronisation between replays) equals the eager result bit for bit."""
    b, H, P, N, R, steps = 4, 3, 64, 64, 4, 8
    inp = numpy_inputs(b, steps, H, P, N, R, io="bf16", seed=55, with_h0=True, with_prev=True)
    d = to_dev(inp, "bf16")
    sm = {k: d[k].transpose(0, 1).contiguous() for k in ("x", "B", "C", "dt", "A", "lam", "theta")}
    st = torch.empty_like(d["h0"])
    y = torch.empty(sm["x"].shape[1:], dtype=torch.bfloat16, device="cuda")

    def run_all():
        for t in range(steps):
            pb = sm["B"][t - 1] if t > 0 else d["prev_B"]
            px = sm["x"][t - 1] if t > 0 else d["prev_x"]
            ops.decode_step(st, sm["x"][t], sm["B"][t], sm["C"][t], sm["dt"][t], sm["A"][t], sm["lam"][t],
                            sm["theta"][t], pb, px, y=y)

    say("decode graph: eager")
    st.copy_(d["h0"])
    run_all()
    torch.cuda.synchronize()
    ref_state, ref_y = st.clone(), y.clone()
    g = torch.cuda.CUDAGraph()
    st.copy_(d["h0"])
    with torch.cuda.graph(g):
        run_all()
    for rep in range(3):
        say(f"decode graph: replay {rep}")
        st.copy_(d["h0"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st, ref_state) and torch.equal(y, ref_y)
        _ = (st * 2).sum().item()  # eager work between replays
