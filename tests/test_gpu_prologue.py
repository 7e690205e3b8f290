"""Parity of the HIP B/C prologue (mamba3_bc_prologue) with the fp64 oracle
(oracle/prologue.py, pinned in tests/test_oracle_prologue_pins.py).  Needs an
MI355X.

Metric as for the core: per (b, h) slice, max|gpu - ref| / max|ref|,
maximised over slices, bound 2e-2 (the outputs are bf16); angle_final within
1e-4 of the largest angle.
"""
import zlib

import numpy as np
import pytest

import oracle
from state_space_sequence_03_amd.inputs import (PROLOGUE, PROLOGUE_SEED, numpy_inputs, prologue_numpy,
                                                 prologue_torch)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_03_amd import ops as o
    o.lib()
    return o


def slice_err(gpu, ref, bh_axes=(0, 2)):
    g = np.moveaxis(gpu, bh_axes, (0, 1))
    r = np.moveaxis(ref, bh_axes, (0, 1))
    worst = 0.0
    for i in range(g.shape[0]):
        for j in range(g.shape[1]):
            den = np.max(np.abs(r[i, j]))
            den = den if den > 0 else 1.0
            worst = max(worst, float(np.max(np.abs(g[i, j] - r[i, j])) / den))
    return worst


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if bf16 else t.float()


def run_gpu(ops, inp, H, R, N, eps):
    return ops.bc_prologue(dev(inp["u"], True), dev(inp["W"], True), dev(inp["dt"]), dev(inp["theta"]), H, R, N,
                           gain=dev(inp["gain"]) if "gain" in inp else None,
                           bias=dev(inp["bias"]) if "bias" in inp else None, eps=eps,
                           angle0=dev(inp["angle0"]) if "angle0" in inp else None)


# several token tiles (256 tokens) with a ragged last one, ragged feature
# tiles (256 features), every N, every R, optional gain / bias / angle0
CASES = [
    # b, L,   H, R, N,   D,   gain,  bias,  angle0, eps
    (1, 64, 1, 1, 16, 64, True, True, False, 1e-5),
    (2, 300, 3, 1, 32, 128, True, True, True, 1e-5),
    (1, 257, 2, 4, 16, 192, True, False, False, 1e-5),
    (1, 300, 5, 2, 128, 128, False, True, True, 1e-5),
    (2, 520, 4, 4, 64, 256, True, True, True, 1e-5),
    (1, 700, 2, 2, 64, 64, False, False, False, 0.1),
    (3, 1, 2, 4, 64, 64, True, True, True, 1e-5),
    # H a multiple of 256 / N: the angle pass takes several adjacent heads per block
    (1, 130, 16, 1, 16, 64, True, True, True, 1e-5),
    (2, 100, 8, 2, 32, 64, False, True, True, 1e-5),
    (1, 150, 2, 4, 128, 64, True, False, True, 1e-5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_prologue_matches_oracle(ops, case):
    b, L, H, R, N, D, g, bi, a0, eps = case
    say(f"bc_prologue {case}")
    inp = prologue_numpy(b, L, H, N, R, D, seed=zlib.crc32(repr(case).encode()) % 10000, with_gain=g, with_bias=bi, with_angle0=a0)
    Bg, Cg, ag = run_gpu(ops, inp, H, R, N, eps)
    torch.cuda.synchronize()
    Bo, Co, ao = oracle.bc_prologue(inp["u"], inp["W"], inp["dt"], inp["theta"], H, R, N, gain=inp.get("gain"),
                                    bias=inp.get("bias"), eps=eps, angle0=inp.get("angle0"))
    eb, ec = slice_err(host(Bg), Bo), slice_err(host(Cg), Co)
    ea = float(np.max(np.abs(host(ag) - ao)) / max(1.0, np.max(np.abs(ao))))
    say(f"   B {eb:.2e}  C {ec:.2e}  angle {ea:.2e}")
    assert eb < TOL and ec < TOL and ea < 1e-4


def test_prologue_feeds_the_core_in_its_frame(ops):
    """The core given the prologue's B_rot, C_rot and theta = 0 gives the y of
    the oracle core on the unrotated normalised B, C with theta."""
    b, L, H, R, N, D, P = 1, 200, 2, 4, 64, 128, 64
    pin = prologue_numpy(b, L, H, N, R, D, seed=77)
    core = numpy_inputs(b, L, H, P, N, R, io="bf16", seed=78)
    pin["dt"], pin["theta"] = core["dt"], core["theta"]
    say("bc_prologue -> chunked_fwd (theta = 0)")
    Bg, Cg, _ = run_gpu(ops, pin, H, R, N, 1e-5)
    zero = torch.zeros_like(dev(core["theta"]))
    y, _ = ops.chunked_fwd(dev(core["x"], True), Bg, Cg, dev(core["dt"]), dev(core["A"]), dev(core["lam"]), zero)
    torch.cuda.synchronize()
    Bn, Cn, _ = oracle.bc_prologue(pin["u"], pin["W"], pin["dt"], np.zeros_like(pin["theta"]), H, R, N,
                                   gain=pin["gain"], bias=pin["bias"], eps=1e-5)
    yo, _ = oracle.forward(core["x"], Bn, Cn, core["dt"], core["A"], core["lam"], core["theta"])
    e = slice_err(host(y), yo)
    say(f"   y {e:.2e}")
    assert e < TOL


def test_prologue_empty_sequence(ops):
    """L = 0: nothing is projected; angle_final is angle0 (zero without it)."""
    b, H, R, N, D = 2, 3, 2, 16, 64
    u = torch.zeros((b, 0, D), device="cuda", dtype=torch.bfloat16)
    W = torch.randn((2 * H * R * N, D), device="cuda").to(torch.bfloat16)
    dt = torch.zeros((b, 0, H), device="cuda")
    th = torch.zeros((b, 0, H, N // 2), device="cuda")
    a0 = torch.randn((b, H, N // 2), device="cuda")
    Bo, Co, af = ops.bc_prologue(u, W, dt, th, H, R, N, angle0=a0)
    torch.cuda.synchronize()
    assert Bo.numel() == 0 and Co.numel() == 0
    assert torch.equal(af, a0)
    _, _, af0 = ops.bc_prologue(u, W, dt, th, H, R, N)
    torch.cuda.synchronize()
    assert torch.count_nonzero(af0).item() == 0


def test_prologue_rejections(ops):
    d = ops.make_dims(1, 8, 1, 16, 16, 1, 16, ops.M3_BF16)
    u = torch.zeros((1, 8, 96), device="cuda", dtype=torch.bfloat16)
    W = torch.zeros((32, 96), device="cuda", dtype=torch.bfloat16)
    s = torch.zeros((1, 8, 1), device="cuda")
    th = torch.zeros((1, 8, 1, 8), device="cuda")
    with pytest.raises(ops.Mamba3Error) as e:
        ops.bc_prologue(u, W, s, th, 1, 1, 16)   # D = 96 is not a multiple of 64
    assert e.value.status == ops.M3_ERR_UNSUPPORTED
    with pytest.raises(ops.Mamba3Error) as e:
        ops.bc_prologue(u[..., :64].float().contiguous(), W[:, :64].float().contiguous(), s, th, 1, 1, 16)
    assert e.value.status == ops.M3_ERR_UNSUPPORTED   # fp32 io
    with pytest.raises(ops.Mamba3Error) as e:
        ops.bc_prologue(u[..., :64].contiguous(), W[:, :64].contiguous(), s, th, 1, 1, 16, eps=-1.0)
    assert e.value.status == ops.M3_ERR_UNSUPPORTED


# the 1.5B shapes, and the long-context head shape (N = 128) with the same
# reading of the model width (d_model = H P / 2)
FULL = {"1p5b": PROLOGUE,
        "long": dict(batch=1, seqlen=65536, nheads=32, dstate=128, rank=4, d_model=1024)}


@pytest.mark.parametrize("shape", sorted(FULL))
def test_prologue_full_size_sampled(ops, shape):
    """Full size; 24 sampled tokens, all heads, against the oracle (each token
    run as a one-token call whose angle0 is the oracle rope's angle after the
    tokens before it)."""
    c = FULL[shape]
    b, L, H, R, N, D = c["batch"], c["seqlen"], c["nheads"], c["rank"], c["dstate"], c["d_model"]
    say("bc_prologue full size: generating")
    d = prologue_torch(b, L, H, N, R, D, seed=PROLOGUE_SEED + (shape == "long"))
    say("bc_prologue full size: running")
    Bg, Cg, ag = ops.bc_prologue(d["u"], d["W"], d["dt"], d["theta"], H, R, N, gain=d["gain"], bias=d["bias"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = [(int(rng.integers(b)), int(rng.integers(L))) for _ in range(22)] + [(0, 0), (b - 1, L - 1)]
    W, gain, bias = host(d["W"]), host(d["gain"]), host(d["bias"])
    worst = 0.0
    say(f"bc_prologue full size: oracle on {len(toks)} tokens")
    for bi, t in toks:
        dt, th = host(d["dt"][bi:bi + 1]), host(d["theta"][bi:bi + 1])
        zeros = np.zeros((1, t, H, 1, N))
        a0 = oracle.rope_bc(zeros, zeros, dt[:, :t], th[:, :t])[2] if t > 0 else None
        Bo, Co, _ = oracle.bc_prologue(host(d["u"][bi:bi + 1, t:t + 1]), W, dt[:, t:t + 1], th[:, t:t + 1], H, R, N,
                                       gain=gain, bias=bias, eps=1e-5, angle0=a0)
        worst = max(worst, slice_err(host(Bg[bi:bi + 1, t:t + 1]), Bo), slice_err(host(Cg[bi:bi + 1, t:t + 1]), Co))
    say(f"   worst {worst:.2e}")
    assert worst < TOL
    zeros = np.zeros((1, L, H, 1, N))   # angle_final of the last batch row
    ao = oracle.rope_bc(zeros, zeros, host(d["dt"][b - 1:]), host(d["theta"][b - 1:]))[2]
    ea = float(np.max(np.abs(host(ag[b - 1:]) - ao)) / max(1.0, np.max(np.abs(ao))))
    say(f"   angle_final {ea:.2e}")
    assert ea < 1e-4
