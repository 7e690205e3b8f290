"""Guard-region and determinism checks of every entry point (needs an MI355X).

Each output is placed inside a larger buffer filled with NaN: after the call
the guard regions before and after it must still be NaN (no write outside the
output) and the output itself must hold no NaN (every element written).  Each
call is then repeated on the same inputs and must give the same bits: the
kernels take no decision that depends on the order in which waves or blocks
arrive (no floating-point atomics).
"""
import numpy as np
import pytest

from state_space_sequence_03_amd.inputs import numpy_inputs, prologue_numpy

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PAD = 4096


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_03_amd import ops as o
    o.lib()
    return o


def dev(inp, io):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    return {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda().to(dt) if k in ("x", "B", "C", "prev_B", "prev_x")
                else torch.from_numpy(np.ascontiguousarray(v)).cuda().float()) for k, v in inp.items()}


class Guarded:
    """A tensor of the given shape and dtype inside a NaN-filled buffer."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape))
        self.n = n
        self.buf = torch.full((n + 2 * PAD,), float("nan"), dtype=dtype, device="cuda")
        self.t = self.buf[PAD:PAD + n].view(shape)

    def check(self, name):
        head, tail = self.buf[:PAD].float(), self.buf[PAD + self.n:].float()
        assert torch.isnan(head).all() and torch.isnan(tail).all(), f"{name}: write outside the output"
        assert not torch.isnan(self.t.float()).any(), f"{name}: element not written"


def test_decode_step_guards_and_repeat(ops):
    b, H, P, N, R = 3, 4, 64, 64, 4
    inp = numpy_inputs(b, 2, H, P, N, R, io="bf16", seed=71, with_h0=True, with_prev=True)
    d = dev(inp, "bf16")
    cut = lambda k: d[k][:, 0].contiguous()
    results = []
    for rep in range(3):
        say(f"decode guards, call {rep}")
        st = Guarded(d["h0"].shape, torch.float32)
        st.t.copy_(d["h0"])
        y = Guarded((b, H, R, P), torch.bfloat16)
        ops.decode_step(st.t, cut("x"), cut("B"), cut("C"), cut("dt"), cut("A"), cut("lam"), cut("theta"),
                        d["prev_B"], d["prev_x"], y=y.t)
        torch.cuda.synchronize()
        st.check("state")
        y.check("y")
        results.append((st.t.clone(), y.t.clone()))
    for s2, y2 in results[1:]:
        assert torch.equal(s2, results[0][0]) and torch.equal(y2, results[0][1])


@pytest.mark.parametrize("io,N,R", [("bf16", 64, 4), ("f32", 128, 2)])
def test_rope_guards_and_repeat(ops, io, N, R):
    b, L, H = 2, 300, 3
    inp = numpy_inputs(b, L, H, 16, N, R, io=io, seed=72)
    d = dev(inp, io)
    a0 = torch.randn((b, H, N // 2), device="cuda")
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    ref = None
    for rep in range(3):
        say(f"rope guards {io} N{N} R{R}, call {rep}")
        Br, Cr = Guarded(d["B"].shape, tdt), Guarded(d["C"].shape, tdt)
        af = Guarded((b, H, N // 2), torch.float32)
        ops.rope_bc(d["B"], d["C"], d["dt"], d["theta"], a0, B_rot=Br.t, C_rot=Cr.t, angle_final=af.t)
        torch.cuda.synchronize()
        Br.check("B_rot")
        Cr.check("C_rot")
        af.check("angle_final")
        got = (Br.t.clone(), Cr.t.clone(), af.t.clone())
        if ref is None:
            ref = got
        assert all(torch.equal(g, r) for g, r in zip(got, ref))


@pytest.mark.parametrize("io,N,P,R,segs", [("bf16", 64, 64, 4, 1), ("bf16", 128, 64, 4, 3), ("f32", 32, 32, 2, 0),
                                           ("f32", 128, 128, 2, 0)])
def test_backward_guards_and_repeat(ops, io, N, P, R, segs):
    b, L, H = 1, 170, 2
    inp = numpy_inputs(b, L, H, P, N, R, io=io, seed=73, with_h0=True, with_prev=True)
    d = dev(inp, io)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    rng = np.random.default_rng(74)
    dy = torch.from_numpy(rng.standard_normal((b, L, H, R, P)).astype(np.float32)).cuda().to(tdt)
    dh = torch.from_numpy(rng.standard_normal((b, H, N, P)).astype(np.float32)).cuda()
    shapes = {"dx": (d["x"].shape, tdt), "dB": (d["B"].shape, tdt), "dC": (d["C"].shape, tdt),
              "ddt": (d["dt"].shape, torch.float32), "dA": (d["A"].shape, torch.float32),
              "dlam": (d["lam"].shape, torch.float32), "dtheta": (d["theta"].shape, torch.float32),
              "dh0": ((b, H, N, P), torch.float32), "dprev_B": (d["prev_B"].shape, tdt),
              "dprev_x": (d["prev_x"].shape, tdt)}
    ref = None
    for rep in range(3):
        say(f"backward guards {io} N{N} P{P} R{R} segments {segs}, call {rep}")
        g = {k: Guarded(*v) for k, v in shapes.items()}
        ops.chunked_bwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], dy, h0=d["h0"],
                        prev_B=d["prev_B"], prev_x=d["prev_x"], dh_final=dh, segments=segs,
                        out={k: v.t for k, v in g.items()})
        torch.cuda.synchronize()
        for k, v in g.items():
            v.check(k)
        got = {k: v.t.clone() for k, v in g.items()}
        if ref is None:
            ref = got
        for k in got:
            assert torch.equal(got[k], ref[k]), k


def test_forward_segments_repeat(ops):
    """The segmented forward (walk, segment scan, fix-up) repeats bit for bit."""
    inp = numpy_inputs(1, 1000, 2, 64, 128, 4, io="bf16", seed=75, with_h0=True, with_prev=True)
    d = dev(inp, "bf16")
    ref = None
    for rep in range(3):
        say(f"forward segments repeat, call {rep}")
        y = Guarded(d["x"].shape, torch.bfloat16)
        hf = Guarded(d["h0"].shape, torch.float32)
        ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"],
                        prev_B=d["prev_B"], prev_x=d["prev_x"], chunk=64, segments=5, y=y.t, h_final=hf.t)
        torch.cuda.synchronize()
        y.check("y")
        hf.check("h_final")
        got = (y.t.clone(), hf.t.clone())
        if ref is None:
            ref = got
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_prologue_guards_and_repeat(ops):
    b, L, H, N, R, D = 1, 300, 2, 64, 4, 128
    pi = prologue_numpy(b, L, H, N, R, D, seed=76)
    t = {k: torch.from_numpy(v).cuda() for k, v in pi.items()}
    u, W = t["u"].to(torch.bfloat16), t["W"].to(torch.bfloat16)
    ref = None
    for rep in range(3):
        say(f"prologue guards, call {rep}")
        Bo, Co = Guarded((b, L, H, R, N), torch.bfloat16), Guarded((b, L, H, R, N), torch.bfloat16)
        af = Guarded((b, H, N // 2), torch.float32)
        ops.bc_prologue(u, W, t["dt"], t["theta"], H, R, N, gain=t["gain"], bias=t["bias"], B_rot=Bo.t, C_rot=Co.t,
                        angle_final=af.t)
        torch.cuda.synchronize()
        Bo.check("B_rot")
        Co.check("C_rot")
        af.check("angle_final")
        got = (Bo.t.clone(), Co.t.clone(), af.t.clone())
        if ref is None:
            ref = got
        assert all(torch.equal(g, r) for g, r in zip(got, ref))
