"""mamba3_ssm_chunked_fwd_noalloc (the chunked forward whose workspace is the
library's fixed per-GPU array) against mamba3_ssm_chunked_fwd with a caller
workspace: the same kernels and plan, so the outputs must agree bit for bit,
and with the fp64 oracle to the bf16 bounds.  Two calls in a row, the second
with a smaller input, both walking segments (so the array is in use)."""
import numpy as np
import pytest

import oracle
from state_space_sequence_03_amd.inputs import numpy_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_03_amd import ops as o
    o.lib()
    return o


def dev(inp):
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        out[k] = t.to(torch.bfloat16) if k in ("x", "B", "C", "prev_B", "prev_x") else t.float()
    return out


def rel(a, b):
    a = a.float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(a - b)) / max(float(np.max(np.abs(b))), 1e-30))


def test_noalloc_matches_chunked_fwd_two_calls(ops):
    for L, H, seed in ((3000, 2, 61), (1000, 1, 62)):
        inp = numpy_inputs(1, L, H, 64, 64, 4, io="bf16", seed=seed, with_h0=True, with_prev=True)
        d = dev(inp)
        dims = ops.make_dims(1, L, H, 64, 64, 4, 64, ops.M3_BF16)
        need = ops.chunked_fwd_workspace_size(dims)
        assert 0 < need <= ops.M3_NOALLOC_SCRATCH_BYTES  # segments: the fixed array is used
        say(f"noalloc L={L} H={H}: workspace {need} bytes")
        y_ref, h_ref = ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"],
                                       prev_B=d["prev_B"], prev_x=d["prev_x"], chunk=64)
        y = torch.full_like(y_ref, float("nan"))
        hf = torch.full_like(h_ref, float("nan"))
        ops.chunked_fwd_noalloc(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"],
                                prev_B=d["prev_B"], prev_x=d["prev_x"], y=y, h_final=hf, chunk=64)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hf, h_ref)
        yo, ho = oracle.forward(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["lam"], inp["theta"],
                                h0=inp["h0"], prev_B=inp["prev_B"], prev_x=inp["prev_x"])
        ey, eh = rel(y, yo), rel(hf, ho)
        say(f"   vs oracle: y {ey:.2e} h_final {eh:.2e}")
        assert ey < 2e-2 and eh < 1e-3


def test_noalloc_without_workspace_and_too_large(ops):
    # many (b,h): one segment, no workspace; the array is not touched
    inp = numpy_inputs(2, 200, 3, 64, 64, 4, io="bf16", seed=63, with_h0=True)
    d = dev(inp)
    say("noalloc without segments")
    y_ref, h_ref = ops.chunked_fwd(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"],
                                   chunk=64, segments=1)
    y, hf = torch.empty_like(y_ref), torch.empty_like(h_ref)
    ops.chunked_fwd_noalloc(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], h0=d["h0"], y=y,
                            h_final=hf, chunk=64, segments=1)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(hf, h_ref)
    # a workspace beyond the array: refused on the host, nothing launched
    dims = ops.make_dims(1, 1 << 20, 200, 128, 128, 4, 64, ops.M3_BF16)
    assert ops.chunked_fwd_workspace_size(dims) > ops.M3_NOALLOC_SCRATCH_BYTES
    import ctypes
    fake = ctypes.c_void_p(0x7F0000000000)
    st = ops.lib().mamba3_ssm_chunked_fwd_noalloc(ctypes.byref(dims), *([fake] * 7), None, None, None, fake, None,
                                                  None)
    assert st == ops.M3_ERR_WORKSPACE
