"""ctypes binding of the C ABI in ``include/mamba3_ssm.h``.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of ``libmamba3_ssm.so``.  PyTorch supplies device memory (tensors are
passed by ``data_ptr()``) and the stream (``torch.cuda.current_stream()``).
If the library is missing this module raises; there is no fallback.

Entry points keep the ABI's names:
  mamba3_ssm_chunked_fwd, mamba3_ssm_chunked_bwd, mamba3_ssm_decode_step,
  mamba3_rope_bc, mamba3_bc_prologue
(and the friendlier aliases chunked_fwd, chunked_bwd, decode_step, rope_bc,
bc_prologue), plus the workspace size queries.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# M3_LIBRARY names another build of the same library (e.g. one whose host
# code is compiled with sanitizers, for the host-side tests)
LIB_PATH = os.environ.get("M3_LIBRARY") or os.path.join(HERE, "libmamba3_ssm.so")

M3_OK, M3_ERR_NULL, M3_ERR_SHAPE, M3_ERR_UNSUPPORTED, M3_ERR_ALIGN, M3_ERR_WORKSPACE, M3_ERR_HIP = range(7)
M3_F32, M3_BF16 = 0, 1
M3_FLAG_CHUNK_WALK = 0x10000   # chunked_fwd: walk chunks even for short sequences
M3_FLAG_TOKEN_PATH = 0x20000   # chunked_fwd: token by token (at most M3_TOKEN_PATH_MAX_L tokens)
M3_TOKEN_PATH_MAX_L = 16       # longest call the token path takes
M3_TOKEN_PATH_SUBWALK_L = 8    # ... chosen by default when the sub-chunk walker covers the sizes
M3_NOALLOC_SCRATCH_BYTES = 48 << 20  # the fixed workspace of mamba3_ssm_chunked_fwd_noalloc, per GPU
ABI_SYMBOLS = ("mamba3_ssm_chunked_fwd", "mamba3_ssm_chunked_fwd_workspace_size", "mamba3_ssm_chunked_fwd_noalloc",
               "mamba3_ssm_chunked_bwd",
               "mamba3_ssm_chunked_bwd_workspace_size", "mamba3_ssm_decode_step",
               "mamba3_rope_bc", "mamba3_rope_bc_workspace_size", "mamba3_bc_prologue",
               "mamba3_bc_prologue_workspace_size", "mamba3_status_string", "mamba3_abi_version")


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class Mamba3Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmamba3_ssm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with state_space_sequence_03_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
        dp = ctypes.POINTER(Dims)
        L.mamba3_ssm_chunked_fwd.argtypes = [dp] + [vp] * 12 + [vp, sz, vp]
        L.mamba3_ssm_chunked_fwd.restype = ctypes.c_int
        L.mamba3_ssm_chunked_fwd_noalloc.argtypes = [dp] + [vp] * 12 + [vp]
        L.mamba3_ssm_chunked_fwd_noalloc.restype = ctypes.c_int
        L.mamba3_ssm_chunked_fwd_workspace_size.argtypes = [dp]
        L.mamba3_ssm_chunked_fwd_workspace_size.restype = sz
        L.mamba3_ssm_chunked_bwd.argtypes = [dp] + [vp] * 22 + [vp, sz, vp]
        L.mamba3_ssm_chunked_bwd.restype = ctypes.c_int
        L.mamba3_ssm_chunked_bwd_workspace_size.argtypes = [dp]
        L.mamba3_ssm_chunked_bwd_workspace_size.restype = sz
        L.mamba3_ssm_decode_step.argtypes = [dp] + [vp] * 11 + [vp]
        L.mamba3_ssm_decode_step.restype = ctypes.c_int
        L.mamba3_rope_bc.argtypes = [dp] + [vp] * 8 + [vp, sz, vp]
        L.mamba3_rope_bc.restype = ctypes.c_int
        L.mamba3_rope_bc_workspace_size.argtypes = [dp]
        L.mamba3_rope_bc_workspace_size.restype = sz
        L.mamba3_bc_prologue.argtypes = [dp, ctypes.c_int64, vp, vp, vp, vp, ctypes.c_float] + [vp] * 6 + [vp, sz, vp]
        L.mamba3_bc_prologue.restype = ctypes.c_int
        L.mamba3_bc_prologue_workspace_size.argtypes = [dp]
        L.mamba3_bc_prologue_workspace_size.restype = sz
        L.mamba3_status_string.argtypes = [ctypes.c_int]
        L.mamba3_status_string.restype = ctypes.c_char_p
        L.mamba3_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().mamba3_status_string(int(status)).decode()
    except Exception:  # library missing: still describe the code
        return "unknown"


def _torch():
    import torch
    return torch


def _io_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return M3_BF16
    if t.dtype == torch.float32:
        return M3_F32
    raise TypeError(f"io dtype must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(name, t, shape, dtype, device):
    """Shape, dtype and device of an operand (None: absent).  The C ABI takes
    raw pointers and cannot see shapes, so the binding checks them before any
    call: a wrong shape would otherwise be read or written out of bounds."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != M3_OK:
        raise Mamba3Error(status, what)


def make_dims(batch, seqlen, nheads, headdim, dstate, rank, chunk, io_dtype, flags=0) -> Dims:
    return Dims(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(rank), int(chunk),
                int(io_dtype), int(flags))


def chunked_fwd_workspace_size(dims: Dims) -> int:
    return int(lib().mamba3_ssm_chunked_fwd_workspace_size(ctypes.byref(dims)))


def rope_bc_workspace_size(dims: Dims) -> int:
    return int(lib().mamba3_rope_bc_workspace_size(ctypes.byref(dims)))


def _core_operands(torch, x, B, C, dt, A, lam, theta, h0, prev_B, prev_x):
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    io, f32, dev = x.dtype, torch.float32, x.device
    for name, t in (("B", B), ("C", C)):
        _expect(name, t, (b, L, H, R, N), io, dev)
    for name, t in (("dt", dt), ("A", A), ("lam", lam)):
        _expect(name, t, (b, L, H), f32, dev)
    _expect("theta", theta, (b, L, H, N // 2), f32, dev)
    _expect("h0", h0, (b, H, N, P), f32, dev)
    _expect("prev_B", prev_B, (b, H, R, N), io, dev)
    _expect("prev_x", prev_x, (b, H, R, P), io, dev)


def mamba3_ssm_chunked_fwd(x, B, C, dt, A, lam, theta, h0=None, prev_B=None, prev_x=None, *, chunk=64,
                           segments=0, chunk_walk=False, token_path=False, y=None, h_final=None, want_final=True,
                           workspace=None, stream=None):
    """Whole-sequence forward.  Returns (y, h_final) (h_final None if not wanted).
    chunk_walk / token_path force one of the two paths for short calls (the
    library picks one by default)."""
    torch = _torch()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    _core_operands(torch, x, B, C, dt, A, lam, theta, h0, prev_B, prev_x)
    _expect("y", y, x.shape, x.dtype, x.device)
    _expect("h_final", h_final, (b, H, N, P), torch.float32, x.device)
    flags = segments | (M3_FLAG_CHUNK_WALK if chunk_walk else 0) | (M3_FLAG_TOKEN_PATH if token_path else 0)
    dims = make_dims(b, L, H, P, N, R, chunk, _io_code(x), flags=flags)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None and want_final:
        h_final = torch.empty((b, H, N, P), device=x.device, dtype=torch.float32)
    ws_bytes = chunked_fwd_workspace_size(dims)
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, device=x.device, dtype=torch.uint8)
    st = lib().mamba3_ssm_chunked_fwd(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A),
                                      _ptr(lam), _ptr(theta), _ptr(h0), _ptr(prev_B), _ptr(prev_x), _ptr(y),
                                      _ptr(h_final), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel() if workspace is not None else 0),
                                      _stream(stream))
    _check(st, "mamba3_ssm_chunked_fwd")
    return y, h_final


def mamba3_ssm_chunked_fwd_noalloc(x, B, C, dt, A, lam, theta, h0=None, prev_B=None, prev_x=None, *, y, h_final,
                                   chunk=64, segments=0, stream=None):
    """mamba3_ssm_chunked_fwd with the workspace taken from the library's fixed
    per-GPU array: the caller passes every output (y, h_final may be None) and
    the call allocates nothing.  Calls that overlap on one GPU race on that
    array."""
    torch = _torch()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    _core_operands(torch, x, B, C, dt, A, lam, theta, h0, prev_B, prev_x)
    if y is None:
        raise ValueError("y is required (this entry point allocates nothing)")
    _expect("y", y, x.shape, x.dtype, x.device)
    _expect("h_final", h_final, (b, H, N, P), torch.float32, x.device)
    dims = make_dims(b, L, H, P, N, R, chunk, _io_code(x), flags=segments)
    st = lib().mamba3_ssm_chunked_fwd_noalloc(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A),
                                              _ptr(lam), _ptr(theta), _ptr(h0), _ptr(prev_B), _ptr(prev_x), _ptr(y),
                                              _ptr(h_final), _stream(stream))
    _check(st, "mamba3_ssm_chunked_fwd_noalloc")
    return y, h_final


def chunked_bwd_workspace_size(dims: Dims) -> int:
    return int(lib().mamba3_ssm_chunked_bwd_workspace_size(ctypes.byref(dims)))


def mamba3_ssm_chunked_bwd(x, B, C, dt, A, lam, theta, dy, h0=None, prev_B=None, prev_x=None, dh_final=None, *,
                           chunk=64, segments=0, want_dh0=True, workspace=None, out=None, stream=None):
    """Backward of the chunked forward.  Returns a dict with dx, dB, dC (io dtype),
    ddt, dA, dlam, dtheta (fp32), dh0 (fp32, if wanted) and, when prev is given,
    dprev_B and dprev_x (io dtype).  segments: 0 = the library's choice, else
    the number of sequence segments walked in parallel (flags' low 16 bits).
    out: optional dict of preallocated outputs (any of the keys above)."""
    torch = _torch()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    _core_operands(torch, x, B, C, dt, A, lam, theta, h0, prev_B, prev_x)
    _expect("dy", dy, x.shape, x.dtype, x.device)
    _expect("dh_final", dh_final, (b, H, N, P), torch.float32, x.device)
    dims = make_dims(b, L, H, P, N, R, chunk, _io_code(x), flags=segments)
    given = dict(out or {})
    out = {"dx": torch.empty_like(x), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
           "ddt": torch.empty_like(dt), "dA": torch.empty_like(A), "dlam": torch.empty_like(lam),
           "dtheta": torch.empty_like(theta)}
    if want_dh0:
        out["dh0"] = torch.empty((b, H, N, P), device=x.device, dtype=torch.float32)
    if prev_B is not None:
        out["dprev_B"] = torch.empty_like(prev_B)
        out["dprev_x"] = torch.empty_like(prev_x)
    for k, t in given.items():
        if k not in out:
            raise ValueError(f"out: unexpected or unwanted output {k!r}")
        _expect(k, t, out[k].shape, out[k].dtype, x.device)
        out[k] = t
    ws_bytes = chunked_bwd_workspace_size(dims)
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, device=x.device, dtype=torch.uint8)
    st = lib().mamba3_ssm_chunked_bwd(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(lam),
                                      _ptr(theta), _ptr(h0), _ptr(prev_B), _ptr(prev_x), _ptr(dy), _ptr(dh_final),
                                      _ptr(out["dx"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["ddt"]),
                                      _ptr(out["dA"]), _ptr(out["dlam"]), _ptr(out["dtheta"]), _ptr(out.get("dh0")),
                                      _ptr(out.get("dprev_B")), _ptr(out.get("dprev_x")), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel() if workspace is not None else 0),
                                      _stream(stream))
    _check(st, "mamba3_ssm_chunked_bwd")
    return out


def mamba3_ssm_decode_step(state, x, B, C, dt, A, lam, theta, prev_B=None, prev_x=None, *, y=None, stream=None):
    """One token, state updated in place.  Shapes: state (b,H,N,P) fp32, x (b,H,R,P),
    B/C (b,H,R,N), dt/A/lam (b,H), theta (b,H,N/2).  Returns y (b,H,R,P)."""
    torch = _torch()
    b, H, R, P = x.shape
    N = B.shape[-1]
    io, f32, dev = x.dtype, torch.float32, x.device
    _expect("state", state, (b, H, N, P), f32, dev)
    for name, t in (("B", B), ("C", C), ("prev_B", prev_B)):
        _expect(name, t, (b, H, R, N), io, dev)
    _expect("prev_x", prev_x, (b, H, R, P), io, dev)
    for name, t in (("dt", dt), ("A", A), ("lam", lam)):
        _expect(name, t, (b, H), f32, dev)
    _expect("theta", theta, (b, H, N // 2), f32, dev)
    _expect("y", y, x.shape, io, dev)
    dims = make_dims(b, 1, H, P, N, R, 16, _io_code(x))
    if y is None:
        y = torch.empty_like(x)
    st = lib().mamba3_ssm_decode_step(ctypes.byref(dims), _ptr(state), _ptr(x), _ptr(B), _ptr(C), _ptr(dt),
                                      _ptr(A), _ptr(lam), _ptr(theta), _ptr(prev_B), _ptr(prev_x), _ptr(y),
                                      _stream(stream))
    _check(st, "mamba3_ssm_decode_step")
    return y


def mamba3_rope_bc(B, C, dt, theta, angle0=None, *, B_rot=None, C_rot=None, angle_final=None,
                   want_final=True, workspace=None, stream=None):
    """Cumulative-angle rotation.  Returns (B_rot, C_rot, angle_final)."""
    torch = _torch()
    b, L, H, R, N = B.shape
    io, f32, dev = B.dtype, torch.float32, B.device
    for name, t in (("C", C), ("B_rot", B_rot), ("C_rot", C_rot)):
        _expect(name, t, B.shape, io, dev)
    _expect("dt", dt, (b, L, H), f32, dev)
    _expect("theta", theta, (b, L, H, N // 2), f32, dev)
    _expect("angle0", angle0, (b, H, N // 2), f32, dev)
    _expect("angle_final", angle_final, (b, H, N // 2), f32, dev)
    dims = make_dims(b, L, H, 16, N, R, 16, _io_code(B))
    if B_rot is None:
        B_rot = torch.empty_like(B)
    if C_rot is None:
        C_rot = torch.empty_like(C)
    if angle_final is None and want_final:
        angle_final = torch.empty((b, H, N // 2), device=B.device, dtype=torch.float32)
    ws_bytes = rope_bc_workspace_size(dims)
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, device=B.device, dtype=torch.uint8)
    st = lib().mamba3_rope_bc(ctypes.byref(dims), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta), _ptr(angle0),
                              _ptr(B_rot), _ptr(C_rot), _ptr(angle_final), _ptr(workspace),
                              ctypes.c_size_t(workspace.numel() if workspace is not None else 0),
                              _stream(stream))
    _check(st, "mamba3_rope_bc")
    return B_rot, C_rot, angle_final


def bc_prologue_workspace_size(dims: Dims) -> int:
    return int(lib().mamba3_bc_prologue_workspace_size(ctypes.byref(dims)))


def mamba3_bc_prologue(u, W, dt, theta, nheads, rank, dstate, gain=None, bias=None, eps=1e-5, angle0=None, *,
                       B_rot=None, C_rot=None, angle_final=None, want_final=True, workspace=None, stream=None):
    """Projection of u (B, L, D) by W (2*H*R*N, D) to B and C, RMS-normalised
    per (token, head, rank) vector with gain and bias, and rotated by the
    cumulative angle.  Returns (B_rot, C_rot, angle_final)."""
    torch = _torch()
    b, L, D = u.shape
    H, R, N = nheads, rank, dstate
    io, f32, dev = u.dtype, torch.float32, u.device
    _expect("W", W, (2 * H * R * N, D), io, dev)
    _expect("dt", dt, (b, L, H), f32, dev)
    _expect("theta", theta, (b, L, H, N // 2), f32, dev)
    for name, t in (("gain", gain), ("bias", bias)):
        _expect(name, t, (2, H, R, N), f32, dev)
    for name, t in (("B_rot", B_rot), ("C_rot", C_rot)):
        _expect(name, t, (b, L, H, R, N), io, dev)
    for name, t in (("angle0", angle0), ("angle_final", angle_final)):
        _expect(name, t, (b, H, N // 2), f32, dev)
    dims = make_dims(b, L, H, 16, N, R, 16, _io_code(u))
    if B_rot is None:
        B_rot = torch.empty((b, L, H, R, N), device=u.device, dtype=u.dtype)
    if C_rot is None:
        C_rot = torch.empty((b, L, H, R, N), device=u.device, dtype=u.dtype)
    if angle_final is None and want_final:
        angle_final = torch.empty((b, H, N // 2), device=u.device, dtype=torch.float32)
    ws_bytes = bc_prologue_workspace_size(dims)
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, device=u.device, dtype=torch.uint8)
    st = lib().mamba3_bc_prologue(ctypes.byref(dims), ctypes.c_int64(D), _ptr(u), _ptr(W), _ptr(gain), _ptr(bias),
                                  ctypes.c_float(eps), _ptr(dt), _ptr(theta), _ptr(angle0), _ptr(B_rot), _ptr(C_rot),
                                  _ptr(angle_final), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel() if workspace is not None else 0), _stream(stream))
    _check(st, "mamba3_bc_prologue")
    return B_rot, C_rot, angle_final


chunked_fwd = mamba3_ssm_chunked_fwd
chunked_fwd_noalloc = mamba3_ssm_chunked_fwd_noalloc
chunked_bwd = mamba3_ssm_chunked_bwd
decode_step = mamba3_ssm_decode_step
rope_bc = mamba3_rope_bc
bc_prologue = mamba3_bc_prologue
