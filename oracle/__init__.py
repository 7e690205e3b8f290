"""fp64 CPU oracle of the Mamba-3 SSM layer core (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
(``state_space_sequence_03_amd``) never does, and this package never imports
the product.

The arithmetic lives in ``mamba3_oracle.c`` (plain C99, libm, pthreads), which
states the recurrence and the passages of the pages it follows: the
exponential-trapezoidal update, the rotation (RoPE) form of the complex state
and the rank-R (MIMO) input and output products, all from linkstar.cloud/
article/869, sections "第一刀", "第二刀" and "第三刀".

This module only converts arrays to contiguous float64, builds the C file with
gcc when the shared object is missing or older than its source, and calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba3_oracle.c")
_LOCK = threading.Lock()
_LIBS: dict[int, ctypes.CDLL] = {}


def so_path(mutant: int = 0) -> str:
    name = "liboracle_mamba3.so" if mutant == 0 else f"liboracle_mamba3_mutant{mutant}.so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    out = so_path(mutant)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _lib(mutant: int = 0) -> ctypes.CDLL:
    with _LOCK:
        if mutant not in _LIBS:
            lib = ctypes.CDLL(build(mutant))
            d = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.mamba3_oracle_forward.argtypes = [i64] * 6 + [d] * 12 + [ctypes.c_int]
            lib.mamba3_oracle_forward.restype = ctypes.c_int
            lib.mamba3_oracle_backward.argtypes = [i64] * 6 + [d] * 22 + [ctypes.c_int]
            lib.mamba3_oracle_backward.restype = ctypes.c_int
            lib.mamba3_oracle_rope_bc.argtypes = [i64] * 5 + [d] * 8
            lib.mamba3_oracle_rope_bc.restype = ctypes.c_int
            lib.mamba3_oracle_version.restype = ctypes.c_int
            _LIBS[mutant] = lib
        return _LIBS[mutant]


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(x, B, C, dt, A, lam, theta, h0=None, prev_B=None, prev_x=None,
            nthreads: int = 0, mutant: int = 0):
    """Token-by-token recurrence over a whole sequence.

    Shapes: x (b,L,H,R,P); B, C (b,L,H,R,N); dt, A, lam (b,L,H);
    theta (b,L,H,N/2); h0 (b,H,N,P) or None; prev_B (b,H,R,N) and
    prev_x (b,H,R,P) or None (both or neither).
    Returns (y (b,L,H,R,P), h_final (b,H,N,P)) as float64 arrays; h_final is
    in the true (un-rotated) frame.
    """
    x, B, C, dt, A, lam, theta = (_f64(a) for a in (x, B, C, dt, A, lam, theta))
    h0, prev_B, prev_x = _f64(h0), _f64(prev_B), _f64(prev_x)
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    assert B.shape == (b, L, H, R, N) and C.shape == B.shape
    assert dt.shape == (b, L, H) and A.shape == dt.shape and lam.shape == dt.shape
    assert theta.shape == (b, L, H, N // 2)
    if h0 is not None:
        assert h0.shape == (b, H, N, P)
    if (prev_B is None) != (prev_x is None):
        raise ValueError("prev_B and prev_x go together")
    if prev_B is not None:
        assert prev_B.shape == (b, H, R, N) and prev_x.shape == (b, H, R, P)
    y = np.zeros((b, L, H, R, P), dtype=np.float64)
    hf = np.zeros((b, H, N, P), dtype=np.float64)
    rc = _lib(mutant).mamba3_oracle_forward(
        b, L, H, P, N, R, _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
        _ptr(h0), _ptr(prev_B), _ptr(prev_x), _ptr(y), _ptr(hf), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return y, hf


def backward(x, B, C, dt, A, lam, theta, dy, h0=None, prev_B=None, prev_x=None, dh_final=None,
             nthreads: int = 0, mutant: int = 0):
    """Gradients of  sum_t <dy_t, y_t> + <dh_final, h_final>  for the forward above.

    Returns a dict with dx, dB, dC, ddt, dA, dlam, dtheta (shapes of the
    inputs), dh0 (b,H,N,P) and, when prev_B is given, dprev_B and dprev_x.
    """
    x, B, C, dt, A, lam, theta, dy = (_f64(a) for a in (x, B, C, dt, A, lam, theta, dy))
    h0, prev_B, prev_x, dh_final = _f64(h0), _f64(prev_B), _f64(prev_x), _f64(dh_final)
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    assert dy.shape == x.shape
    if (prev_B is None) != (prev_x is None):
        raise ValueError("prev_B and prev_x go together")
    out = {k: np.zeros_like(v) for k, v in (("dx", x), ("dB", B), ("dC", C), ("ddt", dt), ("dA", A),
                                                 ("dlam", lam), ("dtheta", theta))}
    out["dh0"] = np.zeros((b, H, N, P), dtype=np.float64)
    if prev_B is not None:
        out["dprev_B"] = np.zeros_like(prev_B)
        out["dprev_x"] = np.zeros_like(prev_x)
    rc = _lib(mutant).mamba3_oracle_backward(
        b, L, H, P, N, R, _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
        _ptr(h0), _ptr(prev_B), _ptr(prev_x), _ptr(dy), _ptr(dh_final),
        *(_ptr(out[k]) for k in ("dx", "dB", "dC", "ddt", "dA", "dlam", "dtheta", "dh0")),
        _ptr(out.get("dprev_B")), _ptr(out.get("dprev_x")), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out


def decode_step(state, x, B, C, dt, A, lam, theta, prev_B=None, prev_x=None, mutant: int = 0):
    """One token: the whole-sequence recurrence with L = 1.

    state (b,H,N,P) true frame; x (b,H,R,P); B, C (b,H,R,N); dt, A, lam (b,H);
    theta (b,H,N/2).  Returns (new_state (b,H,N,P), y (b,H,R,P)).
    """
    add_l = lambda a: None if a is None else _f64(a)[:, None]
    y, hf = forward(add_l(x), add_l(B), add_l(C), add_l(dt), add_l(A), add_l(lam), add_l(theta),
                    h0=state, prev_B=prev_B, prev_x=prev_x, mutant=mutant)
    return hf, y[:, 0]


def rope_bc(B, C, dt, theta, angle0=None, mutant: int = 0):
    """Cumulative-angle rotation of B and C.  Returns (B_rot, C_rot, angle_final)."""
    B, C, dt, theta, angle0 = _f64(B), _f64(C), _f64(dt), _f64(theta), _f64(angle0)
    b, L, H, R, N = B.shape
    Br = np.zeros_like(B)
    Cr = np.zeros_like(C)
    af = np.zeros((b, H, N // 2), dtype=np.float64)
    rc = _lib(mutant).mamba3_oracle_rope_bc(b, L, H, N, R, _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
                                            _ptr(angle0), _ptr(Br), _ptr(Cr), _ptr(af))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return Br, Cr, af


# The B/C prologue (projection, RMS normalisation, bias, rotation) in numpy.
from .prologue import bc_prologue  # noqa: E402
