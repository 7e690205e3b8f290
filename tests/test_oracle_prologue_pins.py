"""Pins of the B/C prologue oracle (oracle/prologue.py) against closed forms,
invariants and the pinned core oracle; CPU only.

  * one-hot projection: with W's rows one-hot, every output vector (no gain,
    bias or rotation) is a positive multiple of the u entries those rows pick,
    which fixes the row order of W and the (B or C, head, rank, entry) split;
  * unit RMS: gain 1, bias 0, eps 0, no rotation: every (token, head, rank)
    vector of B and C has mean square exactly 1 over its N entries;
  * a constant vector c over N: it leaves the normalisation as
    c / sqrt(c^2 + eps) * gain + bias, which fixes where eps enters;
  * u = 0: the output is the rotated bias alone (bias after the normalisation);
  * quarter turns (dt = 1, theta = pi/2): token t (from 1) is rotated by
    -t*pi/2, a 4-cycle of exact pair permutations with signs, and angle_final
    = angle0 + L*pi/2;
  * RoPE frame: the core oracle run on the prologue's rotated B and C with
    theta = 0 gives the same y as the core oracle on the unrotated ones with
    theta (the rotation form of the complex state, pinned in
    test_oracle_pins.py).
Each planted mistake of the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.prologue import bc_prologue
from state_space_sequence_03_amd.inputs import numpy_inputs, prologue_numpy


def base(seed=3, b=2, L=7, H=3, R=2, N=8, D=24, **kw):
    return prologue_numpy(b, L, H, N, R, D, seed=seed, **kw), (H, R, N)


def call(inp, dims, mutant=0, eps=1e-5, **over):
    H, R, N = dims
    a = dict(inp)
    a.update(over)
    return bc_prologue(a["u"], a["W"], a["dt"], a["theta"], H, R, N, gain=a.get("gain"), bias=a.get("bias"),
                       eps=eps, angle0=a.get("angle0"), mutant=mutant)


def pin_one_hot(mutant=0):
    inp, (H, R, N) = base(seed=5)
    D = inp["u"].shape[-1]
    rng = np.random.default_rng(9)
    pick = rng.integers(0, D, 2 * H * R * N)
    W = np.zeros((2 * H * R * N, D))
    W[np.arange(2 * H * R * N), pick] = 1.0
    Bo, Co, _ = call(inp, (H, R, N), mutant, eps=0.0, W=W, gain=None, bias=None,
                     theta=np.zeros_like(inp["theta"]))
    got = np.stack([Bo, Co], axis=2)                               # (b, L, 2, H, R, N)
    want = inp["u"][..., pick].reshape(got.shape)                  # the picked entries
    ratio = got / want
    # one positive factor per (token, B or C, head, rank) vector
    spread = np.max(np.abs(ratio - ratio[..., :1]), axis=-1)
    return bool(np.all(ratio > 0) and np.max(spread) < 1e-12)


def pin_unit_rms(mutant=0):
    inp, dims = base(seed=6)
    Bo, Co, _ = call(inp, dims, mutant, eps=0.0, gain=None, bias=None, theta=np.zeros_like(inp["theta"]))
    ms = np.concatenate([np.mean(Bo ** 2, -1).ravel(), np.mean(Co ** 2, -1).ravel()])
    return bool(np.max(np.abs(ms - 1.0)) < 1e-12)


def pin_constant_vector(mutant=0):
    inp, (H, R, N) = base(seed=7)
    D = inp["u"].shape[-1]
    # every row of W the same: each output vector is the constant c = w . u_t
    w = np.random.default_rng(1).standard_normal(D) * 0.05
    W = np.tile(w, (2 * H * R * N, 1))
    eps = 0.5
    Bo, Co, _ = call(inp, (H, R, N), mutant, eps=eps, W=W, theta=np.zeros_like(inp["theta"]))
    c = inp["u"].astype(np.float64) @ w                            # (b, L)
    scale = (c / np.sqrt(c * c + eps))[:, :, None, None, None]
    g, bi = inp["gain"].astype(np.float64), inp["bias"].astype(np.float64)
    return bool(max(np.max(np.abs(Bo - (scale * g[0] + bi[0]))), np.max(np.abs(Co - (scale * g[1] + bi[1])))) < 1e-12)


def pin_zero_input(mutant=0):
    inp, dims = base(seed=8, with_angle0=True)
    inp["u"] = np.zeros_like(inp["u"])
    Bo, Co, _ = call(inp, dims, mutant, theta=np.zeros_like(inp["theta"]))
    # theta = 0: the rotation is by angle0 alone; check its pair norms and the
    # unrotated case separately
    nb = np.hypot(Bo[..., 0::2], Bo[..., 1::2])
    bias = inp["bias"].astype(np.float64)
    want = np.hypot(bias[0, ..., 0::2], bias[0, ..., 1::2])
    ok = np.isfinite(Bo).all() and np.max(np.abs(nb - want)) < 1e-12
    inp.pop("angle0")
    Bo, Co, _ = call(inp, dims, mutant, theta=np.zeros_like(inp["theta"]))
    ok = ok and np.max(np.abs(Bo - inp["bias"][0])) < 1e-12 and np.max(np.abs(Co - inp["bias"][1])) < 1e-12
    return bool(ok)


def pin_quarter_turns(mutant=0):
    inp, dims = base(seed=10, L=9, with_angle0=False)
    L = inp["u"].shape[1]
    ref_B, ref_C, _ = call(inp, dims, mutant, theta=np.zeros_like(inp["theta"]))
    qt = dict(dt=np.ones(inp["dt"].shape), theta=np.full(inp["theta"].shape, math.pi / 2))
    Bo, Co, af = call(inp, dims, mutant, **qt)
    ok = True
    for out, ref in ((Bo, ref_B), (Co, ref_C)):
        x, y = ref[..., 0::2], ref[..., 1::2]
        for t in range(L):
            turn = (t + 1) % 4                                     # rotation by -turn * pi/2
            ex, ey = [(x, y), (y, -x), (-x, -y), (-y, x)][turn]
            ok = ok and np.max(np.abs(out[:, t, ..., 0::2] - ex[:, t])) < 1e-12
            ok = ok and np.max(np.abs(out[:, t, ..., 1::2] - ey[:, t])) < 1e-12
    ok = ok and np.max(np.abs(af - L * math.pi / 2)) < 1e-12
    return bool(ok)


def pin_rope_frame(mutant=0):
    """Core oracle on (rotated B, C; theta = 0) equals the core oracle on the
    unrotated normalised B, C with theta: the rotation is the RoPE frame of the
    core's complex state."""
    b, L, H, R, N, D, P = 1, 12, 2, 2, 8, 16, 4
    pin, dims = base(seed=11, b=b, L=L, H=H, R=R, N=N, D=D)
    core = numpy_inputs(b, L, H, P, N, R, seed=12)
    Bo, Co, _ = call(pin, dims, mutant, dt=core["dt"], theta=core["theta"])
    Bn, Cn, _ = call(pin, dims, mutant, dt=core["dt"], theta=np.zeros_like(core["theta"]))  # normalised, unrotated
    y_rot, _ = oracle.forward(core["x"], Bo, Co, core["dt"], core["A"], core["lam"], np.zeros_like(core["theta"]))
    y_ref, _ = oracle.forward(core["x"], Bn, Cn, core["dt"], core["A"], core["lam"], core["theta"])
    return bool(np.max(np.abs(y_rot - y_ref)) < 1e-10 * max(1.0, np.max(np.abs(y_ref))))


PINS = [pin_one_hot, pin_unit_rms, pin_constant_vector, pin_zero_input, pin_quarter_turns, pin_rope_frame]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_prologue_pin(pin):
    assert pin(), pin.__name__


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6])
def test_prologue_mutants_are_caught(mutant):
    with np.errstate(divide="ignore", invalid="ignore"):
        failed = [p.__name__ for p in PINS if not p(mutant)]
    assert failed, f"planted mistake {mutant} passed every pin"
