"""Seeded synthetic inputs for the Mamba-3 SSM layer core.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle can be fed from
it.  The pages train on text corpora whose activations are not available;
these draws stand in for the SSM layer's activations at the pages' scale
(1.5B-parameter models, state sizes 64 and 128).

Distributions (std, not variance, as the second argument of N):
  x ~ N(0, 1);  B, C ~ N(0, 1/N) i.e. std 1/sqrt(N);
  dt = softplus(z), z ~ N(-2, 0.5);  A = -exp(U(0, ln 16));
  lam = sigmoid(N(0, 1));  theta ~ U(-pi, pi), one rate per rotation pair.
bf16 inputs are the round-to-nearest-even of the fp32 draws; whoever checks a
result consumes the rounded values.

Two generators:
  * ``numpy_inputs`` -- numpy ``default_rng(seed)``, for CPU tests and for
    small GPU cases (the same arrays go to both sides);
  * ``torch_inputs`` -- torch's Philox generator on the device, for the large
    workloads; parity tests copy sampled (b, h) slices of exactly these
    tensors to the host for the oracle.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32, BF16 = "f32", "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int      # P
    dstate: int       # N (even: N/2 rotation pairs)
    rank: int         # R (MIMO rank)
    chunk: int        # Q tokens per chunk
    io: str           # dtype of x, B, C, y and the previous-token caches
    decode_steps: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five synthetic workloads (sizes as stated for the method at 1.5B scale).
WORKLOADS = {
    "tiny_siso_f32": Workload("tiny_siso_f32", 1, 256, 2, 16, 16, 1, 32, F32),
    "siso_bf16": Workload("siso_bf16", 8, 4096, 64, 64, 64, 1, 64, BF16),
    "mimo_bf16": Workload("mimo_bf16", 8, 4096, 64, 64, 64, 4, 64, BF16),
    "decode_mimo_bf16": Workload("decode_mimo_bf16", 256, 1, 64, 64, 64, 4, 64, BF16, decode_steps=1024),
    "long_mimo_bf16": Workload("long_mimo_bf16", 1, 65536, 32, 64, 128, 4, 64, BF16),
}
WORKLOAD_ORDER = ["tiny_siso_f32", "siso_bf16", "mimo_bf16", "decode_mimo_bf16", "long_mimo_bf16"]


def seed_of(name: str) -> int:
    return 1000 + WORKLOAD_ORDER.index(name)


def round_bf16_np(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return them as fp32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def numpy_inputs(batch, seqlen, nheads, headdim, dstate, rank, io=F32, seed=0,
                 with_h0=False, with_prev=False, a_range=(0.0, math.log(16.0)),
                 dt_mu=-2.0, dt_sigma=0.5, theta_scale=math.pi):
    """Draw one set of inputs with numpy.  Returns a dict of float32 arrays
    (bf16-representable when io == 'bf16')."""
    rng = np.random.default_rng(seed)
    b, L, H, P, N, R = batch, seqlen, nheads, headdim, dstate, rank
    f = np.float32
    x = rng.standard_normal((b, L, H, R, P)).astype(f)
    Bm = (rng.standard_normal((b, L, H, R, N)) / math.sqrt(N)).astype(f)
    Cm = (rng.standard_normal((b, L, H, R, N)) / math.sqrt(N)).astype(f)
    z = rng.normal(dt_mu, dt_sigma, (b, L, H))
    dt = np.logaddexp(0.0, z).astype(f)  # softplus
    A = (-np.exp(rng.uniform(a_range[0], a_range[1], (b, L, H)))).astype(f)
    lam = (1.0 / (1.0 + np.exp(-rng.standard_normal((b, L, H))))).astype(f)
    theta = rng.uniform(-theta_scale, theta_scale, (b, L, H, N // 2)).astype(f)
    out = dict(x=x, B=Bm, C=Cm, dt=dt, A=A, lam=lam, theta=theta)
    if with_h0:
        out["h0"] = rng.standard_normal((b, H, N, P)).astype(f)
    if with_prev:
        out["prev_B"] = (rng.standard_normal((b, H, R, N)) / math.sqrt(N)).astype(f)
        out["prev_x"] = rng.standard_normal((b, H, R, P)).astype(f)
    if io == BF16:
        for k in ("x", "B", "C", "prev_B", "prev_x"):
            if k in out:
                out[k] = round_bf16_np(out[k])
    return out


def workload_numpy(w: Workload, seed=None, **kw):
    return numpy_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, w.io,
                        seed=seed_of(w.name) if seed is None else seed, **kw)


def torch_inputs(batch, seqlen, nheads, headdim, dstate, rank, io=BF16, seed=0, device="cuda",
                 with_h0=False, h0_std=1.0):
    """Draw one set of inputs on the device with torch's generator.
    x, B, C in the io dtype; dt, A, lam, theta (and h0) in fp32."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    b, L, H, P, N, R = batch, seqlen, nheads, headdim, dstate, rank
    io_t = torch.bfloat16 if io == BF16 else torch.float32
    f32 = torch.float32

    def normal(shape, std=1.0, mean=0.0):
        return torch.randn(shape, generator=g, device=device, dtype=f32).mul_(std).add_(mean)

    x = normal((b, L, H, R, P)).to(io_t)
    Bm = normal((b, L, H, R, N), 1.0 / math.sqrt(N)).to(io_t)
    Cm = normal((b, L, H, R, N), 1.0 / math.sqrt(N)).to(io_t)
    dt = torch.nn.functional.softplus(normal((b, L, H), 0.5, -2.0))
    A = -torch.exp(torch.rand((b, L, H), generator=g, device=device, dtype=f32) * math.log(16.0))
    lam = torch.sigmoid(normal((b, L, H)))
    theta = (torch.rand((b, L, H, N // 2), generator=g, device=device, dtype=f32) * 2.0 - 1.0) * math.pi
    out = dict(x=x, B=Bm, C=Cm, dt=dt, A=A, lam=lam, theta=theta)
    if with_h0:
        out["h0"] = normal((b, H, N, P), h0_std)
    return out


# The B/C prologue: the projection of the layer's token activations u to B and
# C, RMS normalisation of every (token, head, rank) vector over N, a bias, and
# the cumulative-angle rotation.  d_model = H*P/2 (an expansion of 2 from the
# model width to the H*P inner width) gives 2048 for the 1.5B shapes.
PROLOGUE = dict(batch=8, seqlen=4096, nheads=64, dstate=64, rank=4, d_model=2048)
PROLOGUE_SEED = 1100

# Prologue draws (std as the second argument of N):
#   u ~ N(0, 1) (activations after the block's input norm), bf16;
#   W ~ N(0, 1/D) i.e. std 1/sqrt(D), the rows of W_B then of W_C, bf16;
#   gain = 1 + N(0, 0.1^2), bias ~ N(0, 0.1^2), fp32, shape (2, H, R, N) (B then C);
#   dt, theta as for the core; angle0 ~ U(-pi, pi).


def prologue_numpy(batch, seqlen, nheads, dstate, rank, d_model, seed=0, with_gain=True, with_bias=True,
                   with_angle0=False):
    """Inputs of the B/C prologue drawn with numpy (u and W bf16-representable)."""
    rng = np.random.default_rng(seed)
    b, L, H, N, R, D = batch, seqlen, nheads, dstate, rank, d_model
    f = np.float32
    out = dict(u=round_bf16_np(rng.standard_normal((b, L, D)).astype(f)),
               W=round_bf16_np((rng.standard_normal((2 * H * R * N, D)) / math.sqrt(D)).astype(f)))
    z = rng.normal(-2.0, 0.5, (b, L, H))
    out["dt"] = np.logaddexp(0.0, z).astype(f)
    out["theta"] = rng.uniform(-math.pi, math.pi, (b, L, H, N // 2)).astype(f)
    if with_gain:
        out["gain"] = (1.0 + 0.1 * rng.standard_normal((2, H, R, N))).astype(f)
    if with_bias:
        out["bias"] = (0.1 * rng.standard_normal((2, H, R, N))).astype(f)
    if with_angle0:
        out["angle0"] = rng.uniform(-math.pi, math.pi, (b, H, N // 2)).astype(f)
    return out


def prologue_torch(batch, seqlen, nheads, dstate, rank, d_model, seed=0, device="cuda"):
    """Inputs of the B/C prologue drawn on the device (u, W bf16; the rest fp32)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    b, L, H, N, R, D = batch, seqlen, nheads, dstate, rank, d_model
    f32 = torch.float32

    def normal(shape, std=1.0, mean=0.0):
        return torch.randn(shape, generator=g, device=device, dtype=f32).mul_(std).add_(mean)

    u = normal((b, L, D)).to(torch.bfloat16)
    W = normal((2 * H * R * N, D), 1.0 / math.sqrt(D)).to(torch.bfloat16)
    dt = torch.nn.functional.softplus(normal((b, L, H), 0.5, -2.0))
    theta = (torch.rand((b, L, H, N // 2), generator=g, device=device, dtype=f32) * 2.0 - 1.0) * math.pi
    gain = normal((2, H, R, N), 0.1, 1.0)
    bias = normal((2, H, R, N), 0.1)
    return dict(u=u, W=W, dt=dt, theta=theta, gain=gain, bias=bias)
