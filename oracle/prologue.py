"""fp64 CPU oracle of the B/C prologue in front of the Mamba-3 SSM core.

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests/,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may call
it; the product never does.

What it computes, per token t, head h, rank r (plain numpy in float64, the
matrix product the only library step):
  1. projection: p = W u_t, the rows of W being those of W_B then of W_C
     (papers.ananclaw.com/promo/explainers__2603-15569, "关键公式与“伪代码”":
     the block's input projection yields the input-dependent b and c);
  2. RMS normalisation of every (t, h, r) vector of B and of C over its N
     entries, with a per-entry gain, then a per-entry bias (linkstar.cloud/
     article/869, "架构上的其他改动": RMS normalisation of B and C in the manner
     of QK normalisation, and a learnable bias on B and C):
         v = p / sqrt(mean_n p^2 + eps) * gain + bias;
  3. the cumulative-angle rotation of rope_bc (linkstar.cloud/article/869,
     "第二刀", the RoPE form; the same page notes that the rotation can be
     fused with the projection so that B and C make no extra round trip):
         phi_t = angle0 + sum_{s<=t} dt_s theta_s,   out = R(-phi_t) v.

Readings where the pages say no more: the normalisation runs over the N
entries of one (token, head, rank) vector; the gain belongs to the
normalisation and the bias comes after it; eps is an argument.

``mutant`` plants one mistake (for the tests that show each pin catches
something): 1 normalises over all ranks of a head instead of each rank,
2 adds the bias before normalising, 3 rotates by +phi, 4 drops eps,
5 uses an exclusive angle sum, 6 splits the projected features as (head,
rank, B or C, entry).
"""
from __future__ import annotations

import numpy as np


def bc_prologue(u, W, dt, theta, nheads, rank, dstate, gain=None, bias=None, eps=1e-5, angle0=None,
                mutant: int = 0):
    """Returns (B_rot, C_rot, angle_final): (b, L, H, R, N) twice and (b, H, N/2), float64.

    u (b, L, D); W (2 H R N, D); dt (b, L, H); theta (b, L, H, N/2);
    gain, bias: None or (2, H, R, N); angle0: None or (b, H, N/2)."""
    H, R, N = nheads, rank, dstate
    u = np.asarray(u, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    b, L, D = u.shape
    if W.shape != (2 * H * R * N, D):
        raise ValueError("W must be (2*H*R*N, D)")
    # 1. projection, then split into (B or C, head, rank, entry)
    p = u.reshape(b * L, D) @ W.T
    if mutant == 6:
        p = np.moveaxis(p.reshape(b, L, H, R, 2, N), 4, 2)
    else:
        p = p.reshape(b, L, 2, H, R, N)
    g = np.ones((2, H, R, N)) if gain is None else np.asarray(gain, dtype=np.float64)
    bi = np.zeros((2, H, R, N)) if bias is None else np.asarray(bias, dtype=np.float64)
    # 2. RMS normalisation over the N entries of each vector, gain, bias
    if mutant == 2:
        p = p + bi
    if mutant == 1:
        ms = np.mean(p * p, axis=(-2, -1), keepdims=True)
    else:
        ms = np.mean(p * p, axis=-1, keepdims=True)
    v = p / np.sqrt(ms + (0.0 if mutant == 4 else eps)) * g
    if mutant != 2:
        v = v + bi
    # 3. angle: inclusive running sum of dt * theta along the sequence
    dt = np.asarray(dt, dtype=np.float64)
    theta = np.asarray(theta, dtype=np.float64)
    a0 = np.zeros((b, H, N // 2)) if angle0 is None else np.asarray(angle0, dtype=np.float64)
    inc = dt[..., None] * theta                      # (b, L, H, N/2)
    phi = a0[:, None] + np.cumsum(inc, axis=1)
    if mutant == 5:
        phi = phi - inc
    sign = -1.0 if mutant == 3 else 1.0
    cs, sn = np.cos(phi), sign * np.sin(phi)         # R(-phi) (x, y) = (c x + s y, -s x + c y)
    cs = cs[:, :, None, :, None, :]                  # broadcast over (B or C) and rank
    sn = sn[:, :, None, :, None, :]
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = cs * x0 + sn * x1
    out[..., 1::2] = -sn * x0 + cs * x1
    angle_final = a0 + inc.sum(axis=1)
    return out[:, :, 0], out[:, :, 1], angle_final
