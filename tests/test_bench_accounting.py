"""The benchmark's algorithmic accounting (bytes and flops per token-head,
bytes per decode step), checked against the figures worked out by hand for
the five workloads: the bytes and causal / dense flop counts of the chunked
form at the configured chunk, the decode step's traffic (the fp32 state read
and written once plus the inputs), and the backward's traffic.  CPU only; the
roofline fractions that bench.py prints rest on these numbers.
"""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from state_space_sequence_03_amd.inputs import PROLOGUE, WORKLOADS  # noqa: E402


@pytest.mark.parametrize("name,s_io,bytes_,causal,dense", [
    # B per token-head = s_io R (2P + 2N) + 12 + 2N; flops causal R^2 (N+P)(Q+1) + 4RNP, dense 2 Q R^2 (N+P) + 4RNP
    ("tiny_siso_f32", 4, 300, 2080, 3072),
    ("siso_bf16", 2, 652, 24704, 32768),
    ("mimo_bf16", 2, 2188, 198656, 327680),
    ("long_mimo_bf16", 2, 3340, 330752, 524288),
])
def test_prefill_accounting(name, s_io, bytes_, causal, dense):
    w = WORKLOADS[name]
    assert bench.prefill_bytes_per_token_head(w, s_io) == bytes_
    assert bench.prefill_flops_per_token_head(w, True, at_configured_chunk=True) == causal
    assert bench.prefill_flops_per_token_head(w, False, at_configured_chunk=True) == dense


def test_walked_chunk_and_kernel():
    assert bench.walked_chunk(WORKLOADS["mimo_bf16"]) == 32
    assert bench.walked_chunk(WORKLOADS["long_mimo_bf16"]) == 16
    assert bench.walked_chunk(WORKLOADS["tiny_siso_f32"]) == 32      # fp32: the configured chunk
    assert bench.walker_kernel(WORKLOADS["mimo_bf16"]) == "subchunk_walk_kernel<64,4>"


def test_decode_step_bytes():
    # batch 256, H 64, N = P = 64, R 4, per (b,h): the fp32 state read and written
    # (2 N P 4 B); x, B, C and prev_B, prev_x (R(P + 2N) + R(N + P) bf16 values);
    # dt, A, lam and theta (12 + 4 N/2 B); y (R P bf16 values)
    w = WORKLOADS["decode_mimo_bf16"]
    BH = 256 * 64
    want = 2 * BH * 64 * 64 * 4 + BH * (4 * 64 + 2 * 4 * 64) * 2 + BH * (4 * 64 + 4 * 64) * 2 \
        + BH * (12 + 32 * 4) + BH * 4 * 64 * 2
    assert bench.decode_bytes_per_step(w) == want == 589_496_320


def test_backward_accounting():
    w = WORKLOADS["mimo_bf16"]
    assert bench.bwd_chunk(w) == 16 and bench.bwd_chunk(WORKLOADS["long_mimo_bf16"]) == 8
    # inputs + dy read (2 R (2P + 2N) + 12 + 2N), gradients written (2 R (P + 2N) + 12 + 2N),
    # the chunk-start states written and read once (2 N P 4 / 16)
    assert bench.backward_bytes_per_token_head(w) == 2 * 4 * 256 + 140 + 2 * 4 * 192 + 140 + 2048 == 5912
    ck, walk = bench.backward_flops_per_token_head(w)
    assert ck == 2 * 64 * 64 * 64 / 16 and ck + walk == 327_680


def test_rope_bytes():
    assert bench.rope_bytes_per_token_head(WORKLOADS["mimo_bf16"]) == 4 * 4 * 64 * 2 + 4 + 128


def test_prologue_flops():
    # 2 M F D with M = B L tokens and F = 2 H R N features
    M = PROLOGUE["batch"] * PROLOGUE["seqlen"]
    F = 2 * PROLOGUE["nheads"] * PROLOGUE["rank"] * PROLOGUE["dstate"]
    assert 2 * M * F * PROLOGUE["d_model"] == 4_398_046_511_104


@pytest.mark.parametrize("name", sorted(bench.TRAFFIC))
def test_counter_summary_traffic_is_near_algorithmic(name):
    """Each committed HBM-traffic summary parses, and while it was taken on the
    current sources (its recorded hash) the calibrated counter bytes lie within
    a few percent above the algorithmic bytes: no wasted re-reads."""
    t = bench.measured_traffic(name)
    if t is None:
        pytest.skip(f"{bench.TRAFFIC[name][0]} was taken on other sources; take the counters again")
    if name == "decode":
        algo = bench.decode_bytes_per_step(WORKLOADS["decode_mimo_bf16"])
    else:
        w = WORKLOADS[name]
        algo = w.batch * w.seqlen * w.nheads * bench.prefill_bytes_per_token_head(w)
    assert 1.0 <= t / algo <= 1.06, (name, t / algo)


@pytest.mark.parametrize("name", sorted(bench.SQ_SUMMARY))
def test_counter_summary_mfma_count(name):
    """The walkers' SQ_INSTS_MFMA x 16,384 flop lies between the causal and the
    dense flop count of the walked chunk (tiles above the causal diagonal are
    skipped, the state's hi + lo products are counted twice)."""
    fl = bench.issued_mfma_flops(name)
    if fl is None:
        pytest.skip(f"{bench.SQ_SUMMARY[name]} was taken on other sources; take the counters again")
    w = WORKLOADS[name]
    th = w.batch * w.seqlen * w.nheads
    assert th * bench.prefill_flops_per_token_head(w, causal=True) <= fl
    assert fl <= 1.5 * th * bench.prefill_flops_per_token_head(w, causal=False)


def test_clock_summary():
    """The prologue's measured clock, when its summary matches the current
    sources, lies between the lowest clock the power management uses under load
    and the 2.4 GHz engine clock (a little above it: the GRBM count and the
    dispatch timestamps are not taken at exactly the same instants)."""
    clk = bench.prologue_clock_ghz()
    if clk is None:
        pytest.skip(f"{bench.CLOCK_SUMMARY} was taken on other sources; take the counters again")
    assert 1.0 < clk < 2.6
