"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function that include/mamba3_ssm.h
declares, and reject bad arguments with the documented status codes before
making any HIP call.  Only error paths are exercised, so the fake device
addresses used here are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba3_ssm.h")


@pytest.fixture(scope="module")
def L():
    from state_space_sequence_03_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ops


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba3_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(L.ABI_SYMBOLS)
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mamba3_abi_version() == 1


def test_header_constants_match_binding(L):
    text = open(HEADER).read()
    for name in ("M3_FLAG_CHUNK_WALK", "M3_FLAG_TOKEN_PATH", "M3_TOKEN_PATH_MAX_L", "M3_TOKEN_PATH_SUBWALK_L"):
        m = re.search(r"#define\s+" + name + r"\s+(\w+)", text)
        assert m, name
        assert int(m.group(1), 0) == getattr(L, name), name


def test_status_strings(L):
    for s in range(7):
        assert len(L.status_string(s)) >= 2 and L.status_string(s) != "unknown status"
    assert L.status_string(0) == "ok"


FAKE = 0x7F0000000000  # 16-byte aligned fake device address (never touched)


def call_fwd(L, dims, **over):
    p = {k: ctypes.c_void_p(FAKE) for k in ("x", "B", "C", "dt", "A", "lam", "theta", "y")}
    p.update(h0=None, prev_B=None, prev_x=None, h_final=None, ws=None)
    p.update(over)
    return L.lib().mamba3_ssm_chunked_fwd(ctypes.byref(dims), p["x"], p["B"], p["C"], p["dt"], p["A"], p["lam"],
                                          p["theta"], p["h0"], p["prev_B"], p["prev_x"], p["y"], p["h_final"],
                                          p["ws"], ctypes.c_size_t(over.get("ws_bytes", 0)), None)


def dims(L, **kw):
    base = dict(batch=2, seqlen=100, nheads=3, headdim=64, dstate=64, rank=4, chunk=64, io_dtype=L.M3_BF16, flags=0)
    base.update(kw)
    return L.make_dims(**base)


@pytest.mark.parametrize("kw,expect", [
    (dict(dstate=63), "M3_ERR_SHAPE"), (dict(batch=-1), "M3_ERR_SHAPE"), (dict(seqlen=-5), "M3_ERR_SHAPE"),
    (dict(headdim=0), "M3_ERR_SHAPE"), (dict(rank=0), "M3_ERR_SHAPE"), (dict(chunk=0), "M3_ERR_SHAPE"),
    (dict(dstate=48), "M3_ERR_UNSUPPORTED"), (dict(headdim=96), "M3_ERR_UNSUPPORTED"),
    (dict(rank=3), "M3_ERR_UNSUPPORTED"), (dict(chunk=128), "M3_ERR_UNSUPPORTED"),
    (dict(io_dtype=7), "M3_ERR_UNSUPPORTED"), (dict(flags=1 << 20), "M3_ERR_UNSUPPORTED"),
    (dict(flags=1 << 18), "M3_ERR_UNSUPPORTED"),
    (dict(flags=0x30000), "M3_ERR_UNSUPPORTED"),                                # both path flags
    (dict(flags=0x20000, seqlen=17), "M3_ERR_UNSUPPORTED"),                     # token path too long
])
def test_chunked_fwd_rejects_bad_sizes(L, kw, expect):
    assert call_fwd(L, dims(L, **kw)) == getattr(L, expect)


def test_chunked_fwd_null_and_alignment(L):
    assert L.lib().mamba3_ssm_chunked_fwd(None, *([None] * 12), None, ctypes.c_size_t(0), None) == L.M3_ERR_NULL
    assert call_fwd(L, dims(L), x=None) == L.M3_ERR_NULL
    assert call_fwd(L, dims(L), theta=None) == L.M3_ERR_NULL
    assert call_fwd(L, dims(L), prev_B=ctypes.c_void_p(FAKE)) == L.M3_ERR_NULL       # prev_x missing
    assert call_fwd(L, dims(L), y=ctypes.c_void_p(FAKE + 8)) == L.M3_ERR_ALIGN
    assert call_fwd(L, dims(L), h0=ctypes.c_void_p(FAKE + 2)) == L.M3_ERR_ALIGN
    assert call_fwd(L, dims(L), dt=ctypes.c_void_p(FAKE + 1)) == L.M3_ERR_ALIGN
    assert call_fwd(L, dims(L), theta=ctypes.c_void_p(FAKE + 4)) == L.M3_ERR_ALIGN   # read in 16-byte vectors


def test_empty_batch_is_a_noop(L):
    # nothing is read or launched for an empty batch, even with null pointers
    d = dims(L, batch=0)
    assert L.lib().mamba3_ssm_chunked_fwd(ctypes.byref(d), *([None] * 12), None, ctypes.c_size_t(0), None) == L.M3_OK


def test_workspace_sizes(L):
    assert L.chunked_fwd_workspace_size(dims(L)) == 0
    # few (b,h) pairs and a long bf16 sequence: walked as segments, workspace needed
    long = dims(L, batch=1, seqlen=65536, nheads=32, dstate=128)
    assert L.chunked_fwd_workspace_size(long) > 0
    assert L.chunked_fwd_workspace_size(dims(L, batch=1, seqlen=65536, nheads=32, dstate=128, flags=1)) == 0
    assert L.chunked_fwd_workspace_size(dims(L, batch=8, seqlen=4096, nheads=64)) == 0
    # segment offsets are kept per requested chunk (the sub-chunk walkers walk
    # shorter pieces): a smaller chunk needs more of them
    few = dict(batch=1, seqlen=8192, nheads=4, dstate=64, headdim=64, rank=4)
    w32, w64 = (L.chunked_fwd_workspace_size(dims(L, chunk=q, **few)) for q in (32, 64))
    assert w32 > w64 > 0
    d = dims(L, seqlen=4096)
    assert L.rope_bc_workspace_size(d) == 4 * 2 * 3 * 64 * 32
    assert L.rope_bc_workspace_size(dims(L, dstate=7)) == 0


BWD_PTRS = ("x", "B", "C", "dt", "A", "lam", "theta", "h0", "prev_B", "prev_x", "dy", "dh_final",
            "dx", "dB", "dC", "ddt", "dA", "dlam", "dtheta", "dh0", "dprev_B", "dprev_x")


def call_bwd(L, d, ws_bytes=None, **over):
    p = {k: ctypes.c_void_p(FAKE) for k in BWD_PTRS}
    p.update(h0=None, prev_B=None, prev_x=None, dh_final=None, dh0=None, dprev_B=None, dprev_x=None, ws=ctypes.c_void_p(FAKE))
    p.update(over)
    need = L.chunked_bwd_workspace_size(d) if ws_bytes is None else ws_bytes
    return L.lib().mamba3_ssm_chunked_bwd(ctypes.byref(d), *(p[k] for k in BWD_PTRS), p["ws"], ctypes.c_size_t(need), None)


def test_backward_validation(L):
    d = dims(L)  # batch 2, L 100, H 3, P 64, N 64, R 4, bf16
    assert L.chunked_bwd_workspace_size(d) == 4 * 6 * ((100 + 15) // 16 + 1) * 64 * 64
    assert call_bwd(L, dims(L, dstate=15)) == L.M3_ERR_SHAPE
    # N = P = 128 at R = 4: 4-token chunks (16 virtual rows), one segment
    assert L.chunked_bwd_workspace_size(dims(L, headdim=128, dstate=128, flags=1)) == 4 * 6 * (25 + 1) * 128 * 128
    long = dims(L, batch=1, seqlen=100, nheads=2, dstate=128, flags=1)             # 8-token chunks at R = 4, one segment
    assert L.chunked_bwd_workspace_size(long) == 4 * 2 * ((100 + 7) // 8 + 1) * 128 * 64
    # segments: 13 chunks of 8 tokens at B*H = 2 -> 3 segments of 5, 5, 3 chunks; checkpoints + four
    # (B*H*S, N, P) state arrays + totals + boundary records, each rounded up to 256 bytes
    up = lambda v: (v + 255) // 256 * 256
    seg = dims(L, batch=1, seqlen=100, nheads=2, dstate=128)
    st = up(4 * 2 * 3 * 128 * 64)
    assert L.chunked_bwd_workspace_size(seg) == up(4 * 2 * 14 * 128 * 64) + 4 * st + up(4 * 2 * 3 * 65) + up(4 * 2 * 3 * 4)
    assert call_bwd(L, dims(L, flags=1 << 16)) == L.M3_ERR_UNSUPPORTED
    assert call_bwd(L, dims(L, batch=1, seqlen=16, nheads=65537)) == L.M3_ERR_UNSUPPORTED  # 32-bit chunk offsets
    assert call_bwd(L, d, dy=None) == L.M3_ERR_NULL
    assert call_bwd(L, d, dtheta=None) == L.M3_ERR_NULL
    assert call_bwd(L, d, prev_B=ctypes.c_void_p(FAKE)) == L.M3_ERR_NULL          # prev_x missing
    assert call_bwd(L, d, dprev_B=ctypes.c_void_p(FAKE)) == L.M3_ERR_NULL         # dprev_x missing
    assert call_bwd(L, d, dx=ctypes.c_void_p(FAKE + 8)) == L.M3_ERR_ALIGN
    assert call_bwd(L, d, dtheta=ctypes.c_void_p(FAKE + 4)) == L.M3_ERR_ALIGN
    assert call_bwd(L, d, ddt=ctypes.c_void_p(FAKE + 2)) == L.M3_ERR_ALIGN
    assert call_bwd(L, d, ws_bytes=1024) == L.M3_ERR_WORKSPACE
    assert call_bwd(L, d, ws=None) == L.M3_ERR_WORKSPACE
    e = dims(L, batch=0)
    assert L.lib().mamba3_ssm_chunked_bwd(ctypes.byref(e), *([None] * 22), None, ctypes.c_size_t(0), None) == L.M3_OK


def call_decode(L, d, **over):
    p = {k: ctypes.c_void_p(FAKE) for k in ("state", "x", "B", "C", "dt", "A", "lam", "theta", "y")}
    p.update(prev_B=None, prev_x=None)
    p.update(over)
    return L.lib().mamba3_ssm_decode_step(ctypes.byref(d), p["state"], p["x"], p["B"], p["C"], p["dt"], p["A"],
                                          p["lam"], p["theta"], p["prev_B"], p["prev_x"], p["y"], None)


def test_decode_validation(L):
    assert call_decode(L, dims(L, dstate=15)) == L.M3_ERR_SHAPE
    assert call_decode(L, dims(L, headdim=100)) == L.M3_ERR_UNSUPPORTED
    assert call_decode(L, dims(L, flags=1)) == L.M3_ERR_UNSUPPORTED
    assert call_decode(L, dims(L), state=None) == L.M3_ERR_NULL
    assert call_decode(L, dims(L), prev_x=ctypes.c_void_p(FAKE)) == L.M3_ERR_NULL
    assert call_decode(L, dims(L), B=ctypes.c_void_p(FAKE + 1)) == L.M3_ERR_ALIGN
    assert call_decode(L, dims(L), state=ctypes.c_void_p(FAKE + 8)) == L.M3_ERR_ALIGN


def test_rope_validation(L):
    lib = L.lib()
    d = dims(L, seqlen=70)
    f = ctypes.c_void_p(FAKE)
    args = lambda **o: [o.get(k, f) for k in ("B", "C", "dt", "theta")] + [None] + [o.get(k, f) for k in ("Br", "Cr")] + [None]
    assert lib.mamba3_rope_bc(ctypes.byref(d), *args(), None, ctypes.c_size_t(0), None) == L.M3_ERR_WORKSPACE
    ws = L.rope_bc_workspace_size(d)
    assert lib.mamba3_rope_bc(ctypes.byref(d), *args(), f, ctypes.c_size_t(ws - 4), None) == L.M3_ERR_WORKSPACE
    assert lib.mamba3_rope_bc(ctypes.byref(d), *args(Br=None), f, ctypes.c_size_t(ws), None) == L.M3_ERR_NULL
    assert lib.mamba3_rope_bc(ctypes.byref(d), *args(dt=ctypes.c_void_p(FAKE + 1)), f, ctypes.c_size_t(ws),
                              None) == L.M3_ERR_ALIGN
    assert lib.mamba3_rope_bc(ctypes.byref(dims(L, rank=8)), *args(), f, ctypes.c_size_t(ws), None) == L.M3_ERR_UNSUPPORTED


PRO_PTRS = ("u", "W", "gain", "bias", "dt", "theta", "angle0", "Br", "Cr", "af")


def call_pro(L, d, D=128, eps=1e-5, ws_bytes=None, **over):
    p = {k: ctypes.c_void_p(FAKE) for k in PRO_PTRS}
    p.update(gain=None, bias=None, angle0=None, af=None, ws=ctypes.c_void_p(FAKE))
    p.update(over)
    need = L.bc_prologue_workspace_size(d) if ws_bytes is None else ws_bytes
    return L.lib().mamba3_bc_prologue(ctypes.byref(d), ctypes.c_int64(D), p["u"], p["W"], p["gain"], p["bias"],
                                      ctypes.c_float(eps), p["dt"], p["theta"], p["angle0"], p["Br"], p["Cr"], p["af"],
                                      p["ws"], ctypes.c_size_t(need), None)


def test_prologue_validation(L):
    d = dims(L, seqlen=70)
    # workspace: the angle chunk totals, then the angles of every token (256-byte aligned)
    tot = (4 * 2 * 3 * 2 * 32 + 255) // 256 * 256
    assert L.bc_prologue_workspace_size(d) == tot + (4 * 2 * 70 * 3 * 32 + 255) // 256 * 256
    assert call_pro(L, d, ws_bytes=0, ws=None) == L.M3_ERR_WORKSPACE
    assert call_pro(L, d, ws_bytes=L.bc_prologue_workspace_size(d) - 4) == L.M3_ERR_WORKSPACE
    assert call_pro(L, d, u=None) == L.M3_ERR_NULL
    assert call_pro(L, d, Cr=None) == L.M3_ERR_NULL
    assert call_pro(L, d, W=ctypes.c_void_p(FAKE + 8)) == L.M3_ERR_ALIGN
    assert call_pro(L, d, gain=ctypes.c_void_p(FAKE + 4)) == L.M3_ERR_ALIGN    # read in 16-byte vectors
    assert call_pro(L, d, dt=ctypes.c_void_p(FAKE + 2)) == L.M3_ERR_ALIGN
    assert call_pro(L, d, D=0) == L.M3_ERR_SHAPE
    assert call_pro(L, d, D=96) == L.M3_ERR_UNSUPPORTED                         # not a multiple of 64
    assert call_pro(L, d, D=(1 << 20) + 64) == L.M3_ERR_UNSUPPORTED
    assert call_pro(L, d, eps=-1.0) == L.M3_ERR_UNSUPPORTED
    assert call_pro(L, d, eps=float("nan")) == L.M3_ERR_UNSUPPORTED
    assert call_pro(L, dims(L, seqlen=70, io_dtype=L.M3_F32)) == L.M3_ERR_UNSUPPORTED
    assert call_pro(L, dims(L, seqlen=70, flags=1)) == L.M3_ERR_UNSUPPORTED
    assert call_pro(L, dims(L, seqlen=70, dstate=48)) == L.M3_ERR_UNSUPPORTED
    # any number of tokens: the product is launched in token slices, so the
    # largest dims the other checks allow pass the size checks (and stop at
    # the missing workspace here, before any launch)
    big = dims(L, batch=65535, seqlen=65535 * 64, nheads=65535, rank=4, dstate=128)  # within the angle pass limits
    assert call_pro(L, big, ws_bytes=0, ws=None) == L.M3_ERR_WORKSPACE
    assert call_pro(L, dims(L, batch=1, seqlen=65535 * 64, nheads=64, rank=4, dstate=64), ws_bytes=0, ws=None) == L.M3_ERR_WORKSPACE
    # an empty batch reads nothing
    assert call_pro(L, dims(L, batch=0), u=None, W=None, dt=None, theta=None, Br=None, Cr=None, ws=None) == L.M3_OK


def test_binding_checks_operand_shapes(L):
    # the C ABI sees raw pointers only; the binding rejects a mis-shaped,
    # mis-typed or misplaced operand before any call (CPU tensors here: the
    # checks come first, nothing is launched)
    import torch
    x = torch.zeros((1, 8, 2, 1, 16))
    B = torch.zeros((1, 8, 2, 1, 16))
    s = torch.zeros((1, 8, 2))
    th = torch.zeros((1, 8, 2, 8))
    with pytest.raises(ValueError):
        L.chunked_fwd(x, B, B, s, s, s, th[..., :4].contiguous())              # theta needs N/2 pairs
    with pytest.raises(TypeError):
        L.chunked_fwd(x, B, B, s.double(), s, s, th)                            # dt must be fp32
    with pytest.raises(TypeError):
        L.chunked_bwd(x, B.bfloat16(), B, s, s, s, th, x)                       # B in x's dtype
    with pytest.raises(ValueError):
        L.chunked_bwd(x, B, B, s, s, s, th, x[:, :4].contiguous())             # dy like x
    with pytest.raises(ValueError):
        L.rope_bc(B, B[:, :4].contiguous(), s, th)                              # C like B
    with pytest.raises(ValueError):
        L.decode_step(torch.zeros((1, 2, 16, 8)), x[:, 0], B[:, 0], B[:, 0], s[:, 0], s[:, 0], s[:, 0], th[:, 0])
    u = torch.zeros((1, 8, 64), dtype=torch.bfloat16)
    W = torch.zeros((64, 64), dtype=torch.bfloat16)                           # 2 H R N = 64 rows for N = 32
    with pytest.raises(ValueError):
        L.bc_prologue(u, W, s, th, 2, 1, 32, gain=torch.zeros((2, 2, 1, 16)))   # gain is (2, H, R, N)
    with pytest.raises(ValueError):
        L.bc_prologue(u, W[:32].contiguous(), s, th, 2, 1, 32)                  # W rows


SUPPORTED = [(io, N, P, R, Q) for io in (0, 1) for N in (16, 32, 64, 128) for P in (16, 32, 64, 128)
             for R in (1, 2, 4) for Q in (16, 32, 64)]


def test_whole_supported_set_is_accepted(L):
    """Every size of the supported set (N, P in {16,32,64,128}, R in {1,2,4},
    Q in {16,32,64}, fp32 or bf16 io: 288 combinations) passes validation of
    the chunked forward and of the backward, and every long-sequence plan
    (few (b,h), segments) too.  An empty batch makes the call return after
    validation, so nothing is launched."""
    lib = L.lib()
    f = ctypes.c_void_p(FAKE)
    assert len(SUPPORTED) == 288
    for io, N, P, R, Q in SUPPORTED:
        for seqlen, nheads in ((100, 3), (65536, 2)):
            d = L.make_dims(0, seqlen, nheads, P, N, R, Q, io)
            st = lib.mamba3_ssm_chunked_fwd(ctypes.byref(d), *([f] * 7), None, None, None, f, None, None,
                                            ctypes.c_size_t(0), None)
            assert st == L.M3_OK, ("fwd", io, N, P, R, Q, L.status_string(st))
            st = lib.mamba3_ssm_chunked_bwd(ctypes.byref(d), *([f] * 7), None, None, None, f, None, *([f] * 7),
                                            None, None, None, None, ctypes.c_size_t(0), None)
            assert st == L.M3_OK, ("bwd", io, N, P, R, Q, L.status_string(st))
            # the workspace the same sizes would need with a non-empty batch
            # is defined (segments for the long bf16 plan, 0 otherwise)
            d1 = L.make_dims(1, seqlen, nheads, P, N, R, Q, io)
            ws = L.chunked_fwd_workspace_size(d1)
            assert ws >= 0 and (ws > 0) == (io == 1 and seqlen == 65536), (io, N, P, R, Q, ws)
            assert L.chunked_bwd_workspace_size(d1) > 0


def test_launch_size_limits(L):
    # one block per (b, h, segment): a launch holds fewer than 2^32 threads, so
    # B*H*S is at most 2^23 - 1 for the forward and the backward (blocks of up
    # to 512 threads) and 2^24 - 1 for the decode step (256 threads); checked
    # before any pointer, so nothing is launched
    over = dict(x=None, y=None)
    assert call_fwd(L, dims(L, batch=65535, nheads=129, seqlen=16), **over) == L.M3_ERR_UNSUPPORTED  # 8.45M > 2^23 - 1
    assert call_fwd(L, dims(L, batch=65535, nheads=128, seqlen=16), **over) == L.M3_ERR_NULL         # 8,388,480: fits
    big_bwd = dims(L, batch=65535, nheads=129, seqlen=16)
    assert call_bwd(L, big_bwd, dx=None) == L.M3_ERR_UNSUPPORTED
    assert call_bwd(L, dims(L, batch=65535, nheads=128, seqlen=16), dx=None, ws=None, ws_bytes=0) != L.M3_ERR_UNSUPPORTED
    # forced segments multiply the blocks: 2^20 (b, h) pairs x 16 segments
    seg_bwd = dims(L, batch=1024, nheads=1024, seqlen=16 * 64, flags=16)
    assert call_bwd(L, seg_bwd, dx=None) == L.M3_ERR_UNSUPPORTED
    assert call_decode(L, dims(L, batch=65535, nheads=257), state=None) == L.M3_ERR_UNSUPPORTED      # 16.8M > 2^24 - 1
    assert call_decode(L, dims(L, batch=65535, nheads=256), state=None) == L.M3_ERR_NULL              # 16,776,960: fits
