"""CPU checks of the C ABI: libmb.so loads, exports every entry point that
include/mb.h declares, and rejects invalid arguments on the host before anything
is enqueued (no GPU needed: every call here fails validation or is a no-op)."""
import ctypes
import os
import re

import pytest

import selective_state_space_amd as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mb.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_WS, E_HIP, E_ALIAS, E_ALIGN = range(8)
FAKE = 0x10000000          # never dereferenced: validation fails before any access
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mb.lib_path()):
        from selective_state_space_amd import _build
        _build.build()
    return mb.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mb_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"mb_selective_scan", "mb_ssm_step", "mb_ssd_chunked", "mb_trap_ssd", "mb_trap_ssd_gated", "mb_trap_ssd_block", "mb_ssd_prologue", "mb_mimo_ssd",
            "mb_ssd_step", "mb_selective_scan_fused", "mb_ssd_chunked_bwd", "mb_selective_scan_bwd", "mb_trap_ssd_bwd", "mb_mimo_ssd_bwd", "mb_workspace_size", "mb_status_str", "mb_last_hip_error", "mb_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "libmb.so does not export " + n


def test_status_strings(lib):
    for s in range(8):
        assert mb.mb_status_str(s)
    assert mb.mb_status_str(99) == "unknown status"
    assert lib.mb_version() >= 100
    assert lib.mb_last_hip_error() == 0


def P(x=FAKE):
    return ctypes.c_void_p(x)


def scan(lib, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, h0=None, y=FAKE + (1 << 24),
         h_out=FAKE + (1 << 25), batch=2, L=8, Dm=16, N=16, dtype=F32, ws=None, ws_bytes=0):
    return lib.mb_selective_scan(P(x) if x else None, P(dt) if dt else None, P(A) if A else None,
                                 P(B) if B else None, P(C) if C else None, P(D) if D else None,
                                 P(h0) if h0 else None, P(y) if y else None,
                                 P(h_out) if h_out else None, batch, L, Dm, N, dtype, P(ws) if ws else None,
                                 ws_bytes, None)


def test_scan_validation(lib):
    base = dict(x=FAKE, dt=FAKE + 4096, A=FAKE + 8192, B=FAKE + 12288, C=FAKE + 16384)
    assert scan(lib, **base, dtype=7) == E_DTYPE
    assert scan(lib, **base, N=0) == E_SHAPE
    assert scan(lib, **base, N=65) == E_SHAPE
    assert scan(lib, **base, L=-1) == E_SHAPE
    assert scan(lib, **dict(base, x=0)) == E_NULL
    assert scan(lib, **dict(base, C=0)) == E_NULL
    # y overlapping x
    assert scan(lib, **base, y=FAKE + 16) == E_ALIAS
    # h_out overlapping B
    assert scan(lib, **base, h_out=FAKE + 12288) == E_ALIAS
    # empty batch is a no-op that succeeds without touching the device
    assert scan(lib, **base, batch=0) == OK
    # one batch row must be addressable in 32-bit byte offsets, tile padding included
    L_max = (1 << 31) // (4 * 512) - 64        # (L + 64) * D * 4 == 2^31 at D = 512
    assert scan(lib, **base, L=L_max, Dm=512) == E_SHAPE
    assert scan(lib, **dict(base, x=0), L=L_max - 1, Dm=512) == E_NULL


def test_scan_workspace(lib):
    """Sequence blocks: the workspace is optional; when given it must hold the
    planned size, be 256-byte aligned and overlap nothing (checked before any
    launch: the pointers are never dereferenced)."""
    ws_size = lib.mb_workspace_size
    b, L, Dm, N = 1, 4096, 64, 16          # one channel group: the planner cuts the sequence
    need = ws_size(0, b, L, Dm, 1, 1, N, 1, 0)
    assert need > 0 and need % 256 == 0
    assert ws_size(0, 64, 64, 1536, 1, 1, 16, 1, 0) == 0     # enough parallel work: one block
    assert ws_size(0, b, L, Dm, 1, 1, 64, 1, 0) == 0         # N = 64: one block
    span = b * L * Dm * 4
    base = dict(x=FAKE, dt=FAKE + span, A=FAKE + 2 * span, B=FAKE + 3 * span, C=FAKE + 4 * span,
                y=FAKE + 5 * span, h_out=FAKE + 6 * span, batch=b, L=L, Dm=Dm, N=N)
    W = FAKE + 8 * span
    assert scan(lib, **base, ws=W, ws_bytes=need - 1) == E_WS
    assert scan(lib, **base, ws=W + 16, ws_bytes=need) == E_WS           # not 256-byte aligned
    assert scan(lib, **base, ws=FAKE + span, ws_bytes=need) == E_ALIAS   # over dt
    assert scan(lib, **dict(base, x=0), ws=W, ws_bytes=need) == E_NULL


def step(lib, h_in=FAKE + (1 << 26), h_out=FAKE + (1 << 26), y=FAKE + (1 << 27), **kw):
    args = dict(x=FAKE, dt=FAKE + 4096, A=FAKE + 8192, B=FAKE + 12288, C=FAKE + 16384)
    args.update(kw)
    b, Dm, N = 4, 16, 16
    return lib.mb_ssm_step(P(args["x"]), P(args["dt"]), P(args["A"]), P(args["B"]), P(args["C"]),
                           None, P(h_in), P(h_out), P(y), b, Dm, N, args.get("dtype", F32), None)


def test_step_validation(lib):
    assert step(lib, dtype=3) == E_DTYPE
    # partial overlap between h_out and h_in is rejected (exact aliasing is allowed)
    assert step(lib, h_out=FAKE + (1 << 26) + 64) == E_ALIAS
    assert step(lib, y=FAKE + 8) == E_ALIAS


def fused(lib, x=FAKE, dt=FAKE + (1 << 22), z=None, y=FAKE + (1 << 24), h_out=FAKE + (1 << 25), conv_w=FAKE + (1 << 26),
          N=16, K=4, dtype=F32, batch=2):
    q = lambda v: P(v) if v else None
    return lib.mb_selective_scan_fused(q(x), q(conv_w), None, None, q(dt), None, P(FAKE + (1 << 23)),
                                       P(FAKE + (1 << 23) + (1 << 20)), P(FAKE + (1 << 23) + (1 << 21)), None,
                                       q(z), None, q(y), q(h_out), batch, 8, 16, N, K, dtype, None)


def test_fused_scan_validation(lib):
    assert fused(lib, dtype=BF16) == E_DTYPE
    assert fused(lib, N=32) == E_SHAPE
    assert fused(lib, K=5) == E_SHAPE
    assert fused(lib, K=0) == E_SHAPE
    assert fused(lib, conv_w=0) == E_NULL
    assert fused(lib, x=FAKE + 4) == E_ALIGN
    assert fused(lib, z=FAKE + (1 << 27) + 8) == E_ALIGN
    assert fused(lib, y=FAKE + 64) == E_ALIAS          # y over x
    assert fused(lib, z=FAKE + (1 << 24)) == E_ALIAS   # y over z
    assert fused(lib, batch=0) == OK


def ssd_step(lib, X=FAKE, B=FAKE + (1 << 22), Bp=None, Xp=None, h_in=FAKE + (1 << 26), h_out=FAKE + (1 << 26),
             Y=FAKE + (1 << 27), theta=None, batch=2, H=4, P_=64, G=1, N=128, R=1, dtype=F32):
    q = lambda v: P(v) if v else None
    return lib.mb_ssd_step(q(X), P(FAKE + (1 << 21)), q(B), P(FAKE + (1 << 23)), None, None, q(theta), q(Xp), q(Bp),
                           q(h_in), q(h_out), q(Y), batch, H, P_, G, N, R, dtype, None)


def test_ssd_step_validation(lib):
    assert ssd_step(lib, dtype=2) == E_DTYPE
    assert ssd_step(lib, G=3) == E_SHAPE            # H % G != 0
    assert ssd_step(lib, N=7) == E_SHAPE            # odd N
    assert ssd_step(lib, P_=6) == E_SHAPE           # P % 4 != 0
    assert ssd_step(lib, P_=1028) == E_SHAPE        # P > 1024
    assert ssd_step(lib, R=3) == E_SHAPE
    assert ssd_step(lib, X=0) == E_NULL
    assert ssd_step(lib, Y=0) == E_NULL
    assert ssd_step(lib, Bp=FAKE + (1 << 24)) == E_NULL   # B_prev without X_prev
    assert ssd_step(lib, h_out=FAKE + (1 << 26) + 8) == E_ALIGN
    assert ssd_step(lib, X=FAKE + 4) == E_ALIGN
    assert ssd_step(lib, B=FAKE + (1 << 22) + 8) == E_ALIGN
    assert ssd_step(lib, h_out=FAKE + (1 << 26) + 256) == E_ALIAS   # partial overlap with h_in
    assert ssd_step(lib, Y=FAKE + 64) == E_ALIAS      # Y over X
    assert ssd_step(lib, h_in=None, h_out=FAKE + (1 << 22)) == E_ALIAS   # h_out over B
    assert ssd_step(lib, batch=0) == OK


def ssd(lib, ws=FAKE + (1 << 28), ws_bytes=1 << 30, H=4, P_=64, G=1, N=128, L=100, chunk=0,
        dtype=F32, Y=FAKE + (1 << 27), batch=2):
    return lib.mb_ssd_chunked(P(FAKE), P(FAKE + (1 << 22)), P(FAKE + (1 << 23)), P(FAKE + (1 << 24)),
                              None, P(Y), P(FAKE + (1 << 26)), batch, L, H, P_, G, N, chunk, dtype,
                              P(ws) if ws else None, ws_bytes, None)


def test_ssd_validation(lib):
    assert ssd(lib, dtype=2) == E_DTYPE
    assert ssd(lib, G=3) == E_SHAPE            # H % G != 0
    assert ssd(lib, N=130) == E_SHAPE
    assert ssd(lib, N=0) == E_SHAPE
    assert ssd(lib, P_=0) == E_SHAPE
    # P % 16 != 0 or N % 4 != 0 run through padded copies: they pass the shape
    # checks and then need the larger workspace
    assert ssd(lib, N=6, ws_bytes=16) == E_WS
    assert ssd(lib, P_=40, ws_bytes=16) == E_WS
    assert ssd(lib, P_=1, N=2, ws_bytes=16) == E_WS
    assert ssd(lib, chunk=32) == E_SHAPE
    assert ssd(lib, ws=0) == E_WS
    assert ssd(lib, ws_bytes=16) == E_WS
    assert ssd(lib, ws=FAKE + (1 << 28) + 4) == E_WS   # misaligned
    assert ssd(lib, Y=FAKE + 64) == E_ALIAS
    assert ssd(lib, Y=FAKE + (1 << 27) + 8) == E_ALIGN
    assert ssd(lib, batch=0) == OK
    # one batch row of the score workspace (64 x 64 fp32 per chunk and group)
    # must be addressable in 32-bit byte offsets: 64 chunks x 4096 groups is 2^32 bytes
    assert ssd(lib, L=4096, H=4096, G=4096, P_=16, N=16) == E_SHAPE
    ws_size = lib.mb_workspace_size
    ws_size.restype = ctypes.c_size_t
    assert ws_size(2, 1, 4096, 4096, 16, 4096, 16, 1, 0) == 0
    assert ws_size(2, 1, 1984, 4096, 16, 4096, 16, 1, 0) > 0     # 31 chunks: below 2^31 bytes


def ssd_bwd(lib, X=FAKE, dY=FAKE + (1 << 24), dX=FAKE + (1 << 25), dB=FAKE + (1 << 26), dh0=FAKE + (1 << 27),
            ws=FAKE + (1 << 28), ws_bytes=1 << 30, H=4, P_=64, G=1, N=128, L=100, batch=2, dtype=F32):
    q = lambda v: P(v) if v else None
    return lib.mb_ssd_chunked_bwd(q(X), P(FAKE + (1 << 22)), P(FAKE + (1 << 23)), P(FAKE + (1 << 23) + (1 << 21)),
                                  None, q(dY), None, q(dX), P(FAKE + (1 << 25) + (1 << 21)), q(dB),
                                  P(FAKE + (1 << 26) + (1 << 21)), q(dh0), batch, L, H, P_, G, N, dtype, q(ws),
                                  ws_bytes, None)


def test_ssd_bwd_validation(lib):
    assert ssd_bwd(lib, dtype=BF16) == E_DTYPE
    assert ssd_bwd(lib, N=32) == E_SHAPE
    assert ssd_bwd(lib, P_=48) == E_SHAPE
    assert ssd_bwd(lib, G=3) == E_SHAPE
    assert ssd_bwd(lib, X=0) == E_NULL
    assert ssd_bwd(lib, dB=0) == E_NULL
    assert ssd_bwd(lib, dX=FAKE + (1 << 25) + 4) == E_ALIGN
    assert ssd_bwd(lib, dh0=FAKE + (1 << 27) + 8) == E_ALIGN
    assert ssd_bwd(lib, dX=FAKE + 256) == E_ALIAS          # dX over X
    assert ssd_bwd(lib, dB=FAKE + (1 << 25) + 1024) == E_ALIAS   # dB over dX
    assert ssd_bwd(lib, dh0=FAKE + (1 << 28)) == E_ALIAS   # dh0 over the workspace
    assert ssd_bwd(lib, ws=0) == E_WS
    assert ssd_bwd(lib, ws_bytes=4096) == E_WS
    assert ssd_bwd(lib, ws=FAKE + (1 << 28) + 16) == E_WS
    assert ssd_bwd(lib, batch=0) == OK
    need = mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED_BWD, 2, 100, 4, 64, 1, 128)
    assert need >= 2 * 4 * 2 * 2 * 128 * 64 * 4
    assert mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED_BWD, 2, 100, 4, 48, 1, 128) == 0
    assert mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED_BWD, 2, 0, 4, 64, 1, 128) == 0


def m1_bwd(lib, x=FAKE, dy=FAKE + (1 << 24), dx=FAKE + (1 << 25), dB=FAKE + (1 << 26), dh0=None,
           ws=FAKE + (1 << 28), ws_bytes=1 << 30, L=100, Dm=64, N=16, batch=2, dtype=F32):
    q = lambda v: P(v) if v else None
    return lib.mb_selective_scan_bwd(q(x), P(FAKE + (1 << 22)), P(FAKE + (1 << 23)), P(FAKE + (1 << 23) + (1 << 20)),
                                     P(FAKE + (1 << 23) + (1 << 21)), None, None, q(dy), None, q(dx),
                                     P(FAKE + (1 << 25) + (1 << 21)), P(FAKE + (1 << 27)), q(dB),
                                     P(FAKE + (1 << 26) + (1 << 21)), None, q(dh0), batch, L, Dm, N, dtype, q(ws),
                                     ws_bytes, None)


def test_m1_bwd_validation(lib):
    assert m1_bwd(lib, dtype=BF16) == E_DTYPE
    assert m1_bwd(lib, N=32) == E_SHAPE
    assert m1_bwd(lib, N=6) == E_SHAPE
    assert m1_bwd(lib, x=0) == E_NULL
    assert m1_bwd(lib, dB=0) == E_NULL
    assert m1_bwd(lib, dy=FAKE + (1 << 24) + 4) == E_ALIGN
    assert m1_bwd(lib, dx=FAKE + 64) == E_ALIAS                       # dx over x
    assert m1_bwd(lib, dh0=FAKE + (1 << 25) + 512) == E_ALIAS          # dh0 over dx
    assert m1_bwd(lib, ws=0) == E_WS
    assert m1_bwd(lib, ws_bytes=4096) == E_WS
    assert m1_bwd(lib, ws=FAKE + (1 << 28) + 64) == E_WS
    need = mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN_BWD, 2, 100, 64, 1, 1, 16)
    assert need >= 2 * 4 * 64 * 16 * 4
    assert mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN_BWD, 2, 100, 64, 1, 1, 32) == 0


def trap_bwd(lib, X=FAKE, dX=FAKE + (1 << 25), theta=FAKE + (1 << 24) + (1 << 22), dtheta=FAKE + (1 << 27),
             Xp=None, Bp=None, N=128, P_=64, G=1, dtype=F32, ws=FAKE + (1 << 28), ws_bytes=1 << 33):
    q = lambda v: P(v) if v else None
    return lib.mb_trap_ssd_bwd(q(X), P(FAKE + (1 << 22)), P(FAKE + (1 << 23)), P(FAKE + (1 << 23) + (1 << 21)),
                               P(FAKE + (1 << 22) + (1 << 20)), P(FAKE + (1 << 22) + (1 << 21)), q(theta), None,
                               q(Xp), q(Bp), P(FAKE + (1 << 24)), None, q(dX), P(FAKE + (1 << 25) + (1 << 23)),
                               P(FAKE + (1 << 26)), P(FAKE + (1 << 26) + (1 << 21)), P(FAKE + (1 << 26) + (1 << 22)),
                               P(FAKE + (1 << 26) + (1 << 23)), q(dtheta), None, None, None, 2, 50, 4, P_, G, N,
                               dtype, q(ws), ws_bytes, None)


def test_trap_bwd_validation(lib):
    assert trap_bwd(lib, dtype=BF16) == E_DTYPE
    assert trap_bwd(lib, N=32) == E_SHAPE
    assert trap_bwd(lib, P_=16) == E_SHAPE
    assert trap_bwd(lib, G=3) == E_SHAPE
    assert trap_bwd(lib, X=0) == E_NULL
    assert trap_bwd(lib, dtheta=0) == E_NULL                      # theta given, dtheta missing
    assert trap_bwd(lib, Xp=FAKE + (1 << 29)) == E_NULL             # X_prev without B_prev
    assert trap_bwd(lib, dX=FAKE + (1 << 25) + 4) == E_ALIGN
    assert trap_bwd(lib, dX=FAKE + 128) == E_ALIAS                  # dX over X
    assert trap_bwd(lib, ws=0) == E_WS
    assert trap_bwd(lib, ws_bytes=1 << 12) == E_WS
    assert mb.mb_workspace_size(mb.MB_OP_TRAP_SSD_BWD, 2, 50, 4, 64, 1, 128) > 0
    assert mb.mb_workspace_size(mb.MB_OP_TRAP_SSD_BWD, 2, 50, 4, 48, 1, 128) == 0


def test_mimo_bwd_validation(lib):
    def call(N=128, P_=64, R=4, dtype=F32, X=FAKE, dX=FAKE + (1 << 25), dh0=None, ws=FAKE + (1 << 28)):
        q = lambda v: P(v) if v else None
        return lib.mb_mimo_ssd_bwd(q(X), P(FAKE + (1 << 22)), P(FAKE + (1 << 23)), P(FAKE + (1 << 23) + (1 << 21)),
                                   P(FAKE + (1 << 22) + (1 << 20)), P(FAKE + (1 << 22) + (1 << 21)), None, None,
                                   None, None, P(FAKE + (1 << 24)), None, q(dX), P(FAKE + (1 << 25) + (1 << 23)),
                                   P(FAKE + (1 << 26)), P(FAKE + (1 << 26) + (1 << 22)), P(FAKE + (1 << 27)),
                                   P(FAKE + (1 << 27) + (1 << 20)), None, q(dh0), None, None, 1, 20, 2, P_, N, R,
                                   dtype, q(ws), 1 << 33, None)
    assert call(dtype=BF16) == E_DTYPE
    assert call(N=96) == E_SHAPE
    assert call(R=17) == E_SHAPE
    assert call(R=3) == E_SHAPE
    assert call(X=0) == E_NULL
    assert call(dh0=FAKE + (1 << 29) + 4) == E_ALIGN
    assert call(dX=FAKE + 64) == E_ALIAS
    assert call(ws=0) == E_WS
    assert mb.mb_workspace_size(mb.MB_OP_MIMO_SSD_BWD, 1, 20, 2, 64, 1, 128, 4) > 0
    assert mb.mb_workspace_size(mb.MB_OP_MIMO_SSD_BWD, 1, 20, 2, 64, 1, 128, 0) == 0


def test_trap_and_mimo_validation(lib):
    args = [P(FAKE), P(FAKE + (1 << 22)), P(FAKE + (1 << 23)), P(FAKE + (1 << 24)),
            P(FAKE + (1 << 25)), P(FAKE + (1 << 25) + (1 << 21)), P(FAKE + (1 << 29)), None, None, None,
            P(FAKE + (1 << 27)), P(FAKE + (1 << 26))]
    # odd N with rotation angles
    assert lib.mb_trap_ssd(*args, 1, 10, 2, 16, 1, 6, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == E_SHAPE
    # beta missing
    a2 = list(args)
    a2[4] = None
    assert lib.mb_trap_ssd(*a2, 1, 10, 2, 16, 1, 8, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == E_NULL
    # the previous token: X_prev and B_prev together, 16-byte aligned, not under an output
    a3 = list(args)
    a3[8] = P(FAKE + (1 << 30))
    assert lib.mb_trap_ssd(*a3, 1, 10, 2, 16, 1, 8, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == E_NULL
    a3[9] = P(FAKE + (1 << 30) + (1 << 20) + 4)
    assert lib.mb_trap_ssd(*a3, 1, 10, 2, 16, 1, 8, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == E_ALIGN
    a3[9] = P(FAKE + (1 << 27))    # under Y
    assert lib.mb_trap_ssd(*a3, 1, 10, 2, 16, 1, 8, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == E_ALIAS
    # the output epilogue: z 16-byte aligned, D 4-byte aligned, neither under an output
    ws = (P(FAKE + (1 << 28)), 1 << 30, None)
    dims = (1, 10, 2, 16, 1, 8, 0, F32)
    assert lib.mb_trap_ssd_gated(*args[:10], None, P(FAKE + (1 << 31) + 8), *args[10:], *dims, *ws) == E_ALIGN
    assert lib.mb_trap_ssd_gated(*args[:10], P(FAKE + (1 << 31) + 2), None, *args[10:], *dims, *ws) == E_ALIGN
    assert lib.mb_trap_ssd_gated(*args[:10], None, P(FAKE + (1 << 27) + 64), *args[10:], *dims, *ws) == E_ALIAS
    assert lib.mb_trap_ssd_gated(*args[:10], P(FAKE + (1 << 26) + 4), None, *args[10:], *dims, *ws) == E_ALIAS
    assert lib.mb_trap_ssd_gated(*args[:10], P(FAKE + (1 << 31)), P(FAKE + (1 << 31) + 256), *args[10:],
                                 0, *dims[1:], *ws) == OK
    assert lib.mb_trap_ssd_gated(*args[:10], None, None, *args[10:], 1, 10, 2, 16, 1, 6, 0, F32, *ws) == E_SHAPE
    # the block: eps > 0; parameter arrays 4-byte aligned and not under an output
    par = P(FAKE + (1 << 31))
    blk = lambda nb, nc, bb, bc, eps, d, z, *rest: lib.mb_trap_ssd_block(
        *args[:10], nb, nc, bb, bc, eps, d, z, *args[10:], *rest)
    assert blk(par, par, None, None, 0.0, None, None, *dims, *ws) == E_SHAPE
    assert blk(par, par, None, None, float("nan"), None, None, *dims, *ws) == E_SHAPE
    assert blk(P(FAKE + (1 << 31) + 2), None, None, None, 1e-5, None, None, *dims, *ws) == E_ALIGN
    assert blk(None, None, P(FAKE + (1 << 27) + 8), None, 1e-5, None, None, *dims, *ws) == E_ALIAS
    assert blk(None, None, None, P(FAKE + (1 << 26)), 1e-5, None, None, *dims, *ws) == E_ALIAS
    assert blk(par, par, par, par, 1e-5, par, P(FAKE + (1 << 31) + 4096), 0, *dims[1:], *ws) == OK
    # unsupported rank
    assert lib.mb_mimo_ssd(*args, 1, 10, 2, 16, 8, 3, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == E_SHAPE
    assert lib.mb_mimo_ssd(*args, 0, 10, 2, 16, 8, 4, 0, F32, P(FAKE + (1 << 28)), 1 << 30, None) == OK
    # the MIMO block takes every rank the plain MIMO scan takes
    mblk = lambda R, batch: lib.mb_mimo_ssd_block(*args[:10], None, None, None, None, 1e-5, None, None,
                                                  *args[10:], batch, 10, 2, 16, 8, R, 0, F32,
                                                  P(FAKE + (1 << 28)), 1 << 30, None)
    for R in (1, 2, 4, 8, 16):
        assert mblk(R, 0) == OK
    for R in (3, 32):
        assert mblk(R, 1) == E_SHAPE


def _a256(v):
    return (v + 255) // 256 * 256


def _plan(batch, L, H, P, R):
    """Chunks and sequence segments as the library chooses them: 64 rows per
    chunk; the segment count minimises (full-pass rounds + 0.45 state-only
    rounds) x (chunks per segment + 2) on 256 compute units, with at least 4
    chunks per segment and at most 64 segments."""
    nch = -(-L // (64 // R))
    units = batch * H * (-(-P // 64))
    best, best_cost = 1, None
    for ns in range(1, 65):
        if ns > 1 and nch // ns < 4:
            break
        cps = -(-nch // ns)
        nse = -(-nch // cps)
        cost = (-(-(nse * units) // 256) + 0.45 * (-(-((nse - 1) * units) // 512))) * (cps + 2)
        if best_cost is None or cost < best_cost - 1e-9:
            best, best_cost = ns, cost
    cps = -(-nch // best)
    return nch, -(-nch // cps)


def _ws(op, batch, L, H, P, G, N, R=1):
    nch, nseg = _plan(batch, L, H, P, R if op == mb.MB_OP_MIMO_SSD else 1)
    trap = op != mb.MB_OP_SSD_CHUNKED
    total = 0 if trap else _a256(batch * nch * G * 64 * 64 * 4)     # Mamba-2 scores
    if not trap:                                                    # Mamba-2 B^T (bf16)
        total += _a256(batch * nch * G * (64 if N <= 64 else 128) * 64 * 2)
    nsg = batch * H * (nseg - 1)
    total += _a256(nsg * N * P * 4) + _a256(nsg * 4)                  # segment states, decays
    if trap:
        total += _a256(nsg * (N // 2) * 4)                            # segment angles
    return total if (nseg > 1 or not trap) else 0


def test_workspace_sizes(lib):
    # Mamba-1 block workload (batch 8, L 2048, D 1536, N 16): 192 workgroups of 64
    # channels fill three quarters of the SIMDs (256 compute units without a
    # device), so one sequence block and no workspace; batch 1 at L 16384 has 24
    # workgroups and runs in 32 blocks: a state and a step-size sum per (batch,
    # block, channel)
    assert mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN, 8, 2048, 1536, 1, 1, 16) == 0
    assert mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN, 1, 16384, 1536, 1, 1, 16) == \
        32 * 1536 * 16 * 4 + 32 * 1536 * 4
    # Mamba-2 block workload: 5 segments of 13 chunks; scores 4 MiB + B^T 4 MiB + 4
    # segment states
    assert mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, 4, 4096, 24, 64, 1, 128) == \
        4 * 64 * 64 * 64 * 4 + 4 * 64 * 128 * 64 * 2 + 4 * 24 * 4 * 128 * 64 * 4 + 1536
    for args in [(mb.MB_OP_SSD_CHUNKED, 4, 4096, 24, 64, 1, 128), (mb.MB_OP_TRAP_SSD, 4, 4096, 24, 64, 1, 128),
                 (mb.MB_OP_SSD_CHUNKED, 2, 333, 3, 48, 1, 64), (mb.MB_OP_TRAP_SSD, 1, 2000, 2, 16, 1, 32),
                 (mb.MB_OP_TRAP_SSD, 2, 130, 4, 16, 2, 128)]:
        assert mb.mb_workspace_size(*args) == _ws(*args), args
    for R in (1, 2, 4, 8, 16):
        args = (mb.MB_OP_MIMO_SSD, 2, 8192, 16, 64, 1, 128, R)
        assert mb.mb_workspace_size(*args) == _ws(*args), args
    # padded shapes: the plan at P' = 48, N' = 8, then X, Y, z (P' columns), B, C
    # (N' states) and one N' x P' state per (batch, head)
    a = _a256
    assert mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, 2, 100, 4, 40, 1, 6) == \
        _ws(mb.MB_OP_SSD_CHUNKED, 2, 100, 4, 48, 1, 8) + 3 * a(2 * 100 * 4 * 48 * 4) + \
        2 * a(2 * 100 * 1 * 8 * 4) + a(2 * 4 * 8 * 48 * 4)
    assert mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, 1, 50, 3, 1, 1, 2) == \
        _ws(mb.MB_OP_SSD_CHUNKED, 1, 50, 3, 16, 1, 4) + 3 * a(50 * 3 * 16 * 4) + 2 * a(50 * 4 * 4) + \
        a(3 * 4 * 16 * 4)
    # short sequences need no segments; the trapezoid then needs no workspace
    assert mb.mb_workspace_size(mb.MB_OP_TRAP_SSD, 1, 100, 2, 16, 1, 16) == 0
    assert mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, 4, 4096, 24, 64, 5, 128) == 0   # invalid G
    assert mb.mb_workspace_size(mb.MB_OP_MIMO_SSD, 2, 8192, 16, 64, 1, 128, 3) == 0   # invalid R


def test_ssd_prologue_validation(lib):
    q = [P(FAKE + (k << 24)) for k in range(12)]     # xBC, conv_w, conv_b, x_hist, dt, dt_bias, A, X, B, C, ld, dt'
    dims = (1, 10, 2, 16, 1, 8, 4)
    a = list(q)
    a[0] = None
    assert lib.mb_ssd_prologue(*a, *dims, F32, None) == E_NULL
    assert lib.mb_ssd_prologue(*q, 1, 10, 2, 16, 1, 8, 5, F32, None) == E_SHAPE        # K > 4
    assert lib.mb_ssd_prologue(*q, 1, 10, 3, 16, 2, 8, 4, F32, None) == E_SHAPE        # H % G
    assert lib.mb_ssd_prologue(*q, 1, 16 * 65536, 2, 16, 1, 8, 4, F32, None) == E_SHAPE
    a = list(q)
    a[8] = P(FAKE + (8 << 24) + 4)
    assert lib.mb_ssd_prologue(*a, *dims, F32, None) == E_ALIGN
    a = list(q)
    a[9] = P(FAKE + (8 << 24) + 16)                  # C over B
    assert lib.mb_ssd_prologue(*a, *dims, F32, None) == E_ALIAS
    a = list(q)
    a[7] = P(FAKE + 64)                              # X over xBC
    assert lib.mb_ssd_prologue(*a, *dims, F32, None) == E_ALIAS
    assert lib.mb_ssd_prologue(*q, *dims, 7, None) == E_DTYPE
    assert lib.mb_ssd_prologue(*q, 0, *dims[1:], F32, None) == OK
