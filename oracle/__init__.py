"""fp64 CPU oracle for the selective state-space scans.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``selective_state_space_amd``: the loops live in
``oracle.c`` (plain C, fp64, OpenMP over independent units) and this module only
converts numpy arrays to contiguous float64 and calls them through ctypes.

Each function returns ``(y, h_out)`` as float64 numpy arrays.  Inputs are taken
exactly as given (a bf16 input is expected already rounded to bf16 and then
widened, so that the oracle sees the values the GPU sees).

Which passage each loop follows is cited at the loop in ``oracle.c``:
  m1_scan / m1_step  - TorchMamba README (Models table, Math notes M1);
                       burn_mamba Mamba1 docs (selective_scan, selective_scan_step)
  m1_block           - the same scan with the block's causal conv1d + SiLU,
                       softplus(dt + bias) and SiLU(z) gate around it
  ssd                - TorchMamba README (Models table, Math notes M2)
  trap               - TorchMamba README (Math notes M3 SISO);
                       mamba3-minimal README (Two-SSD Decomposition)
  mimo               - TorchMamba README (Math notes MIMO)
  ssd_step           - the same recurrences one token at a time, state in the
                       physical frame (Math notes M2, M3 SISO, MIMO)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    with _lock:
        if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
        ):
            tmp = _LIB_PATH + ".tmp%d" % os.getpid()
            subprocess.check_call(
                ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                 "-Wall", "-o", tmp, _SRC, "-lm"]
            )
            os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_m1_scan.argtypes = [_D] * 9 + [_I] * 4
        lib.oracle_m1_step.argtypes = [_D] * 9 + [_I] * 3
        lib.oracle_m1_scan_bwd.argtypes = [_D] * 16 + [_I] * 4
        lib.oracle_ssd.argtypes = [_D] * 7 + [_I] * 6
        lib.oracle_ssd_bwd.argtypes = [_D] * 12 + [_I] * 6
        lib.oracle_trap.argtypes = [_D] * 12 + [_I] * 6
        lib.oracle_trap_bwd.argtypes = [_D] * 22 + [_I] * 6
        lib.oracle_mimo_bwd.argtypes = [_D] * 22 + [_I] * 6
        lib.oracle_mimo.argtypes = [_D] * 12 + [_I] * 6
        lib.oracle_ssd_step.argtypes = [_D] * 12 + [_I] * 6
        lib.oracle_m1_block.argtypes = [_D] * 14 + [_I] * 5
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_get_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


def _opt(a, shape):
    if a is None:
        return None
    a = _f64(a)
    if a.shape != tuple(shape):
        raise ValueError("shape %s, expected %s" % (a.shape, tuple(shape)))
    return a


def _chk(a, shape, name):
    a = _f64(a)
    if a.shape != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, a.shape, tuple(shape)))
    return a


def m1_scan(x, dt, A, B, C, D=None, h0=None):
    """Mamba-1 selective scan.  x, dt (b, L, D); A (D, N); B, C (b, L, N)."""
    x = _f64(x)
    b, L, Dm = x.shape
    A = _f64(A)
    N = A.shape[1]
    dt = _chk(dt, (b, L, Dm), "dt")
    A = _chk(A, (Dm, N), "A")
    B = _chk(B, (b, L, N), "B")
    C = _chk(C, (b, L, N), "C")
    D = _opt(D, (Dm,))
    h0 = _opt(h0, (b, Dm, N))
    y = np.empty((b, L, Dm))
    h = np.empty((b, Dm, N))
    _load().oracle_m1_scan(_p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(h0),
                           _p(y), _p(h), b, L, Dm, N)
    return y, h


def m1_scan_bwd(x, dt, A, B, C, dy, D=None, h0=None, dh_out=None):
    """Backward of the Mamba-1 scan: the gradients of sum dy . y + sum dh_out .
    h_out with respect to x, dt, A, B, C, D and h0.  Shapes as m1_scan(); dy
    like x, dh_out like h0.  Returns (dx, ddt, dA, dB, dC, dD, dh0)."""
    x = _f64(x)
    b, L, Dm = x.shape
    A = _f64(A)
    N = A.shape[1]
    dt = _chk(dt, (b, L, Dm), "dt")
    A = _chk(A, (Dm, N), "A")
    B = _chk(B, (b, L, N), "B")
    C = _chk(C, (b, L, N), "C")
    dy = _chk(dy, (b, L, Dm), "dy")
    D = _opt(D, (Dm,))
    h0 = _opt(h0, (b, Dm, N))
    dh_out = _opt(dh_out, (b, Dm, N))
    dx, ddt = np.empty((b, L, Dm)), np.empty((b, L, Dm))
    dA = np.empty((Dm, N))
    dB, dC = np.empty((b, L, N)), np.empty((b, L, N))
    dD = np.empty(Dm)
    dh0 = np.empty((b, Dm, N))
    _load().oracle_m1_scan_bwd(_p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(h0), _p(dy), _p(dh_out), _p(dx),
                               _p(ddt), _p(dA), _p(dB), _p(dC), _p(dD), _p(dh0), b, L, Dm, N)
    return dx, ddt, dA, dB, dC, dD, dh0


def m1_step(x, dt, A, B, C, D, h):
    """One Mamba-1 step.  x, dt (b, D); B, C (b, N); h (b, D, N)."""
    x = _f64(x)
    b, Dm = x.shape
    A = _f64(A)
    N = A.shape[1]
    dt = _chk(dt, (b, Dm), "dt")
    B = _chk(B, (b, N), "B")
    C = _chk(C, (b, N), "C")
    D = _opt(D, (Dm,))
    h = _chk(h, (b, Dm, N), "h")
    y = np.empty((b, Dm))
    h_out = np.empty((b, Dm, N))
    _load().oracle_m1_step(_p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(h),
                           _p(h_out), _p(y), b, Dm, N)
    return y, h_out


def ssd(X, logdecay, B, C, h0=None):
    """Mamba-2 SSD.  X (b, L, H, P); logdecay (b, L, H); B, C (b, L, G, N)."""
    X = _f64(X)
    b, L, H, P = X.shape
    B = _f64(B)
    G, N = B.shape[2], B.shape[3]
    if G <= 0 or H % G:
        raise ValueError("H must be a multiple of G")
    logdecay = _chk(logdecay, (b, L, H), "logdecay")
    B = _chk(B, (b, L, G, N), "B")
    C = _chk(C, (b, L, G, N), "C")
    h0 = _opt(h0, (b, H, N, P))
    Y = np.empty((b, L, H, P))
    h = np.empty((b, H, N, P))
    _load().oracle_ssd(_p(X), _p(logdecay), _p(B), _p(C), _p(h0), _p(Y), _p(h),
                       b, L, H, P, G, N)
    return Y, h


def ssd_bwd(X, logdecay, B, C, dY, h0=None, dh_out=None):
    """Backward of the Mamba-2 SSD: the gradients of sum dY . Y + sum dh_out .
    h_out with respect to X, logdecay, B, C, h0.  Shapes as ssd(); dY like X,
    dh_out like h0.  Returns (dX, dlogdecay, dB, dC, dh0)."""
    X = _f64(X)
    b, L, H, P = X.shape
    B = _f64(B)
    G, N = B.shape[2], B.shape[3]
    if G <= 0 or H % G:
        raise ValueError("H must be a multiple of G")
    logdecay = _chk(logdecay, (b, L, H), "logdecay")
    B = _chk(B, (b, L, G, N), "B")
    C = _chk(C, (b, L, G, N), "C")
    dY = _chk(dY, (b, L, H, P), "dY")
    h0 = _opt(h0, (b, H, N, P))
    dh_out = _opt(dh_out, (b, H, N, P))
    dX = np.empty((b, L, H, P))
    dld = np.empty((b, L, H))
    dB = np.empty((b, L, G, N))
    dC = np.empty((b, L, G, N))
    dh0 = np.empty((b, H, N, P))
    _load().oracle_ssd_bwd(_p(X), _p(logdecay), _p(B), _p(C), _p(h0), _p(dY), _p(dh_out), _p(dX), _p(dld),
                           _p(dB), _p(dC), _p(dh0), b, L, H, P, G, N)
    return dX, dld, dB, dC, dh0


def trap(X, logdecay, B, C, beta, gamma, theta=None, h0=None, X_prev=None, B_prev=None):
    """Mamba-3 SISO.  X (b, L, H, P); logdecay, beta, gamma (b, L, H);
    B, C (b, L, G, N); theta (b, L, H, N/2) or None; X_prev (b, H, P) and
    B_prev (b, G, N): the token before the call, or None (zeros)."""
    X = _f64(X)
    b, L, H, P = X.shape
    B = _f64(B)
    G, N = B.shape[2], B.shape[3]
    if G <= 0 or H % G:
        raise ValueError("H must be a multiple of G")
    if theta is not None and N % 2:
        raise ValueError("rotation needs an even N")
    logdecay = _chk(logdecay, (b, L, H), "logdecay")
    beta = _chk(beta, (b, L, H), "beta")
    gamma = _chk(gamma, (b, L, H), "gamma")
    B = _chk(B, (b, L, G, N), "B")
    C = _chk(C, (b, L, G, N), "C")
    theta = _opt(theta, (b, L, H, N // 2))
    h0 = _opt(h0, (b, H, N, P))
    X_prev = _opt(X_prev, (b, H, P))
    B_prev = _opt(B_prev, (b, G, N))
    Y = np.empty((b, L, H, P))
    h = np.empty((b, H, N, P))
    _load().oracle_trap(_p(X), _p(logdecay), _p(B), _p(C), _p(beta), _p(gamma),
                        _p(theta), _p(h0), _p(X_prev), _p(B_prev), _p(Y), _p(h), b, L, H, P, G, N)
    return Y, h


def ssd_gated(X, logdecay, B, C, h0=None, D=None, z=None):
    """The Mamba-2 SSD followed by the block's output side (TorchMamba README, API
    reference Mamba2Block, psi = SiLU; the same skip-and-gate epilogue as the
    Mamba-3 block's, mamba3-minimal README, Architecture): Y = (ssd output + D[h]
    X) * SiLU(z), SiLU(v) = v / (1 + e^-v), x the scan's own input X.  D (H,) or
    None; z like X or None.  Returns (Y, h_out)."""
    Y, h = ssd(X, logdecay, B, C, h0)
    X = _f64(X)
    if D is not None:
        Y = Y + _f64(D)[None, None, :, None] * X
    if z is not None:
        z = _f64(z)
        Y = Y * (z / (1.0 + np.exp(-z)))
    return Y, h


def trap_gated(X, logdecay, B, C, beta, gamma, theta=None, h0=None, X_prev=None, B_prev=None, D=None, z=None):
    """Mamba-3 SISO followed by the block's output epilogue (mamba3-minimal
    README, Architecture): Y = (trap output + D[h] X) * SiLU(z), SiLU(v) =
    v / (1 + e^-v).  D (H,) or None; z like X or None.  Returns (Y, h_out)."""
    Y, h = trap(X, logdecay, B, C, beta, gamma, theta, h0, X_prev, B_prev)
    X = _f64(X)
    if D is not None:
        Y = Y + _f64(D)[None, None, :, None] * X
    if z is not None:
        z = _f64(z)
        Y = Y * (z / (1.0 + np.exp(-z)))
    return Y, h


def bc_norm_bias(Bg, H, w=None, bias=None, eps=1e-5):
    """The Mamba-3 B / C prologue (mamba3-minimal README, Architecture: a QK-style
    norm, then a bias, before the rotations): each row of the last axis (N
    states) divided by its root mean square (with eps inside the root), times
    the per-state weight w (N,), then the head's bias (H, N).  Bg (..., G, N)
    with the group axis second to last; returns (..., H, N), head h reading
    group h // (H / G)."""
    Bg = _f64(Bg)
    G, N = Bg.shape[-2], Bg.shape[-1]
    rms = np.sqrt(np.mean(Bg * Bg, axis=-1, keepdims=True) + eps)
    v = Bg / rms
    if w is not None:
        v = v * _f64(w)
    v = np.repeat(v, H // G, axis=-2)
    if bias is not None:
        v = v + _f64(bias)
    return v


def trap_block(X, logdecay, B, C, beta, gamma, theta=None, h0=None, X_prev=None, B_prev=None, normB_w=None,
               normC_w=None, biasB=None, biasC=None, eps=1e-5, D=None, z=None):
    """Mamba-3 SISO with both ends of its block: bc_norm_bias on B, C (and on the
    previous token's B), the trapezoid scan on the per-head rows, then the output
    epilogue of trap_gated.  Returns (Y, h_out)."""
    H = _f64(X).shape[2]
    Bh = bc_norm_bias(B, H, normB_w, biasB, eps)
    Ch = bc_norm_bias(C, H, normC_w, biasC, eps)
    Bp = None if B_prev is None else bc_norm_bias(B_prev, H, normB_w, biasB, eps)
    return trap_gated(X, logdecay, Bh, Ch, beta, gamma, theta, h0, X_prev, Bp, D=D, z=z)


def ssd_prologue(xBC, conv_w, dt, A, H, P, G, N, conv_b=None, dt_bias=None, x_hist=None):
    """The Mamba-2 block prologue (TorchMamba README, API reference Mamba2Block:
    d_conv taps, psi = SiLU; Math notes M1: the input scaled by dt, decay dt A):
    causal depthwise conv over time of each channel of xBC (the K - 1 steps
    before the call from x_hist, zeros without it), plus conv_b, SiLU; dt' =
    softplus(dt + dt_bias); X = x dt' per head, then B, C; logdecay = dt' A.
    Returns (X, B, C, logdecay, dt')."""
    xBC = _f64(xBC)
    conv_w = _f64(conv_w)
    b, L, cin = xBC.shape
    K = conv_w.shape[1]
    hist = np.zeros((b, K - 1, cin)) if x_hist is None else _f64(x_hist)
    full = np.concatenate([hist, xBC], axis=1)          # step t of the call is row t + K - 1
    pre = np.zeros((b, L, cin)) if conv_b is None else np.broadcast_to(_f64(conv_b), (b, L, cin)).copy()
    for k in range(K):                                   # tap k reads step t - K + 1 + k
        pre += conv_w[:, k] * full[:, k:k + L, :]
    v = pre / (1.0 + np.exp(-pre))
    u = _f64(dt) + (0.0 if dt_bias is None else _f64(dt_bias))
    dtp = np.logaddexp(0.0, u)
    HP, GN = H * P, G * N
    X = v[..., :HP].reshape(b, L, H, P) * dtp[..., None]
    Bo = v[..., HP:HP + GN].reshape(b, L, G, N)
    Co = v[..., HP + GN:].reshape(b, L, G, N)
    return X, Bo, Co, dtp * _f64(A), dtp


def ssd_block(xBC, conv_w, dt, A, H, P, G, N, conv_b=None, dt_bias=None, x_hist=None, h0=None, D=None, z=None):
    """The Mamba-2 layer around its scan (TorchMamba README, API reference
    Mamba2Block: d_conv taps, psi = SiLU; Math notes M2): ssd_prologue, the SSD
    on its outputs, then the output side Y = (ssd output + D[h] x) * SiLU(z),
    where x is the convolved, activated channel before the step size scales it
    (x = X / dt').  D (H,) or None; z (b, L, H, P) or None.  Returns (Y, h_out)."""
    X, Bo, Co, ld, dtp = ssd_prologue(xBC, conv_w, dt, A, H, P, G, N, conv_b, dt_bias, x_hist)
    Y, h = ssd(X, ld, Bo, Co, h0)
    if D is not None:
        Y = Y + _f64(D)[None, None, :, None] * (X / dtp[..., None])
    if z is not None:
        z = _f64(z)
        Y = Y * (z / (1.0 + np.exp(-z)))
    return Y, h


def trap_bwd(X, logdecay, B, C, beta, gamma, dY, theta=None, h0=None, dh_out=None, X_prev=None, B_prev=None):
    """Backward of the Mamba-3 SISO recurrence: the gradients of sum dY . Y + sum
    dh_out . h_out with respect to X, logdecay, B, C, beta, gamma, theta, h0,
    X_prev, B_prev.  Shapes as trap(); dY like X, dh_out like h0.  Returns (dX,
    dlogdecay, dB, dC, dbeta, dgamma, dtheta or None, dh0, dX_prev, dB_prev)."""
    X = _f64(X)
    b, L, H, P = X.shape
    B = _f64(B)
    G, N = B.shape[2], B.shape[3]
    if G <= 0 or H % G:
        raise ValueError("H must be a multiple of G")
    logdecay = _chk(logdecay, (b, L, H), "logdecay")
    beta = _chk(beta, (b, L, H), "beta")
    gamma = _chk(gamma, (b, L, H), "gamma")
    B = _chk(B, (b, L, G, N), "B")
    C = _chk(C, (b, L, G, N), "C")
    dY = _chk(dY, (b, L, H, P), "dY")
    theta = _opt(theta, (b, L, H, N // 2))
    h0 = _opt(h0, (b, H, N, P))
    dh_out = _opt(dh_out, (b, H, N, P))
    X_prev = _opt(X_prev, (b, H, P))
    B_prev = _opt(B_prev, (b, G, N))
    out = dict(dX=np.empty((b, L, H, P)), dld=np.empty((b, L, H)), dB=np.empty((b, L, G, N)),
               dC=np.empty((b, L, G, N)), dbeta=np.empty((b, L, H)), dgamma=np.empty((b, L, H)),
               dtheta=np.empty((b, L, H, N // 2)) if theta is not None else None, dh0=np.empty((b, H, N, P)),
               dX_prev=np.empty((b, H, P)), dB_prev=np.empty((b, G, N)))
    _load().oracle_trap_bwd(_p(X), _p(logdecay), _p(B), _p(C), _p(beta), _p(gamma), _p(theta), _p(h0), _p(X_prev),
                            _p(B_prev), _p(dY), _p(dh_out), _p(out["dX"]), _p(out["dld"]), _p(out["dB"]),
                            _p(out["dC"]), _p(out["dbeta"]), _p(out["dgamma"]), _p(out["dtheta"]), _p(out["dh0"]),
                            _p(out["dX_prev"]), _p(out["dB_prev"]), b, L, H, P, G, N)
    return (out["dX"], out["dld"], out["dB"], out["dC"], out["dbeta"], out["dgamma"], out["dtheta"], out["dh0"],
            out["dX_prev"], out["dB_prev"])


def mimo(X, logdecay, B, C, beta, gamma, theta=None, h0=None, X_prev=None, B_prev=None):
    """Mamba-3 MIMO.  X (b, L, H, P, R); B, C (b, L, H, N, R);
    logdecay, beta, gamma (b, L, H); theta (b, L, H, N/2) or None; X_prev
    (b, H, P, R) and B_prev (b, H, N, R): the token before the call, or None."""
    X = _f64(X)
    b, L, H, P, R = X.shape
    B = _f64(B)
    N = B.shape[3]
    if theta is not None and N % 2:
        raise ValueError("rotation needs an even N")
    logdecay = _chk(logdecay, (b, L, H), "logdecay")
    beta = _chk(beta, (b, L, H), "beta")
    gamma = _chk(gamma, (b, L, H), "gamma")
    B = _chk(B, (b, L, H, N, R), "B")
    C = _chk(C, (b, L, H, N, R), "C")
    theta = _opt(theta, (b, L, H, N // 2))
    h0 = _opt(h0, (b, H, N, P))
    X_prev = _opt(X_prev, (b, H, P, R))
    B_prev = _opt(B_prev, (b, H, N, R))
    Y = np.empty((b, L, H, P, R))
    h = np.empty((b, H, N, P))
    _load().oracle_mimo(_p(X), _p(logdecay), _p(B), _p(C), _p(beta), _p(gamma),
                        _p(theta), _p(h0), _p(X_prev), _p(B_prev), _p(Y), _p(h), b, L, H, P, N, R)
    return Y, h


def mimo_block(X, logdecay, B, C, beta, gamma, theta=None, h0=None, X_prev=None, B_prev=None, normB_w=None,
               normC_w=None, biasB=None, biasC=None, eps=1e-5, D=None, z=None):
    """Mamba-3 MIMO with both ends of its block (mamba3-minimal README,
    Architecture: B, C through the QK-style norm and the bias before the
    rotations; y + D x, then gated by SiLU(z); TorchMamba README, API reference:
    the MIMO block takes the SISO block's parameters plus the rank).  Reading:
    every rank's row of B and C over the N states (and of the previous token's
    B) goes through bc_norm_bias with the per-state weight and the head's bias,
    the same for all ranks; then the MIMO scan; then per rank Y_r = (Y_r + D[h]
    X_r) * SiLU(z_r), z like X.  B, C (b, L, H, N, R); B_prev (b, H, N, R) or
    None; D (H,) or None.  Returns (Y, h_out)."""
    X = _f64(X)
    H, R = X.shape[2], X.shape[4]

    def pro(Bv, w, bias):
        # rows (head, rank) over the states: head-major, rank-minor
        Bv = _f64(Bv)
        lead, (Hh, N, Rr) = Bv.shape[:-3], Bv.shape[-3:]
        rows = np.moveaxis(Bv, -1, -2).reshape(lead + (Hh * Rr, N))
        bias_rows = None if bias is None else np.repeat(_f64(bias), Rr, axis=0)
        v = bc_norm_bias(rows, Hh * Rr, w, bias_rows, eps)
        return np.moveaxis(v.reshape(lead + (Hh, Rr, N)), -1, -2)

    Bh = pro(B, normB_w, biasB)
    Ch = pro(C, normC_w, biasC)
    Bp = None if B_prev is None else pro(B_prev, normB_w, biasB)
    Y, h = mimo(X, logdecay, Bh, Ch, beta, gamma, theta, h0, X_prev, Bp)
    if D is not None:
        Y = Y + _f64(D)[None, None, :, None, None] * X
    if z is not None:
        z = _f64(z)
        Y = Y * (z / (1.0 + np.exp(-z)))
    return Y, h


def mimo_bwd(X, logdecay, B, C, beta, gamma, dY, theta=None, h0=None, dh_out=None, X_prev=None, B_prev=None):
    """Backward of the Mamba-3 MIMO recurrence: the gradients of sum dY . Y + sum
    dh_out . h_out with respect to X, logdecay, B, C, beta, gamma, theta, h0,
    X_prev, B_prev.  Shapes as mimo(); dY like X, dh_out like h0.  Returns (dX,
    dlogdecay, dB, dC, dbeta, dgamma, dtheta or None, dh0, dX_prev, dB_prev)."""
    X = _f64(X)
    b, L, H, P, R = X.shape
    B = _f64(B)
    N = B.shape[3]
    logdecay = _chk(logdecay, (b, L, H), "logdecay")
    beta = _chk(beta, (b, L, H), "beta")
    gamma = _chk(gamma, (b, L, H), "gamma")
    B = _chk(B, (b, L, H, N, R), "B")
    C = _chk(C, (b, L, H, N, R), "C")
    dY = _chk(dY, (b, L, H, P, R), "dY")
    theta = _opt(theta, (b, L, H, N // 2))
    h0 = _opt(h0, (b, H, N, P))
    dh_out = _opt(dh_out, (b, H, N, P))
    X_prev = _opt(X_prev, (b, H, P, R))
    B_prev = _opt(B_prev, (b, H, N, R))
    out = dict(dX=np.empty((b, L, H, P, R)), dld=np.empty((b, L, H)), dB=np.empty((b, L, H, N, R)),
               dC=np.empty((b, L, H, N, R)), dbeta=np.empty((b, L, H)), dgamma=np.empty((b, L, H)),
               dtheta=np.empty((b, L, H, N // 2)) if theta is not None else None, dh0=np.empty((b, H, N, P)),
               dX_prev=np.empty((b, H, P, R)), dB_prev=np.empty((b, H, N, R)))
    _load().oracle_mimo_bwd(_p(X), _p(logdecay), _p(B), _p(C), _p(beta), _p(gamma), _p(theta), _p(h0), _p(X_prev),
                            _p(B_prev), _p(dY), _p(dh_out), _p(out["dX"]), _p(out["dld"]), _p(out["dB"]),
                            _p(out["dC"]), _p(out["dbeta"]), _p(out["dgamma"]), _p(out["dtheta"]), _p(out["dh0"]),
                            _p(out["dX_prev"]), _p(out["dB_prev"]), b, L, H, P, N, R)
    return (out["dX"], out["dld"], out["dB"], out["dC"], out["dbeta"], out["dgamma"], out["dtheta"], out["dh0"],
            out["dX_prev"], out["dB_prev"])


def ssd_step(X, logdecay, B, C, h=None, beta=None, gamma=None, theta=None, X_prev=None, B_prev=None):
    """One decode token of the SSD family, physical-frame state.
    X, X_prev (b, H, P[, R]); B, C, B_prev (b, G, N[, R]); logdecay, beta,
    gamma (b, H); theta (b, H, N/2); h (b, H, N, P).  Without the R axis, R = 1.
    beta None = 0, gamma None = 1, theta None = no rotation, X_prev / B_prev /
    h None = 0.  Returns (Y, h_out) with Y shaped like X."""
    X = _f64(X)
    squeeze = X.ndim == 3
    if squeeze:
        X = X[..., None]
    b, H, P, R = X.shape
    B = _f64(B)
    if B.ndim == 3:
        B = B[..., None]
    G, N = B.shape[1], B.shape[2]
    if G <= 0 or H % G:
        raise ValueError("H must be a multiple of G")
    if theta is not None and N % 2:
        raise ValueError("rotation needs an even N")

    def r4(a, shape, name):
        if a is None:
            return None
        a = _f64(a)
        return _chk(a[..., None] if a.ndim == len(shape) - 1 else a, shape, name)

    B = _chk(B, (b, G, N, R), "B")
    C = r4(C, (b, G, N, R), "C")
    B_prev = r4(B_prev, (b, G, N, R), "B_prev")
    X_prev = r4(X_prev, (b, H, P, R), "X_prev")
    logdecay = _chk(logdecay, (b, H), "logdecay")
    beta = _opt(beta, (b, H))
    gamma = _opt(gamma, (b, H))
    theta = _opt(theta, (b, H, N // 2))
    h = _opt(h, (b, H, N, P))
    Y = np.empty((b, H, P, R))
    hout = np.empty((b, H, N, P))
    _load().oracle_ssd_step(_p(X), _p(logdecay), _p(B), _p(C), _p(beta), _p(gamma), _p(theta),
                            _p(X_prev), _p(B_prev), _p(h), _p(Y), _p(hout), b, H, P, G, N, R)
    return (Y[..., 0] if squeeze else Y), hout


def m1_block(x, conv_w, dt, A, B, C, D=None, h0=None, conv_b=None, dt_bias=None, z=None, x_hist=None):
    """Mamba-1 scan with the block prologue and epilogue.  x, dt, z (b, L, D);
    conv_w (D, K); conv_b, dt_bias, D (D,); A (D, N); B, C (b, L, N); h0
    (b, D, N); x_hist (b, K-1, D).  Returns (y, h_out)."""
    x = _f64(x)
    b, L, Dm = x.shape
    conv_w = _f64(conv_w)
    K = conv_w.shape[1]
    A = _f64(A)
    N = A.shape[1]
    conv_w = _chk(conv_w, (Dm, K), "conv_w")
    dt = _chk(dt, (b, L, Dm), "dt")
    A = _chk(A, (Dm, N), "A")
    B = _chk(B, (b, L, N), "B")
    C = _chk(C, (b, L, N), "C")
    D = _opt(D, (Dm,))
    h0 = _opt(h0, (b, Dm, N))
    conv_b = _opt(conv_b, (Dm,))
    dt_bias = _opt(dt_bias, (Dm,))
    z = _opt(z, (b, L, Dm))
    x_hist = _opt(x_hist, (b, K - 1, Dm)) if K > 1 else None
    y = np.empty((b, L, Dm))
    h = np.empty((b, Dm, N))
    _load().oracle_m1_block(_p(x), _p(x_hist), _p(conv_w), _p(conv_b), _p(dt), _p(dt_bias), _p(A), _p(B),
                            _p(C), _p(D), _p(z), _p(h0), _p(y), _p(h), b, L, Dm, N, K)
    return y, h
