"""MI355X-native selective state-space scans.

Thin Python binding over the C ABI in ``include/mb.h`` (``libmb.so``, built by
``python -m selective_state_space_amd._build``).  The functions carry the same
names as the C entry points and do argument marshalling only: check that the
torch tensors are contiguous CUDA tensors of the right dtype and shape, allocate
missing outputs and workspace with torch, and call the library on the current
stream.  Every step of every scan runs in the HIP kernels; there is no fallback.
If the library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "mb_selective_scan", "mb_ssm_step", "mb_ssd_chunked", "mb_trap_ssd", "mb_mimo_ssd",
    "mb_ssd_step", "mb_selective_scan_fused", "mb_ssd_chunked_bwd", "mb_selective_scan_bwd", "mb_trap_ssd_bwd", "mb_mimo_ssd_bwd", "mb_trap_ssd_gated", "mb_trap_ssd_block", "mb_ssd_prologue", "mb_mimo_ssd_block", "mb_ssd_chunked_gated", "mb_ssd_chunked_noalloc", "mb_workspace_size", "mb_status_str", "lib_path", "load_library", "MBError",
    "MB_OP_SELECTIVE_SCAN", "MB_OP_SSM_STEP", "MB_OP_SSD_CHUNKED", "MB_OP_TRAP_SSD",
    "MB_OP_MIMO_SSD", "MB_OP_SSD_CHUNKED_BWD", "MB_OP_SELECTIVE_SCAN_BWD", "MB_OP_TRAP_SSD_BWD",
    "MB_OP_MIMO_SSD_BWD", "MB_OP_SSD_BLOCK", "MB_OP_SSD_BLOCK_BF16", "mb_ssd_block",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmb.so")
_lock = threading.Lock()
_lib = None

MB_F32, MB_BF16 = 0, 1
(MB_OP_SELECTIVE_SCAN, MB_OP_SSM_STEP, MB_OP_SSD_CHUNKED, MB_OP_TRAP_SSD,
 MB_OP_MIMO_SSD, MB_OP_SSD_CHUNKED_BWD, MB_OP_SELECTIVE_SCAN_BWD, MB_OP_TRAP_SSD_BWD,
 MB_OP_MIMO_SSD_BWD, MB_OP_SSD_BLOCK, MB_OP_SSD_BLOCK_BF16) = range(11)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class MBError(ValueError):
    """A libmb entry point returned a status other than MB_OK."""

    def __init__(self, fn, status):
        msg = "%s failed: %s (status %d)" % (fn, mb_status_str(status), status)
        if status == 5:
            msg += ", hipError %d" % load_library().mb_last_hip_error()
        super().__init__(msg)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmb.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libmb.so not built: run `python -m selective_state_space_amd._build`")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.mb_selective_scan.argtypes = [_vp] * 9 + [_i64] * 4 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        lib.mb_ssm_step.argtypes = [_vp] * 9 + [_i64] * 3 + [ctypes.c_int, _vp]
        if hasattr(lib, "mb_ssd_chunked"):
            lib.mb_ssd_chunked.argtypes = [_vp] * 7 + [_i64] * 7 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_trap_ssd.argtypes = [_vp] * 12 + [_i64] * 7 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_mimo_ssd.argtypes = [_vp] * 12 + [_i64] * 7 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_workspace_size.argtypes = [ctypes.c_int] + [_i64] * 8
            lib.mb_workspace_size.restype = ctypes.c_size_t
            for f in ("mb_ssd_chunked", "mb_trap_ssd", "mb_mimo_ssd"):
                getattr(lib, f).restype = ctypes.c_int
        if hasattr(lib, "mb_ssd_block"):
            lib.mb_ssd_block.argtypes = [_vp] * 12 + [_i64] * 7 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_ssd_block.restype = ctypes.c_int
        if hasattr(lib, "mb_ssd_chunked_gated"):
            lib.mb_ssd_chunked_gated.argtypes = [_vp] * 9 + [_i64] * 7 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_ssd_chunked_gated.restype = ctypes.c_int
        if hasattr(lib, "mb_ssd_chunked_noalloc"):
            lib.mb_ssd_chunked_noalloc.argtypes = [_vp] * 7 + [_i64] * 7 + [ctypes.c_int, _vp]
            lib.mb_ssd_chunked_noalloc.restype = ctypes.c_int
        if hasattr(lib, "mb_trap_ssd_gated"):
            lib.mb_trap_ssd_gated.argtypes = [_vp] * 14 + [_i64] * 7 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_trap_ssd_gated.restype = ctypes.c_int
        if hasattr(lib, "mb_ssd_prologue"):
            lib.mb_ssd_prologue.argtypes = [_vp] * 12 + [_i64] * 7 + [ctypes.c_int, _vp]
            lib.mb_ssd_prologue.restype = ctypes.c_int
        if hasattr(lib, "mb_trap_ssd_block"):
            lib.mb_trap_ssd_block.argtypes = [_vp] * 14 + [ctypes.c_float] + [_vp] * 4 + [_i64] * 7 + \
                [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_trap_ssd_block.restype = ctypes.c_int
        if hasattr(lib, "mb_mimo_ssd_block"):
            lib.mb_mimo_ssd_block.argtypes = [_vp] * 14 + [ctypes.c_float] + [_vp] * 4 + [_i64] * 7 + \
                [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_mimo_ssd_block.restype = ctypes.c_int
        if hasattr(lib, "mb_mimo_ssd_bwd"):
            lib.mb_mimo_ssd_bwd.argtypes = [_vp] * 22 + [_i64] * 6 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_mimo_ssd_bwd.restype = ctypes.c_int
        if hasattr(lib, "mb_trap_ssd_bwd"):
            lib.mb_trap_ssd_bwd.argtypes = [_vp] * 22 + [_i64] * 6 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_trap_ssd_bwd.restype = ctypes.c_int
        if hasattr(lib, "mb_selective_scan_bwd"):
            lib.mb_selective_scan_bwd.argtypes = [_vp] * 16 + [_i64] * 4 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_selective_scan_bwd.restype = ctypes.c_int
        if hasattr(lib, "mb_ssd_chunked_bwd"):
            lib.mb_ssd_chunked_bwd.argtypes = [_vp] * 12 + [_i64] * 6 + [ctypes.c_int, _vp, ctypes.c_size_t, _vp]
            lib.mb_ssd_chunked_bwd.restype = ctypes.c_int
        if hasattr(lib, "mb_selective_scan_fused"):
            lib.mb_selective_scan_fused.argtypes = [_vp] * 14 + [_i64] * 5 + [ctypes.c_int, _vp]
            lib.mb_selective_scan_fused.restype = ctypes.c_int
        if hasattr(lib, "mb_ssd_step"):
            lib.mb_ssd_step.argtypes = [_vp] * 12 + [_i64] * 6 + [ctypes.c_int, _vp]
            lib.mb_ssd_step.restype = ctypes.c_int
        lib.mb_status_str.argtypes = [ctypes.c_int]
        lib.mb_status_str.restype = ctypes.c_char_p
        lib.mb_last_hip_error.restype = ctypes.c_int
        lib.mb_version.restype = ctypes.c_int
        for f in ("mb_selective_scan", "mb_ssm_step"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
        return lib


def mb_status_str(status: int) -> str:
    return load_library().mb_status_str(int(status)).decode()


def mb_workspace_size(op, batch, L, H, P, G, N, R=1, chunk=0) -> int:
    return int(load_library().mb_workspace_size(int(op), batch, L, H, P, G, N, R, chunk))


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t, name):
    torch = _torch()
    if t.dtype == torch.float32:
        return MB_F32
    if t.dtype == torch.bfloat16:
        return MB_BF16
    raise TypeError("%s must be float32 or bfloat16, got %s" % (name, t.dtype))


def _check(t, name, shape, dtype, device):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(fn, *args):
    st = getattr(load_library(), fn)(*args)
    if st != 0:
        raise MBError(fn, st)


def _device_of(t):
    if not t.is_cuda:
        raise ValueError("tensors must be on a CUDA (HIP) device, got %s" % t.device)
    return t.device


def _workspace(op, device, ws, dims):
    torch = _torch()
    need = mb_workspace_size(op, *dims)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return ws, ws.numel() * ws.element_size()


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def mb_selective_scan(x, dt, A, B, C, D=None, h0=None, *, y=None, h_out=None, ws=None, seq_blocks=True):
    """Mamba-1 selective scan.  x, dt (batch, L, D) and B, C (batch, L, N) share
    one dtype (float32 or bfloat16); A (D, N), D (D,), h0 (batch, D, N) float32.
    With seq_blocks (the default) the library may cut the sequence into blocks
    run in parallel (a workspace is allocated here unless `ws` is given);
    seq_blocks=False runs the whole sequence in one block.  Returns (y, h_out)."""
    torch = _torch()
    dev = _device_of(x)
    dtype = x.dtype
    code = _dtype_code(x, "x")
    b, L, Dm = x.shape
    N = A.shape[1]
    _check(x, "x", (b, L, Dm), dtype, dev)
    _check(dt, "dt", (b, L, Dm), dtype, dev)
    _check(A, "A", (Dm, N), torch.float32, dev)
    _check(B, "B", (b, L, N), dtype, dev)
    _check(C, "C", (b, L, N), dtype, dev)
    _check(D, "D", (Dm,), torch.float32, dev)
    _check(h0, "h0", (b, Dm, N), torch.float32, dev)
    y = torch.empty((b, L, Dm), dtype=dtype, device=dev) if y is None else _check(y, "y", (b, L, Dm), dtype, dev)
    h_out = torch.empty((b, Dm, N), dtype=torch.float32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, Dm, N), torch.float32, dev)
    nws = 0
    if seq_blocks and mb_workspace_size(MB_OP_SELECTIVE_SCAN, b, L, Dm, 1, 1, N) > 0:
        ws, nws = _workspace(MB_OP_SELECTIVE_SCAN, dev, ws, (b, L, Dm, 1, 1, N, 1, 0))
    else:
        ws = None
    _call("mb_selective_scan", _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
          _ptr(y), _ptr(h_out), b, L, Dm, N, code, _ptr(ws), nws, _stream(dev))
    return y, h_out


def mb_ssm_step(x, dt, A, B, C, D, h, *, y=None, h_out=None):
    """Mamba-1 decode step.  x, dt (batch, D), B, C (batch, N) in one dtype; A
    (D, N), D (D,) or None, h (batch, D, N) float32.  With h_out=None the state
    is updated in place.  Returns (y, h_out)."""
    torch = _torch()
    dev = _device_of(x)
    dtype = x.dtype
    code = _dtype_code(x, "x")
    b, Dm = x.shape
    N = A.shape[1]
    _check(dt, "dt", (b, Dm), dtype, dev)
    _check(A, "A", (Dm, N), torch.float32, dev)
    _check(B, "B", (b, N), dtype, dev)
    _check(C, "C", (b, N), dtype, dev)
    _check(D, "D", (Dm,), torch.float32, dev)
    _check(h, "h", (b, Dm, N), torch.float32, dev)
    h_out = h if h_out is None else _check(h_out, "h_out", (b, Dm, N), torch.float32, dev)
    y = torch.empty((b, Dm), dtype=dtype, device=dev) if y is None else _check(y, "y", (b, Dm), dtype, dev)
    _call("mb_ssm_step", _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h), _ptr(h_out),
          _ptr(y), b, Dm, N, code, _stream(dev))
    return y, h_out


def mb_ssd_chunked(X, logdecay, B, C, h0=None, *, chunk=0, Y=None, h_out=None, ws=None):
    """Mamba-2 SSD.  X (batch, L, H, P), B, C (batch, L, G, N) in one dtype;
    logdecay (batch, L, H), h0 (batch, H, N, P) float32.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check(logdecay, "logdecay", (b, L, H), torch.float32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, G, N), dtype, dev)
    _check(h0, "h0", (b, H, N, P), torch.float32, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), torch.float32, dev)
    ws, nws = _workspace(MB_OP_SSD_CHUNKED, dev, ws, (b, L, H, P, G, N, 1, chunk))
    _call("mb_ssd_chunked", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(h0), _ptr(Y), _ptr(h_out),
          b, L, H, P, G, N, chunk, code, _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_ssd_block(xBC, conv_w, dt, A, H, P, G, N, *, conv_b=None, dt_bias=None, x_hist=None, D=None, z=None,
                 h0=None, Y=None, h_out=None, ws=None):
    """The Mamba-2 layer around its scan in one call: conv1d + SiLU over xBC
    (batch, L, H*P + 2*G*N), softplus(dt + dt_bias), the chunked SSD and the
    output side (y + D[h] x) * SiLU(z).  xBC, x_hist, z and Y share one dtype
    (float32 or bfloat16); conv_w (channels, K), conv_b, dt (batch, L, H),
    dt_bias, A, D float32.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(xBC)
    dtype = xBC.dtype
    code = _dtype_code(xBC, "xBC")
    b, L, cin = xBC.shape
    if cin != H * P + 2 * G * N:
        raise ValueError("xBC has %d channels; H*P + 2*G*N = %d" % (cin, H * P + 2 * G * N))
    K = conv_w.shape[1]
    f32 = torch.float32
    _check(xBC, "xBC", (b, L, cin), dtype, dev)
    _check(conv_w, "conv_w", (cin, K), f32, dev)
    _check(conv_b, "conv_b", (cin,), f32, dev)
    _check(x_hist, "x_hist", (b, K - 1, cin), dtype, dev)
    _check(dt, "dt", (b, L, H), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(z, "z", (b, L, H, P), dtype, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), f32, dev)
    ws, nws = _workspace(MB_OP_SSD_BLOCK_BF16 if code == MB_BF16 else MB_OP_SSD_BLOCK, dev, ws,
                         (b, L, H, P, G, N, 1, 0))
    _call("mb_ssd_block", _ptr(xBC), _ptr(conv_w), _ptr(conv_b), _ptr(x_hist), _ptr(dt), _ptr(dt_bias), _ptr(A),
          _ptr(D), _ptr(z), _ptr(h0), _ptr(Y), _ptr(h_out), b, L, H, P, G, N, K, code, _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_ssd_chunked_gated(X, logdecay, B, C, h0=None, *, D=None, z=None, chunk=0, Y=None, h_out=None, ws=None):
    """Mamba-2 SSD with the block's output side fused into the store: Y = (SSD
    output + D[h] X) * SiLU(z).  D (H,) float32 or None; z like X (same dtype) or
    None; the rest as mb_ssd_chunked.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check(logdecay, "logdecay", (b, L, H), torch.float32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, G, N), dtype, dev)
    _check(h0, "h0", (b, H, N, P), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(z, "z", (b, L, H, P), dtype, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), torch.float32, dev)
    ws, nws = _workspace(MB_OP_SSD_CHUNKED, dev, ws, (b, L, H, P, G, N, 1, chunk))
    _call("mb_ssd_chunked_gated", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(h0), _ptr(D), _ptr(z), _ptr(Y),
          _ptr(h_out), b, L, H, P, G, N, chunk, code, _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_ssd_chunked_noalloc(X, logdecay, B, C, h0=None, *, chunk=0, Y=None, h_out=None):
    """mb_ssd_chunked on the library's static device workspace (the C entry
    point allocates nothing; pass Y and h_out to keep this wrapper from
    allocating them).  Same shapes and result as mb_ssd_chunked; sizes needing
    more than 32 MiB of workspace are rejected.  Calls that overlap in time on
    one device share that workspace and race.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check(logdecay, "logdecay", (b, L, H), torch.float32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, G, N), dtype, dev)
    _check(h0, "h0", (b, H, N, P), torch.float32, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), torch.float32, dev)
    _call("mb_ssd_chunked_noalloc", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(h0), _ptr(Y), _ptr(h_out),
          b, L, H, P, G, N, chunk, code, _stream(dev))
    return Y, h_out


def mb_selective_scan_bwd(x, dt, A, B, C, dy, D=None, h0=None, dh_out=None, *, dx=None, ddt=None, dA=None,
                          dB=None, dC=None, dD=None, dh0=None, ws=None):
    """Backward of the Mamba-1 scan (float32): the gradients of sum dy . y + sum
    dh_out . h_out with respect to x, dt, A, B, C, D and h0.  Shapes as
    mb_selective_scan; dy like x, dh_out like h0 (None: zero).  Returns (dx, ddt,
    dA, dB, dC, dD, dh0)."""
    torch = _torch()
    dev = _device_of(x)
    f32 = torch.float32
    b, L, Dm = x.shape
    N = A.shape[1]
    _check(x, "x", (b, L, Dm), f32, dev)
    _check(dt, "dt", (b, L, Dm), f32, dev)
    _check(A, "A", (Dm, N), f32, dev)
    _check(B, "B", (b, L, N), f32, dev)
    _check(C, "C", (b, L, N), f32, dev)
    _check(dy, "dy", (b, L, Dm), f32, dev)
    _check(D, "D", (Dm,), f32, dev)
    _check(h0, "h0", (b, Dm, N), f32, dev)
    _check(dh_out, "dh_out", (b, Dm, N), f32, dev)
    out = []
    for t, n, shp in ((dx, "dx", (b, L, Dm)), (ddt, "ddt", (b, L, Dm)), (dA, "dA", (Dm, N)), (dB, "dB", (b, L, N)),
                      (dC, "dC", (b, L, N)), (dD, "dD", (Dm,)), (dh0, "dh0", (b, Dm, N))):
        out.append(torch.empty(shp, dtype=f32, device=dev) if t is None else _check(t, n, shp, f32, dev))
    ws, nws = _workspace(MB_OP_SELECTIVE_SCAN_BWD, dev, ws, (b, L, Dm, 1, 1, N, 1, 0))
    _call("mb_selective_scan_bwd", _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy),
          _ptr(dh_out), *[_ptr(t) for t in out], b, L, Dm, N, MB_F32, _ptr(ws), nws, _stream(dev))
    return tuple(out)


def mb_trap_ssd_bwd(X, logdecay, B, C, beta, gamma, dY, theta=None, h0=None, dh_out=None, *, X_prev=None,
                    B_prev=None, ws=None):
    """Backward of the Mamba-3 SISO recurrence (float32): the gradients of sum
    dY . Y + sum dh_out . h_out with respect to X, logdecay, B, C, beta, gamma,
    theta, h0, X_prev, B_prev.  Shapes as mb_trap_ssd.  Returns (dX, dlogdecay,
    dB, dC, dbeta, dgamma, dtheta or None, dh0, dX_prev or None, dB_prev or None)."""
    torch = _torch()
    dev = _device_of(X)
    f32 = torch.float32
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check(X, "X", (b, L, H, P), f32, dev)
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, G, N), f32, dev)
    _check(C, "C", (b, L, G, N), f32, dev)
    _check(dY, "dY", (b, L, H, P), f32, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(dh_out, "dh_out", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P), f32, dev)
    _check(B_prev, "B_prev", (b, G, N), f32, dev)
    e = lambda shp: torch.empty(shp, dtype=f32, device=dev)
    dX, dld, dB, dC = e((b, L, H, P)), e((b, L, H)), e((b, L, G, N)), e((b, L, G, N))
    dbeta, dgamma, dh0 = e((b, L, H)), e((b, L, H)), e((b, H, N, P))
    dtheta = e((b, L, H, N // 2)) if theta is not None else None
    dXp = e((b, H, P)) if X_prev is not None else None
    dBp = e((b, G, N)) if B_prev is not None else None
    ws, nws = _workspace(MB_OP_TRAP_SSD_BWD, dev, ws, (b, L, H, P, G, N, 1, 0))
    _call("mb_trap_ssd_bwd", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma), _ptr(theta),
          _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(dY), _ptr(dh_out), _ptr(dX), _ptr(dld), _ptr(dB), _ptr(dC),
          _ptr(dbeta), _ptr(dgamma), _ptr(dtheta), _ptr(dh0), _ptr(dXp), _ptr(dBp), b, L, H, P, G, N, MB_F32,
          _ptr(ws), nws, _stream(dev))
    return dX, dld, dB, dC, dbeta, dgamma, dtheta, dh0, dXp, dBp


def mb_mimo_ssd_bwd(X, logdecay, B, C, beta, gamma, dY, theta=None, h0=None, dh_out=None, *, X_prev=None,
                    B_prev=None, ws=None):
    """Backward of the Mamba-3 MIMO recurrence (float32).  Shapes as mb_mimo_ssd;
    dY like X, dh_out like h0.  Returns (dX, dlogdecay, dB, dC, dbeta, dgamma,
    dtheta or None, dh0, dX_prev or None, dB_prev or None)."""
    torch = _torch()
    dev = _device_of(X)
    f32 = torch.float32
    b, L, H, P, R = X.shape
    N = B.shape[3]
    _check(X, "X", (b, L, H, P, R), f32, dev)
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, H, N, R), f32, dev)
    _check(C, "C", (b, L, H, N, R), f32, dev)
    _check(dY, "dY", (b, L, H, P, R), f32, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(dh_out, "dh_out", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P, R), f32, dev)
    _check(B_prev, "B_prev", (b, H, N, R), f32, dev)
    e = lambda shp: torch.empty(shp, dtype=f32, device=dev)
    dX, dld, dB, dC = e((b, L, H, P, R)), e((b, L, H)), e((b, L, H, N, R)), e((b, L, H, N, R))
    dbeta, dgamma, dh0 = e((b, L, H)), e((b, L, H)), e((b, H, N, P))
    dtheta = e((b, L, H, N // 2)) if theta is not None else None
    dXp = e((b, H, P, R)) if X_prev is not None else None
    dBp = e((b, H, N, R)) if B_prev is not None else None
    ws, nws = _workspace(MB_OP_MIMO_SSD_BWD, dev, ws, (b, L, H, P, 1, N, R, 0))
    _call("mb_mimo_ssd_bwd", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma), _ptr(theta),
          _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(dY), _ptr(dh_out), _ptr(dX), _ptr(dld), _ptr(dB), _ptr(dC),
          _ptr(dbeta), _ptr(dgamma), _ptr(dtheta), _ptr(dh0), _ptr(dXp), _ptr(dBp), b, L, H, P, N, R, MB_F32,
          _ptr(ws), nws, _stream(dev))
    return dX, dld, dB, dC, dbeta, dgamma, dtheta, dh0, dXp, dBp


def mb_ssd_chunked_bwd(X, logdecay, B, C, dY, h0=None, dh_out=None, *, dX=None, dlogdecay=None, dB=None,
                       dC=None, dh0=None, ws=None):
    """Backward of the Mamba-2 SSD (float32): the gradients of sum dY . Y + sum
    dh_out . h_out with respect to X, logdecay, B, C and h0.  Shapes as
    mb_ssd_chunked; dY like X, dh_out like h0 (None: zero).  Returns (dX,
    dlogdecay, dB, dC, dh0)."""
    torch = _torch()
    dev = _device_of(X)
    f32 = torch.float32
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check(X, "X", (b, L, H, P), f32, dev)
    _check(logdecay, "logdecay", (b, L, H), f32, dev)
    _check(B, "B", (b, L, G, N), f32, dev)
    _check(C, "C", (b, L, G, N), f32, dev)
    _check(dY, "dY", (b, L, H, P), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(dh_out, "dh_out", (b, H, N, P), f32, dev)
    out = []
    for t, n, shp in ((dX, "dX", (b, L, H, P)), (dlogdecay, "dlogdecay", (b, L, H)), (dB, "dB", (b, L, G, N)),
                      (dC, "dC", (b, L, G, N)), (dh0, "dh0", (b, H, N, P))):
        out.append(torch.empty(shp, dtype=f32, device=dev) if t is None else _check(t, n, shp, f32, dev))
    ws, nws = _workspace(MB_OP_SSD_CHUNKED_BWD, dev, ws, (b, L, H, P, G, N, 1, 0))
    _call("mb_ssd_chunked_bwd", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(h0), _ptr(dY), _ptr(dh_out),
          *[_ptr(t) for t in out], b, L, H, P, G, N, MB_F32, _ptr(ws), nws, _stream(dev))
    return tuple(out)


def mb_trap_ssd(X, logdecay, B, C, beta, gamma, theta=None, h0=None, *, X_prev=None, B_prev=None,
                chunk=0, Y=None, h_out=None, ws=None):
    """Mamba-3 SISO.  X (batch, L, H, P), B, C (batch, L, G, N) in one dtype;
    logdecay, beta, gamma (batch, L, H), theta (batch, L, H, N/2) or None, h0
    (batch, H, N, P) float32 (physical frame); X_prev (batch, H, P) and B_prev
    (batch, G, N): the token before the call, or None.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    f32 = torch.float32
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, G, N), dtype, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P), dtype, dev)
    _check(B_prev, "B_prev", (b, G, N), dtype, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), f32, dev)
    ws, nws = _workspace(MB_OP_TRAP_SSD, dev, ws, (b, L, H, P, G, N, 1, chunk))
    _call("mb_trap_ssd", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma),
          _ptr(theta), _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(Y), _ptr(h_out), b, L, H, P, G, N, chunk,
          code, _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_trap_ssd_gated(X, logdecay, B, C, beta, gamma, theta=None, h0=None, *, D=None, z=None, X_prev=None,
                      B_prev=None, chunk=0, Y=None, h_out=None, ws=None):
    """Mamba-3 SISO with the block's output epilogue fused: Y = (SSD output + D[h]
    X) * SiLU(z).  D (H,) float32 or None; z like X (same dtype) or None; the rest
    as mb_trap_ssd.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    f32 = torch.float32
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, G, N), dtype, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P), dtype, dev)
    _check(B_prev, "B_prev", (b, G, N), dtype, dev)
    _check(D, "D", (H,), f32, dev)
    _check(z, "z", (b, L, H, P), dtype, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), f32, dev)
    ws, nws = _workspace(MB_OP_TRAP_SSD, dev, ws, (b, L, H, P, G, N, 1, chunk))
    _call("mb_trap_ssd_gated", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma),
          _ptr(theta), _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(D), _ptr(z), _ptr(Y), _ptr(h_out), b, L, H, P, G,
          N, chunk, code, _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_trap_ssd_block(X, logdecay, B, C, beta, gamma, theta=None, h0=None, *, normB_w=None, normC_w=None,
                      biasB=None, biasC=None, eps=1e-5, D=None, z=None, X_prev=None, B_prev=None, chunk=0,
                      Y=None, h_out=None, ws=None):
    """Mamba-3 SISO with the block's BCNorm + bias prologue on B, C and its output
    epilogue fused into the scan.  normB_w, normC_w (N,) float32 or None; biasB,
    biasC (H, N) float32 or None; eps > 0; D, z and the rest as
    mb_trap_ssd_gated.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    f32 = torch.float32
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, G, N), dtype, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P), dtype, dev)
    _check(B_prev, "B_prev", (b, G, N), dtype, dev)
    _check(normB_w, "normB_w", (N,), f32, dev)
    _check(normC_w, "normC_w", (N,), f32, dev)
    _check(biasB, "biasB", (H, N), f32, dev)
    _check(biasC, "biasC", (H, N), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(z, "z", (b, L, H, P), dtype, dev)
    Y = torch.empty((b, L, H, P), dtype=dtype, device=dev) if Y is None else _check(Y, "Y", (b, L, H, P), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), f32, dev)
    ws, nws = _workspace(MB_OP_TRAP_SSD, dev, ws, (b, L, H, P, G, N, 1, chunk))
    _call("mb_trap_ssd_block", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma),
          _ptr(theta), _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(normB_w), _ptr(normC_w), _ptr(biasB),
          _ptr(biasC), float(eps), _ptr(D), _ptr(z), _ptr(Y), _ptr(h_out), b, L, H, P, G, N, chunk, code,
          _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_mimo_ssd_block(X, logdecay, B, C, beta, gamma, theta=None, h0=None, *, normB_w=None, normC_w=None,
                      biasB=None, biasC=None, eps=1e-5, D=None, z=None, X_prev=None, B_prev=None, chunk=0,
                      Y=None, h_out=None, ws=None):
    """Mamba-3 MIMO with the block's BCNorm + bias prologue on every rank row of
    B, C and the skip term and SiLU(z) gate per rank fused into the scan.  X, z
    (batch, L, H, P, R), B, C (batch, L, H, N, R) in one dtype; normB_w, normC_w
    (N,), biasB, biasC (H, N), D (H,) float32 or None; the rest as mb_mimo_ssd.
    R in {1, 2, 4, 8, 16}.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P, R = X.shape
    N = B.shape[3]
    f32 = torch.float32
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, H, N, R), dtype, dev)
    _check(C, "C", (b, L, H, N, R), dtype, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P, R), dtype, dev)
    _check(B_prev, "B_prev", (b, H, N, R), dtype, dev)
    _check(normB_w, "normB_w", (N,), f32, dev)
    _check(normC_w, "normC_w", (N,), f32, dev)
    _check(biasB, "biasB", (H, N), f32, dev)
    _check(biasC, "biasC", (H, N), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(z, "z", (b, L, H, P, R), dtype, dev)
    Y = torch.empty((b, L, H, P, R), dtype=dtype, device=dev) if Y is None else \
        _check(Y, "Y", (b, L, H, P, R), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), f32, dev)
    ws, nws = _workspace(MB_OP_MIMO_SSD, dev, ws, (b, L, H, P, 1, N, R, chunk))
    _call("mb_mimo_ssd_block", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma),
          _ptr(theta), _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(normB_w), _ptr(normC_w), _ptr(biasB),
          _ptr(biasC), float(eps), _ptr(D), _ptr(z), _ptr(Y), _ptr(h_out), b, L, H, P, N, R, chunk, code,
          _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_ssd_prologue(xBC, conv_w, dt, A, H, P, G, N, *, conv_b=None, x_hist=None, dt_bias=None, X=None, B=None,
                    C=None, logdecay=None, dt_out=False):
    """Mamba-2 block prologue: conv1d + SiLU over xBC (batch, L, H*P + 2*G*N),
    softplus(dt + dt_bias), split into the SSD inputs.  xBC, x_hist and the
    outputs X, B, C in one dtype (float32 or bfloat16); the rest float32.  Returns
    (X, B, C, logdecay) or, with dt_out=True, (X, B, C, logdecay, dt')."""
    torch = _torch()
    dev = _device_of(xBC)
    f32 = torch.float32
    act = xBC.dtype
    code = _dtype_code(xBC, "xBC")
    b, L, cin = xBC.shape
    K = conv_w.shape[1]
    _check(xBC, "xBC", (b, L, H * P + 2 * G * N), act, dev)
    _check(conv_w, "conv_w", (cin, K), f32, dev)
    _check(conv_b, "conv_b", (cin,), f32, dev)
    _check(x_hist, "x_hist", (b, K - 1, cin), act, dev)
    _check(dt, "dt", (b, L, H), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    _check(A, "A", (H,), f32, dev)
    X = torch.empty((b, L, H, P), dtype=act, device=dev) if X is None else _check(X, "X", (b, L, H, P), act, dev)
    B = torch.empty((b, L, G, N), dtype=act, device=dev) if B is None else _check(B, "B", (b, L, G, N), act, dev)
    C = torch.empty((b, L, G, N), dtype=act, device=dev) if C is None else _check(C, "C", (b, L, G, N), act, dev)
    logdecay = torch.empty((b, L, H), dtype=f32, device=dev) if logdecay is None else \
        _check(logdecay, "logdecay", (b, L, H), f32, dev)
    dto = torch.empty((b, L, H), dtype=f32, device=dev) if dt_out else None
    _call("mb_ssd_prologue", _ptr(xBC), _ptr(conv_w), _ptr(conv_b), _ptr(x_hist), _ptr(dt), _ptr(dt_bias),
          _ptr(A), _ptr(X), _ptr(B), _ptr(C), _ptr(logdecay), _ptr(dto), b, L, H, P, G, N, K, code, _stream(dev))
    return (X, B, C, logdecay, dto) if dt_out else (X, B, C, logdecay)


def mb_mimo_ssd(X, logdecay, B, C, beta, gamma, theta=None, h0=None, *, X_prev=None, B_prev=None,
                chunk=0, Y=None, h_out=None, ws=None):
    """Mamba-3 MIMO.  X (batch, L, H, P, R), B, C (batch, L, H, N, R) in one
    dtype; X_prev (batch, H, P, R), B_prev (batch, H, N, R) or None; the rest
    as mb_trap_ssd.  Returns (Y, h_out)."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    b, L, H, P, R = X.shape
    N = B.shape[3]
    f32 = torch.float32
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, L, H), f32, dev)
    _check(B, "B", (b, L, H, N, R), dtype, dev)
    _check(C, "C", (b, L, H, N, R), dtype, dev)
    _check(theta, "theta", (b, L, H, N // 2), f32, dev)
    _check(h0, "h0", (b, H, N, P), f32, dev)
    _check(X_prev, "X_prev", (b, H, P, R), dtype, dev)
    _check(B_prev, "B_prev", (b, H, N, R), dtype, dev)
    Y = torch.empty((b, L, H, P, R), dtype=dtype, device=dev) if Y is None else \
        _check(Y, "Y", (b, L, H, P, R), dtype, dev)
    h_out = torch.empty((b, H, N, P), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, H, N, P), f32, dev)
    ws, nws = _workspace(MB_OP_MIMO_SSD, dev, ws, (b, L, H, P, 1, N, R, chunk))
    _call("mb_mimo_ssd", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma),
          _ptr(theta), _ptr(h0), _ptr(X_prev), _ptr(B_prev), _ptr(Y), _ptr(h_out), b, L, H, P, N, R, chunk,
          code, _ptr(ws), nws, _stream(dev))
    return Y, h_out


def mb_ssd_step(X, logdecay, B, C, h, *, beta=None, gamma=None, theta=None, X_prev=None, B_prev=None,
                Y=None, h_out=None):
    """Decode step of the SSD family (one token per sequence), state in the
    physical frame.  X, X_prev (batch, H, P[, R]); B, C, B_prev (batch, G, N[, R])
    in one dtype; logdecay, beta, gamma (batch, H), theta (batch, H, N/2) and
    h (batch, H, N, P) float32.  Mamba-2: beta, gamma, theta None.  With
    h_out=None the state is updated in place.  Returns (Y, h_out), Y shaped
    like X."""
    torch = _torch()
    dev = _device_of(X)
    dtype = X.dtype
    code = _dtype_code(X, "X")
    ranked = X.dim() == 4
    b, H, P = X.shape[:3]
    R = X.shape[3] if ranked else 1
    G, N = B.shape[1], B.shape[2]
    xs = (b, H, P, R) if ranked else (b, H, P)
    bs = (b, G, N, R) if ranked else (b, G, N)
    f32 = torch.float32
    _check(B, "B", bs, dtype, dev)
    _check(C, "C", bs, dtype, dev)
    _check(X_prev, "X_prev", xs, dtype, dev)
    _check(B_prev, "B_prev", bs, dtype, dev)
    for t, n in ((logdecay, "logdecay"), (beta, "beta"), (gamma, "gamma")):
        _check(t, n, (b, H), f32, dev)
    _check(theta, "theta", (b, H, N // 2), f32, dev)
    _check(h, "h", (b, H, N, P), f32, dev)
    h_out = h if h_out is None else _check(h_out, "h_out", (b, H, N, P), f32, dev)
    Y = torch.empty(xs, dtype=dtype, device=dev) if Y is None else _check(Y, "Y", xs, dtype, dev)
    _call("mb_ssd_step", _ptr(X), _ptr(logdecay), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma), _ptr(theta),
          _ptr(X_prev), _ptr(B_prev), _ptr(h), _ptr(h_out), _ptr(Y), b, H, P, G, N, R, code, _stream(dev))
    return Y, h_out


def mb_selective_scan_fused(x, conv_w, dt, A, B, C, D=None, h0=None, *, conv_b=None, dt_bias=None, z=None,
                            x_hist=None, y=None, h_out=None):
    """Mamba-1 scan with the block prologue and epilogue: causal conv1d + SiLU on
    x, softplus(dt + dt_bias), and the output gated by SiLU(z).  x, dt, z (batch,
    L, D), conv_w (D, K), conv_b, dt_bias, D (D,), A (D, N), B, C (batch, L, N),
    h0 (batch, D, N), x_hist (batch, K-1, D), all float32.  Returns (y, h_out)."""
    torch = _torch()
    dev = _device_of(x)
    f32 = torch.float32
    b, L, Dm = x.shape
    K = conv_w.shape[1]
    N = A.shape[1]
    _check(x, "x", (b, L, Dm), f32, dev)
    _check(conv_w, "conv_w", (Dm, K), f32, dev)
    for t, n in ((conv_b, "conv_b"), (dt_bias, "dt_bias"), (D, "D")):
        _check(t, n, (Dm,), f32, dev)
    _check(x_hist, "x_hist", (b, K - 1, Dm), f32, dev)
    _check(dt, "dt", (b, L, Dm), f32, dev)
    _check(z, "z", (b, L, Dm), f32, dev)
    _check(A, "A", (Dm, N), f32, dev)
    _check(B, "B", (b, L, N), f32, dev)
    _check(C, "C", (b, L, N), f32, dev)
    _check(h0, "h0", (b, Dm, N), f32, dev)
    y = torch.empty((b, L, Dm), dtype=f32, device=dev) if y is None else _check(y, "y", (b, L, Dm), f32, dev)
    h_out = torch.empty((b, Dm, N), dtype=f32, device=dev) if h_out is None else \
        _check(h_out, "h_out", (b, Dm, N), f32, dev)
    _call("mb_selective_scan_fused", _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(x_hist), _ptr(dt), _ptr(dt_bias),
          _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_out), b, L, Dm, N, K, MB_F32,
          _stream(dev))
    return y, h_out
