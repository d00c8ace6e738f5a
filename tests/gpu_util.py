"""Helpers for the GPU parity tests: move seeded numpy inputs to the device in
the run dtype, hand the oracle exactly the values the device sees, and measure
the error the way the tolerances are stated: max|gpu - ref| / max|ref|."""
import numpy as np
import pytest
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}
# Names of the "activation" tensors that take the run dtype; all others stay fp32.
ACT = {"x", "dt", "B", "C", "X", "X_prev", "B_prev"}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def prepare(inp, dtype):
    """Return (device tensors, fp64 arrays the oracle should see)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev, ref = {}, {}
    for k, v in inp.items():
        if v is None:
            dev[k], ref[k] = None, None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        t = t.to(tdt if k in ACT else torch.float32)
        ref[k] = t.to(torch.float64).numpy()
        dev[k] = t.cuda()
    return dev, ref


def rel_err(got, ref):
    got = got.detach().to(torch.float64).cpu().numpy() if isinstance(got, torch.Tensor) else got
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def assert_close(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    assert e <= TOL[dtype], "%s: max|err|/max|ref| = %.3e > %.0e" % (what, e, TOL[dtype])
    return e


def assert_close_slices(got, ref, dtype, what, axes):
    """The tolerance per slice (e.g. per batch row and head): max|gpu - ref|
    over the slice divided by the slice's own max|ref|, floored at 1e-2 of the
    whole tensor's, so a slice whose output is small next to the others is
    held to its own scale."""
    g = got.detach().to(torch.float64).cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "%s: non-finite output" % what
    other = tuple(i for i in range(r.ndim) if i not in axes)
    den = np.max(np.abs(r), axis=other)
    num = np.max(np.abs(g - r), axis=other)
    floor = 1e-2 * float(np.max(np.abs(r)))
    if floor == 0.0:
        assert float(np.max(num)) == 0.0, "%s: output should be exactly zero" % what
        return 0.0
    e = num / np.maximum(den, floor)
    k = np.unravel_index(int(np.argmax(e)), e.shape)
    assert e[k] <= TOL[dtype], "%s: slice %s max|err|/max|ref| = %.3e > %.0e" % (what, k, e[k], TOL[dtype])
    return float(e[k])
