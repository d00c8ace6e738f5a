"""GPU parity of the Mamba-3 MIMO backward against the fp64 oracle's
back-propagation through the recurrence, through the C ABI."""
import zlib

import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-4
NAMES = ("dX", "dlogdecay", "dB", "dC", "dbeta", "dgamma", "dtheta", "dh0", "dX_prev", "dB_prev")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def make(case, b, L, H, P, N, R, rot=True, prev=True, dh=True, inp=None):
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    if inp is None:
        inp = wl.mimo_inputs(rng, b, L, H, P, N, R, h0_sd=0.1, rotate=rot)
    if not rot:
        inp["theta"] = None
    s = 1.0 / np.sqrt(N * R)
    inp["X_prev"] = rng.standard_normal((b, H, P, R)) * s if prev else None
    inp["B_prev"] = rng.standard_normal((b, H, N, R)) * s if prev else None
    inp["dY"] = rng.standard_normal((b, L, H, P, R))
    inp["dh_out"] = rng.standard_normal((b, H, N, P)) if dh else None
    host = {k: (np.asarray(v, np.float32).astype(np.float64) if v is not None else None) for k, v in inp.items()}
    dev = {k: (torch.from_numpy(v).float().cuda() if v is not None else None) for k, v in host.items()}
    return host, dev


def run(dev):
    return mb.mb_mimo_ssd_bwd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"], dev["dY"],
                              dev.get("theta"), dev.get("h0"), dev.get("dh_out"), X_prev=dev.get("X_prev"),
                              B_prev=dev.get("B_prev"))


def reference(oracle_mod, host):
    return oracle_mod.mimo_bwd(host["X"], host["logdecay"], host["B"], host["C"], host["beta"], host["gamma"],
                               host["dY"], host.get("theta"), host.get("h0"), host.get("dh_out"),
                               host.get("X_prev"), host.get("B_prev"))


def check(got, ref):
    errs = {n: rel_err(g, r) for n, g, r in zip(NAMES, got, ref) if g is not None}
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, "max|err|/max|ref| above %.0e: %s (all: %s)" % (TOL, bad, errs)


# (batch, L, H, P, N, R)
SHAPES = [(1, 1, 2, 32, 64, 4), (1, 30, 2, 64, 128, 4), (2, 50, 2, 32, 64, 2), (1, 40, 3, 64, 64, 1),
          (1, 23, 2, 32, 128, 8), (1, 200, 2, 64, 128, 4), (1, 9, 1, 32, 64, 16)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mimo_bwd_shapes(oracle_mod, shape):
    host, dev = make(shape, *shape)
    check(run(dev), reference(oracle_mod, host))


@pytest.mark.parametrize("rot,prev,dh", [(False, True, True), (True, False, False)])
def test_mimo_bwd_options(oracle_mod, rot, prev, dh):
    host, dev = make(("opt", rot, prev, dh), 2, 33, 2, 64, 128, 4, rot=rot, prev=prev, dh=dh)
    check(run(dev), reference(oracle_mod, host))


@pytest.mark.slow
def test_mimo_bwd_block_workload_full(oracle_mod):
    """batch 2, L 8192, H 16, P 64, N 128, R 4 -- the MIMO block configuration."""
    host, dev = make("full", 2, 8192, 16, 64, 128, 4, inp=wl.mimo_block())
    got = run(dev)
    torch.cuda.synchronize()
    check(got, reference(oracle_mod, host))
