"""GPU parity of the Mamba-3 SISO backward (X, logdecay, B, C, beta, gamma,
theta, h0 and the previous token) against the fp64 oracle's back-propagation
through the recurrence, through the C ABI."""
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


def make(case, b, L, H, P, N, G, rot=True, prev=True, dh=True, inp=None):
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    if inp is None:
        inp = wl.trap_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.1)
    if not rot:
        inp["theta"] = None
    inp["X_prev"] = rng.standard_normal((b, H, P)) / np.sqrt(N) if prev else None
    inp["B_prev"] = rng.standard_normal((b, G, N)) / np.sqrt(N) if prev else None
    inp["dY"] = rng.standard_normal((b, L, H, P))
    inp["dh_out"] = rng.standard_normal((b, H, N, P)) if dh else None
    host = {k: (np.asarray(v, np.float32).astype(np.float64) if v is not None else None) for k, v in inp.items()}
    dev = {k: (torch.from_numpy(v).float().cuda() if v is not None else None) for k, v in host.items()}
    return host, dev


def run(dev):
    return mb.mb_trap_ssd_bwd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"], dev["dY"],
                              dev.get("theta"), dev.get("h0"), dev.get("dh_out"), X_prev=dev.get("X_prev"),
                              B_prev=dev.get("B_prev"))


def reference(oracle_mod, host):
    return oracle_mod.trap_bwd(host["X"], host["logdecay"], host["B"], host["C"], host["beta"], host["gamma"],
                               host["dY"], host.get("theta"), host.get("h0"), host.get("dh_out"),
                               host.get("X_prev"), host.get("B_prev"))


def check(got, ref):
    errs = {}
    for n, g, r in zip(NAMES, got, ref):
        if g is None:
            continue
        errs[n] = rel_err(g, r)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, "max|err|/max|ref| above %.0e: %s (all: %s)" % (TOL, bad, errs)


SHAPES = [(1, 1, 2, 32, 64, 1), (1, 64, 2, 64, 128, 1), (2, 100, 4, 32, 64, 2), (1, 150, 3, 64, 128, 3),
          (2, 257, 2, 64, 64, 1), (1, 1000, 2, 32, 128, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_trap_bwd_shapes(oracle_mod, shape):
    host, dev = make(shape, *shape)
    check(run(dev), reference(oracle_mod, host))


@pytest.mark.parametrize("rot,prev,dh", [(False, True, True), (True, False, True), (True, True, False),
                                         (False, False, False)])
def test_trap_bwd_options(oracle_mod, rot, prev, dh):
    host, dev = make(("opt", rot, prev, dh), 2, 130, 2, 64, 128, 1, rot=rot, prev=prev, dh=dh)
    got = run(dev)
    if not rot:
        assert got[6] is None
    if not prev:
        assert got[8] is None and got[9] is None
    check(got, reference(oracle_mod, host))


def test_trap_bwd_deterministic():
    host, dev = make("det", 1, 200, 4, 64, 128, 2)
    a = run(dev)
    b = run(dev)
    for x, y in zip(a, b):
        if x is not None:
            assert torch.equal(x, y)


@pytest.mark.slow
def test_trap_bwd_block_workload_full(oracle_mod):
    """batch 4, L 4096, H 24, P 64, N 128, G 1 -- the SISO block configuration."""
    host, dev = make("full", 4, 4096, 24, 64, 128, 1, inp=wl.siso_block())
    got = run(dev)
    torch.cuda.synchronize()
    check(got, reference(oracle_mod, host))
