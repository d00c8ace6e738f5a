"""GPU parity of the Mamba-2 SSD backward (dX, dlogdecay, dB, dC, dh0) against
the fp64 oracle's back-propagation through the recurrence, through the C ABI."""
import zlib

import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import rel_err, require_gpu

pytestmark = pytest.mark.gpu

# fp32 throughout; the gradients sum over up to L steps and N x P state
# elements, so the bar is the forward's 1e-4 of the largest magnitude
TOL = 1e-4
NAMES = ("dX", "dlogdecay", "dB", "dC", "dh0")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _seed(case):
    return zlib.crc32(repr(case).encode())


def make(case, b, L, H, P, N, G, h0=True, dh=True):
    rng = np.random.default_rng(_seed(case))
    inp = wl.ssd_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.3 if h0 else 0.0)
    dY = rng.standard_normal((b, L, H, P))
    dhv = rng.standard_normal((b, H, N, P)) if dh else None
    host = {k: (np.asarray(v, np.float32).astype(np.float64) if v is not None else None) for k, v in inp.items()}
    host["dY"] = dY.astype(np.float32).astype(np.float64)
    host["dh_out"] = dhv.astype(np.float32).astype(np.float64) if dhv is not None else None
    dev = {k: (torch.from_numpy(v).float().cuda() if v is not None else None) for k, v in host.items()}
    return host, dev


def run(dev, **kw):
    return mb.mb_ssd_chunked_bwd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["dY"], dev.get("h0"),
                                 dev.get("dh_out"), **kw)


def reference(oracle_mod, host):
    return oracle_mod.ssd_bwd(host["X"], host["logdecay"], host["B"], host["C"], host["dY"], host.get("h0"),
                              host.get("dh_out"))


def check(got, ref):
    errs = {}
    for n, g, r in zip(NAMES, got, ref):
        errs[n] = rel_err(g, r)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, "max|err|/max|ref| above %.0e: %s (all: %s)" % (TOL, bad, errs)


# (batch, L, H, P, N, G): one step, one chunk, ragged tails, several chunks,
# G = 1 (all heads share B, C), G = H, grouped heads
SHAPES = [(1, 1, 2, 32, 64, 1), (1, 64, 1, 32, 64, 1), (1, 63, 2, 64, 128, 1), (2, 65, 2, 64, 64, 2),
          (2, 150, 4, 64, 128, 2), (1, 200, 3, 32, 64, 3), (2, 300, 8, 32, 128, 1), (1, 257, 6, 64, 128, 3)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes(oracle_mod, shape):
    host, dev = make(shape, *shape)
    got = run(dev)
    check(got, reference(oracle_mod, host))


@pytest.mark.parametrize("h0,dh", [(False, False), (True, False), (False, True)])
def test_bwd_optional_states(oracle_mod, h0, dh):
    shape = (2, 130, 2, 64, 128, 1)
    host, dev = make(("opt", h0, dh), *shape, h0=h0, dh=dh)
    got = run(dev)
    check(got, reference(oracle_mod, host))


def test_bwd_zero_length_passes_state_gradient():
    host, dev = make("zero", 2, 1, 2, 32, 64, 1)
    for k in ("X", "logdecay", "B", "C", "dY"):
        dev[k] = dev[k][:, :0].contiguous()
    got = run(dev)
    assert got[0].shape == (2, 0, 2, 32)
    assert torch.equal(got[4], dev["dh_out"])


def test_bwd_deterministic():
    host, dev = make("det", 1, 190, 4, 64, 128, 2)
    a = run(dev)
    b = run(dev)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_matches_forward_directional_derivative():
    """<grad, v> equals the central difference of the GPU forward loss along v
    (fp32 forward, so a loose bar): the backward is the forward's derivative."""
    host, dev = make("dir", 1, 128, 2, 64, 128, 1)
    got = run(dev)
    rng = np.random.default_rng(3)
    names = ("X", "logdecay", "B", "C", "h0")

    def loss(d):
        Y, h = mb.mb_ssd_chunked(d["X"], d["logdecay"], d["B"], d["C"], d["h0"])
        return float((Y.double() * dev["dY"].double()).sum() + (h.double() * dev["dh_out"].double()).sum())
    for name, g in zip(names, got):
        v = torch.from_numpy(rng.standard_normal(tuple(dev[name].shape))).float().cuda()
        eps = 1e-2
        up = loss(dict(dev, **{name: dev[name] + eps * v}))
        dn = loss(dict(dev, **{name: dev[name] - eps * v}))
        fd = (up - dn) / (2 * eps)
        an = float((g.double() * v.double()).sum())
        assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.slow
def test_bwd_block_workload_full(oracle_mod):
    """batch 4, L 4096, H 24, P 64, N 128, G 1 -- the SSD block configuration."""
    host, dev = make("full", 4, 4096, 24, 64, 128, 1)
    got = run(dev)
    torch.cuda.synchronize()
    check(got, reference(oracle_mod, host))
