"""GPU parity of the Mamba-3 SISO layer with its output epilogue fused into the
scan's store (skip term D[h] X, then the SiLU(z) gate) against the fp64 oracle,
through the C ABI; without D and z the call is the plain SISO scan, bit for bit."""
import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import assert_close, prepare, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


SHAPES = [  # batch, L, H, P, N, G
    (1, 1, 1, 16, 4, 1), (2, 130, 3, 32, 64, 1), (1, 333, 4, 16, 32, 2),
    (1, 2000, 2, 64, 128, 1)]    # several sequence segments


def _inputs(shape, seed, dtype, rotate):
    b, L, H, P, N, G = shape
    rng = np.random.default_rng(seed)
    inp = wl.trap_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.05, rotate=rotate)
    D = rng.standard_normal(H)
    z = rng.standard_normal((b, L, H, P)) * 2.0
    dev, ref = prepare(inp, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    zt = torch.from_numpy(z).to(tdt)
    Dt = torch.from_numpy(D).to(torch.float32)
    return dev, ref, Dt.cuda(), Dt.to(torch.float64).numpy(), zt.cuda(), zt.to(torch.float64).numpy()


def _call(dev, D=None, z=None):
    return mb.mb_trap_ssd_gated(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                                dev["theta"], dev["h0"], D=D, z=z, X_prev=dev.get("X_prev"), B_prev=dev.get("B_prev"))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["D", "z", "Dz"])
def test_gated_parity(oracle_mod, shape, dtype, mode):
    rotate = shape[1] != 333
    dev, ref, Dd, Dr, zd, zr = _inputs(shape, 7 + len(mode) + shape[1], dtype, rotate)
    useD, usez = "D" in mode, "z" in mode
    Y, h = _call(dev, Dd if useD else None, zd if usez else None)
    Yr, hr = oracle_mod.trap_gated(**ref, D=Dr if useD else None, z=zr if usez else None)
    assert Y.dtype == dev["X"].dtype
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, "f32", "h_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_without_epilogue_is_plain_scan(dtype):
    dev, _, _, _, _, _ = _inputs((2, 130, 3, 32, 64, 1), 19, dtype, True)
    Y, h = _call(dev)
    Y0, h0 = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                            dev["theta"], dev["h0"], X_prev=dev.get("X_prev"), B_prev=dev.get("B_prev"))
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0) and torch.equal(h, h0)


def test_gated_zero_gate_and_empty(oracle_mod):
    dev, _, Dd, _, zd, _ = _inputs((1, 130, 2, 16, 32, 1), 23, "f32", True)
    Y, h = _call(dev, Dd, torch.zeros_like(zd))
    _, h0 = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                           dev["theta"], dev["h0"], X_prev=dev.get("X_prev"), B_prev=dev.get("B_prev"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(Y).item() == 0 and torch.equal(h, h0)
    e = {k: (v[:, :0].contiguous() if (v is not None and v.dim() >= 3 and k not in ("h0", "X_prev", "B_prev"))
             else v) for k, v in dev.items()}
    Y, h = _call(e, Dd, zd[:, :0].contiguous())
    assert Y.shape[1] == 0 and torch.equal(h, dev["h0"])


@pytest.mark.slow
def test_gated_block_workload_full(oracle_mod):
    """batch 4, L 4096, H 24, P 64, N 128 with rotations, skip term and gate -- the
    configuration measured beside the step."""
    inp = wl.siso_gated()
    D, z = inp.pop("D"), inp.pop("z")
    dev, ref = prepare(inp, "f32")
    Dd = torch.from_numpy(D).float().cuda()
    zd = torch.from_numpy(z).float().cuda()
    Y, h = mb.mb_trap_ssd_gated(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                                dev["theta"], None, D=Dd, z=zd)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.trap_gated(**ref, D=Dd.double().cpu().numpy(), z=zd.double().cpu().numpy())
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
