"""GPU parity of the Mamba-3 SISO layer with both ends of its block fused into
the scan -- BCNorm + bias on the B, C rows before the rotations, skip term and
SiLU gate at the store -- against the fp64 oracle, through the C ABI."""
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
    (1, 150, 2, 32, 96, 1),      # state rows padded to 128
    (1, 2000, 2, 64, 128, 1)]    # several sequence segments


def _params(rng, H, N, full):
    """Norm weights around 1, biases, skip weights, gate; None for the parts a
    case leaves out."""
    nb = 1.0 + 0.3 * rng.standard_normal(N)
    nc = 1.0 + 0.3 * rng.standard_normal(N)
    bb = 0.5 * rng.standard_normal((H, N))
    bc = 0.5 * rng.standard_normal((H, N))
    D = rng.standard_normal(H)
    if not full:
        nb, bc, D = None, None, None
    return dict(normB_w=nb, normC_w=nc, biasB=bb, biasC=bc, D=D)


def _run(oracle_mod, shape, dtype, rotate, full, prev, seed, eps=1e-5):
    b, L, H, P, N, G = shape
    rng = np.random.default_rng(seed)
    inp = wl.trap_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.05, rotate=rotate)
    if prev:
        s = 1.0 / np.sqrt(N)
        inp["X_prev"] = rng.standard_normal((b, H, P)) * s
        inp["B_prev"] = rng.standard_normal((b, G, N)) * s
    pr = _params(rng, H, N, full)
    z = rng.standard_normal((b, L, H, P)) * 2.0 if full else None
    dev, ref = prepare(inp, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pd = {k: (None if v is None else torch.from_numpy(v).float().cuda()) for k, v in pr.items()}
    pr = {k: (None if v is None else t.double().cpu().numpy()) for (k, v), t in zip(pr.items(), pd.values())}
    zd = None if z is None else torch.from_numpy(z).to(tdt).cuda()
    zr = None if zd is None else zd.double().cpu().numpy()
    Y, h = mb.mb_trap_ssd_block(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                                dev["theta"], dev["h0"], X_prev=dev.get("X_prev"), B_prev=dev.get("B_prev"),
                                eps=eps, z=zd, **pd)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.trap_block(**ref, eps=eps, z=zr, **pr)
    return Y, h, Yr, hr


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("full", [True, False], ids=["all", "part"])
def test_block_parity(oracle_mod, shape, dtype, full):
    rotate = shape[1] != 333
    Y, h, Yr, hr = _run(oracle_mod, shape, dtype, rotate, full, prev=shape[1] == 130, seed=31 + shape[1] + full)
    assert Y.dtype == (torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, "f32", "h_out")


def test_block_large_eps_and_prev_only_row(oracle_mod):
    """eps comparable to the rows' mean square (the norm no longer unit), and a
    call whose only step is preceded by the previous token."""
    Y, h, Yr, hr = _run(oracle_mod, (1, 90, 2, 16, 16, 1), "f32", True, True, prev=False, seed=5, eps=0.05)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h_out")
    Y, h, Yr, hr = _run(oracle_mod, (2, 1, 2, 16, 16, 1), "f32", True, True, prev=True, seed=6)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h_out")


@pytest.mark.slow
def test_block_workload_full(oracle_mod):
    """batch 4, L 4096, H 24, P 64, N 128 with rotations and every parameter --
    the configuration measured beside the step."""
    inp = wl.siso_block_full()
    extra = {k: inp.pop(k) for k in ("normB_w", "normC_w", "biasB", "biasC", "D", "z")}
    dev, ref = prepare(inp, "f32")
    ed = {k: torch.from_numpy(v).float().cuda() for k, v in extra.items()}
    er = {k: t.double().cpu().numpy() for k, t in ed.items()}
    Y, h = mb.mb_trap_ssd_block(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                                dev["theta"], None, **ed)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.trap_block(**ref, **er)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
