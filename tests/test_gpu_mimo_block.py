"""GPU parity of the Mamba-3 MIMO layer with both ends of its block fused into
the scan -- BCNorm + bias on every rank row of B and C before the rotations,
skip term and SiLU gate per rank at the store -- against the fp64 oracle
(mimo_block), through the C ABI."""
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


PARAMS = ("normB_w", "normC_w", "biasB", "biasC", "D")


def _run(oracle_mod, shape, dtype="f32", rotate=True, prev=False, drop=(), seed=0, eps=1e-5, split=None):
    b, L, H, P, N, R = shape
    inp = wl.mimo_block_inputs(np.random.default_rng(seed), b, L, H, P, N, R, h0_sd=0.05, rotate=rotate,
                               prev=prev)
    for k in drop:
        inp[k] = None
    z = inp.pop("z")
    pars = {k: inp.pop(k) for k in PARAMS}
    dev, ref = prepare(inp, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pd = {k: (None if v is None else torch.from_numpy(v).float().cuda()) for k, v in pars.items()}
    pr = {k: (None if v is None else t.double().cpu().numpy()) for (k, v), t in zip(pars.items(), pd.values())}
    zd = None if (z is None or "z" in drop) else torch.from_numpy(z).to(tdt).cuda()
    zr = None if zd is None else zd.double().cpu().numpy()
    Yr, hr = oracle_mod.mimo_block(**ref, eps=eps, z=zr, **pr)
    kw = dict(eps=eps, **pd)
    if split is None:
        Y, h = mb.mb_mimo_ssd_block(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                                    dev["theta"], dev["h0"], X_prev=dev.get("X_prev"), B_prev=dev.get("B_prev"),
                                    z=zd, **kw)
    else:
        # two calls chained through the state and the raw previous token
        s = split
        cut = lambda t, sl: None if t is None else t[:, sl].contiguous()
        seqk = ("X", "logdecay", "B", "C", "beta", "gamma", "theta")
        A = {k: cut(dev[k], slice(0, s)) for k in seqk}
        Bp = {k: cut(dev[k], slice(s, None)) for k in seqk}
        Ya, ha = mb.mb_mimo_ssd_block(A["X"], A["logdecay"], A["B"], A["C"], A["beta"], A["gamma"], A["theta"],
                                      dev["h0"], X_prev=dev.get("X_prev"), B_prev=dev.get("B_prev"),
                                      z=cut(zd, slice(0, s)), **kw)
        Yb, h = mb.mb_mimo_ssd_block(Bp["X"], Bp["logdecay"], Bp["B"], Bp["C"], Bp["beta"], Bp["gamma"],
                                     Bp["theta"], ha, X_prev=dev["X"][:, s - 1].contiguous(),
                                     B_prev=dev["B"][:, s - 1].contiguous(), z=cut(zd, slice(s, None)), **kw)
        Y = torch.cat([Ya, Yb], 1)
    torch.cuda.synchronize()
    return Y, h, Yr, hr


SHAPES = [  # batch, L, H, P, N, R
    (1, 1, 1, 16, 4, 4), (2, 130, 3, 32, 64, 4), (1, 333, 2, 64, 128, 4),
    (1, 150, 2, 32, 96, 4),        # state rows padded to 128
    (1, 2000, 2, 64, 128, 4),      # several sequence segments
    (2, 200, 3, 32, 64, 1),        # rank 1 (the SISO walk on per-head rows)
    (2, 150, 2, 32, 64, 2), (1, 1300, 2, 64, 128, 2),     # rank 2 (four columns of one rank per lane)
    (2, 120, 2, 32, 64, 8), (1, 700, 2, 64, 128, 8),      # rank 8 (rank rows)
    (1, 90, 3, 16, 32, 16), (1, 1500, 2, 64, 128, 16)]    # rank 16


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("rotate", [True, False])
def test_mimo_block_shapes(oracle_mod, shape, rotate):
    Y, h, Yr, hr = _run(oracle_mod, shape, rotate=rotate, seed=sum(shape) + rotate)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.parametrize("drop", [("D",), ("z",), ("D", "z"), ("normB_w", "biasC"), ("biasB", "normC_w", "z")],
                         ids=lambda d: "-".join(d))
@pytest.mark.parametrize("R", [4, 2])
def test_mimo_block_optional_parts(oracle_mod, drop, R):
    Y, h, Yr, hr = _run(oracle_mod, (2, 300, 2, 64, 128, R), drop=drop, seed=len(drop) + R)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.parametrize("R", [4, 2])
def test_mimo_block_previous_token_and_split(oracle_mod, R):
    shape = (2, 500, 2, 64, 128, R)
    Y, h, Yr, hr = _run(oracle_mod, shape, prev=True, seed=7)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    Y, h, Yr, hr = _run(oracle_mod, shape, prev=True, seed=7, split=131)
    assert_close(Y, Yr, "f32", "Y (split)")
    assert_close(h, hr, "f32", "h (split)")


@pytest.mark.parametrize("R", [4, 2, 16])
def test_mimo_block_bf16(oracle_mod, R):
    Y, h, Yr, hr = _run(oracle_mod, (2, 400, 2, 64, 128, R), dtype="bf16", seed=9 + R)
    assert Y.dtype == torch.bfloat16
    assert_close(Y, Yr, "bf16", "Y")
    assert_close(h, hr, "bf16", "h")


def test_mimo_block_rejects_unsupported_rank():
    X = torch.zeros(1, 4, 1, 16, 3, device="cuda")
    B = torch.zeros(1, 4, 1, 8, 3, device="cuda")
    s = torch.zeros(1, 4, 1, device="cuda")
    with pytest.raises(mb.MBError):
        mb.mb_mimo_ssd_block(X, s, B, B, s, s)


@pytest.mark.slow
def test_mimo_block_workload_full(oracle_mod):
    """The MIMO block shape (batch 2, L 8192, H 16, P 64, N 128, R 4) with every
    part of both block ends."""
    inp = wl.mimo_block_full()
    z = inp.pop("z")
    pars = {k: inp.pop(k) for k in PARAMS}
    dev, ref = prepare(inp, "f32")
    pd = {k: torch.from_numpy(v).float().cuda() for k, v in pars.items()}
    zd = torch.from_numpy(z).float().cuda()
    Y, h = mb.mb_mimo_ssd_block(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                                dev["theta"], None, z=zd, **pd)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.mimo_block(**ref, z=z.astype(np.float32).astype(np.float64),
                                   **{k: v.astype(np.float32).astype(np.float64) for k, v in pars.items()})
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
