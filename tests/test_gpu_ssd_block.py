"""GPU parity of the Mamba-2 layer around its scan in one call (mb_ssd_block:
conv1d + SiLU over xBC, softplus of dt, the chunked SSD, the skip term on the
convolved x and the SiLU(z) gate, with X, B and C never materialised as
tensors of their own) against the fp64 oracle's ssd_block, through the C ABI."""
import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import assert_close, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _inputs(shape, seed, opt=True, parts=True):
    b, L, H, P, G, N, K = shape
    rng = np.random.default_rng(seed)
    i = wl.m2_prologue_inputs(rng, b, L, H, P, G, N, K, hist=opt)
    if not opt:
        i["conv_b"], i["dt_bias"] = None, None
    i["D"] = rng.standard_normal(H) if parts else None
    i["z"] = rng.standard_normal((b, L, H, P)) if parts else None
    i["h0"] = 0.1 * rng.standard_normal((b, H, N, P)) if opt else None
    return i


ACTS = ("xBC", "x_hist", "z")


def _run(oracle_mod, shape, dtype, i):
    b, L, H, P, G, N, K = shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {k: (None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(tdt if k in ACTS else torch.float32)
             .cuda()) for k, v in i.items()}
    r = {k: (None if v is None else t.double().cpu().numpy()) for (k, v), t in zip(i.items(), d.values())}
    Y, h = mb.mb_ssd_block(d["xBC"], d["conv_w"], d["dt"], d["A"], H, P, G, N, conv_b=d["conv_b"],
                           dt_bias=d["dt_bias"], x_hist=d["x_hist"], D=d["D"], z=d["z"], h0=d["h0"])
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.ssd_block(**r, H=H, P=P, G=G, N=N)
    return Y, h, Yr, hr


SHAPES = [  # batch, L, H, P, G, N, K
    (1, 1, 1, 16, 1, 8, 4), (2, 130, 3, 32, 1, 64, 4), (1, 333, 2, 64, 2, 128, 3), (2, 700, 2, 128, 1, 64, 2),
    (1, 2000, 4, 64, 1, 128, 4),   # several sequence segments
    (2, 150, 2, 32, 1, 96, 1)]     # state rows padded to 128, one tap


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_block_shapes(oracle_mod, shape, dtype):
    Y, h, Yr, hr = _run(oracle_mod, shape, dtype, _inputs(shape, sum(shape)))
    assert Y.dtype == (torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_block_without_optional_parts(oracle_mod, dtype):
    shape = (2, 300, 3, 64, 1, 128, 4)
    Y, h, Yr, hr = _run(oracle_mod, shape, dtype, _inputs(shape, 3, opt=False, parts=False))
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


def test_ssd_block_fp32_any_state_size(oracle_mod):
    shape = (1, 90, 2, 16, 1, 12, 4)   # N not a multiple of 8
    Y, h, Yr, hr = _run(oracle_mod, shape, "f32", _inputs(shape, 4))
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


def test_ssd_block_split_chains_through_history_and_state(oracle_mod):
    shape = (2, 500, 2, 64, 1, 128, 4)
    b, L, H, P, G, N, K = shape
    i = _inputs(shape, 5)
    d = {k: (None if v is None else torch.from_numpy(np.ascontiguousarray(v)).float().cuda()) for k, v in i.items()}
    s = 229
    cut = lambda t, sl: None if t is None else t[:, sl].contiguous()
    kw = dict(conv_b=d["conv_b"], dt_bias=d["dt_bias"], D=d["D"])
    Ya, ha = mb.mb_ssd_block(cut(d["xBC"], slice(0, s)), d["conv_w"], cut(d["dt"], slice(0, s)), d["A"], H, P, G, N,
                             x_hist=d["x_hist"], z=cut(d["z"], slice(0, s)), h0=d["h0"], **kw)
    Yb, hb = mb.mb_ssd_block(cut(d["xBC"], slice(s, None)), d["conv_w"], cut(d["dt"], slice(s, None)), d["A"], H, P,
                             G, N, x_hist=d["xBC"][:, s - 3:s].contiguous(), z=cut(d["z"], slice(s, None)), h0=ha,
                             **kw)
    torch.cuda.synchronize()
    r = {k: (None if v is None else np.asarray(v, np.float32).astype(np.float64)) for k, v in i.items()}
    Yr, hr = oracle_mod.ssd_block(**r, H=H, P=P, G=G, N=N)
    assert_close(torch.cat([Ya, Yb], 1), Yr, "f32", "Y")
    assert_close(hb, hr, "f32", "h")


def test_ssd_block_rejects_bf16_state_sizes_off_eight():
    xBC = torch.zeros(1, 4, 16 + 2 * 12, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16 + 2 * 12, 4, device="cuda")
    dt = torch.zeros(1, 4, 1, device="cuda")
    A = -torch.ones(1, device="cuda")
    with pytest.raises(mb.MBError):
        mb.mb_ssd_block(xBC, w, dt, A, 1, 16, 1, 12)


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_block_workload_full(oracle_mod, dtype):
    """The Mamba-2 block shape: batch 4, L 4096, H 24, P 64, G 1, N 128, K 4."""
    i = wl.m2_block_full()
    shape = (4, 4096, 24, 64, 1, 128, 4)
    Y, h, Yr, hr = _run(oracle_mod, shape, dtype, i)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")
