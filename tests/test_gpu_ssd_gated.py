"""GPU parity of the Mamba-2 SSD with the block's output side fused into the
store (skip term D[h] X and SiLU(z) gate) against the fp64 oracle (ssd_gated),
through the C ABI: fp32 (the wave-specialised walk) and bf16 (the bf16 walk,
and the general walk when N is not a multiple of 8)."""
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


def _run(oracle_mod, shape, dtype, seed, use_D=True, use_z=True, inp=None):
    b, L, H, P, N, G = shape
    rng = np.random.default_rng(seed)
    if inp is None:
        inp = wl.ssd_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.05)
    D = rng.standard_normal(H) if use_D else None
    z = rng.standard_normal((b, L, H, P)) if use_z else None
    dev, ref = prepare(inp, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Dd = None if D is None else torch.from_numpy(D).float().cuda()
    zd = None if z is None else torch.from_numpy(z).to(tdt).cuda()
    Y, h = mb.mb_ssd_chunked_gated(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h0"], D=Dd, z=zd)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.ssd_gated(**ref, D=None if Dd is None else Dd.double().cpu().numpy(),
                                  z=None if zd is None else zd.double().cpu().numpy())
    return Y, h, Yr, hr


SHAPES = [  # batch, L, H, P, N, G
    (1, 1, 1, 16, 8, 1), (2, 130, 4, 16, 128, 2), (1, 333, 3, 48, 64, 1), (2, 700, 2, 128, 64, 1),
    (1, 2000, 4, 64, 128, 1), (1, 90, 2, 16, 12, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_gated_shapes(oracle_mod, shape, dtype):
    Y, h, Yr, hr = _run(oracle_mod, shape, dtype, seed=sum(shape))
    assert Y.dtype == (torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


@pytest.mark.parametrize("parts", [(True, False), (False, True)], ids=["D-only", "z-only"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_gated_one_part(oracle_mod, parts, dtype):
    Y, h, Yr, hr = _run(oracle_mod, (2, 300, 3, 64, 128, 1), dtype, seed=5, use_D=parts[0], use_z=parts[1])
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


def test_ssd_gated_without_parts_is_the_plain_call():
    dev, _ = prepare(wl.ssd_inputs(np.random.default_rng(6), 2, 257, 3, 64, 128), "f32")
    Yg, hg = mb.mb_ssd_chunked_gated(dev["X"], dev["logdecay"], dev["B"], dev["C"])
    Yp, hp = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"])
    assert torch.equal(Yg, Yp) and torch.equal(hg, hp)


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_gated_block_workload_full(oracle_mod, dtype):
    """batch 4, L 4096, H 24, P 64, N 128, G 1 with D and z."""
    Y, h, Yr, hr = _run(oracle_mod, (4, 4096, 24, 64, 128, 1), dtype, seed=119, inp=wl.ssd_block())
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")
