"""GPU parity of the Mamba-1 scan with the block prologue and epilogue fused
around it (causal conv1d + SiLU on x, softplus(dt + dt_bias), output gated by
SiLU(z)) against the fp64 oracle of the same block, through the C ABI."""
import zlib

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


def _seed(case):
    return zlib.crc32(repr(case).encode())


def to_dev(inp):
    dev, ref = {}, {}
    for k, v in inp.items():
        if v is None:
            dev[k] = ref[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float32)
        ref[k] = t.to(torch.float64).numpy()
        dev[k] = t.cuda()
    return dev, ref


def run(dev, **kw):
    return mb.mb_selective_scan_fused(dev["x"], dev["conv_w"], dev["dt"], dev["A"], dev["B"], dev["C"],
                                      dev.get("D"), dev.get("h0"), conv_b=dev.get("conv_b"),
                                      dt_bias=dev.get("dt_bias"), z=dev.get("z"), x_hist=dev.get("x_hist"),
                                      **kw)


def check(oracle_mod, dev, ref):
    y, h = run(dev)
    yr, hr = oracle_mod.m1_block(**ref)
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


# (batch, L, D, N, K): one step, ragged tiles (L not a multiple of 32), D not a
# multiple of 4 (the 4-byte copies) or of 64 (a partial channel group)
SHAPES = [(1, 1, 1, 4, 4), (2, 17, 5, 8, 3), (1, 64, 16, 16, 4), (2, 130, 33, 16, 4), (3, 77, 40, 4, 2),
          (1, 95, 7, 4, 1), (2, 300, 64, 16, 4), (2, 1000, 48, 8, 4), (1, 161, 52, 16, 3), (2, 33, 130, 16, 4),
          (1, 3, 12, 8, 4)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_shapes(oracle_mod, shape):
    b, L, D, N, K = shape
    inp = wl.m1_block_inputs(np.random.default_rng(_seed(shape)), b, L, D, N, K, h0_sd=0.3, hist=True)
    check(oracle_mod, *to_dev(inp))


@pytest.mark.parametrize("drop", ["z", "conv_b", "dt_bias", "D", "h0", "x_hist", "all"])
def test_fused_optional_inputs(oracle_mod, drop):
    """Each optional input absent: no gate, no biases, no skip, zero state, zero history."""
    inp = wl.m1_block_inputs(np.random.default_rng(_seed(("opt", drop))), 2, 90, 36, 16, 4, h0_sd=0.3, hist=True)
    for k in (["z", "conv_b", "dt_bias", "D", "h0", "x_hist"] if drop == "all" else [drop]):
        inp[k] = None
    check(oracle_mod, *to_dev(inp))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("N", [4, 8, 16])
def test_fused_split_sequence_chains(oracle_mod, K, N):
    """A sequence split across two calls, the second given the first's final state
    and its last K-1 raw inputs, gives the one-call result."""
    b, L, D, L1 = 2, 150, 40, 61
    inp = wl.m1_block_inputs(np.random.default_rng(_seed(("split", K, N))), b, L, D, N, K, h0_sd=0.2)
    dev, ref = to_dev(inp)
    yr, hr = oracle_mod.m1_block(**ref)
    first = dict(dev)
    second = dict(dev)
    for k in ("x", "dt", "B", "C", "z"):
        first[k] = dev[k][:, :L1].contiguous()
        second[k] = dev[k][:, L1:].contiguous()
    y1, h1 = run(first)
    second["h0"] = h1
    second["x_hist"] = dev["x"][:, L1 - (K - 1):L1].contiguous() if K > 1 else None
    y2, h2 = run(second)
    assert_close(torch.cat([y1, y2], 1), yr, "f32", "y")
    assert_close(h2, hr, "f32", "h")


def test_fused_state_in_place(oracle_mod):
    inp = wl.m1_block_inputs(np.random.default_rng(5), 2, 70, 20, 8, 4, h0_sd=0.4, hist=True)
    dev, ref = to_dev(inp)
    yr, hr = oracle_mod.m1_block(**ref)
    h = dev["h0"].clone()
    dev["h0"] = h
    y, h_out = run(dev, h_out=h)
    assert h_out.data_ptr() == h.data_ptr()
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


def test_fused_large_step_sizes(oracle_mod):
    """Pre-activations far out on both sides: softplus near the identity and near
    zero, SiLU saturated."""
    inp = wl.m1_block_inputs(np.random.default_rng(9), 1, 120, 24, 16, 4, h0_sd=0.1)
    inp["dt"] = inp["dt"] * 12.0
    inp["x"] = inp["x"] * 20.0
    inp["A"] = inp["A"] * 0.05
    check(oracle_mod, *to_dev(inp))


def test_fused_zero_length_copies_state():
    inp = wl.m1_block_inputs(np.random.default_rng(3), 2, 0, 8, 16, 4, h0_sd=0.5)
    dev, _ = to_dev(inp)
    y, h = run(dev)
    assert y.shape == (2, 0, 8)
    assert torch.equal(h, dev["h0"])


def test_fused_matches_unfused_composition():
    """The fused call equals the plain scan run on the prologue's outputs (computed
    here with torch) and then gated: the scan arithmetic is shared."""
    b, L, D, N, K = 2, 200, 64, 16, 4
    inp = wl.m1_block_inputs(np.random.default_rng(21), b, L, D, N, K, h0_sd=0.2)
    dev, _ = to_dev(inp)
    y, h = run(dev)
    x = dev["x"].transpose(1, 2)                                      # (b, D, L)
    xc = torch.nn.functional.conv1d(torch.nn.functional.pad(x, (K - 1, 0)), dev["conv_w"][:, None, :],
                                    dev["conv_b"], groups=D)
    xc = torch.nn.functional.silu(xc).transpose(1, 2).contiguous()
    dtp = torch.nn.functional.softplus(dev["dt"] + dev["dt_bias"]).contiguous()
    y0, h0 = mb.mb_selective_scan(xc, dtp, dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"])
    y0 = y0 * torch.nn.functional.silu(dev["z"])
    scale = y0.abs().max().item()
    assert (y - y0).abs().max().item() <= 1e-4 * scale
    assert (h - h0).abs().max().item() <= 1e-4 * h0.abs().max().item()


@pytest.mark.slow
def test_fused_block_workload_full(oracle_mod):
    """batch 8, L 2048, D 1536, N 16, K 4 -- the fused block configuration, whole tensors."""
    dev, ref = to_dev(wl.m1_fused())
    y, h = run(dev)
    torch.cuda.synchronize()
    yr, hr = oracle_mod.m1_block(**ref)
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")
