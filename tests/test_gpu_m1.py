"""GPU parity of the Mamba-1 scan and decode step against the fp64 oracle,
through the C ABI (libmb.so via the ctypes binding)."""
import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import assert_close, assert_close_slices, prepare, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def run_scan(dev, **kw):
    return mb.mb_selective_scan(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev.get("D"),
                                dev.get("h0"), **kw)


def test_tiny_workload(oracle_mod):
    dev, ref = prepare(wl.m1_tiny(), "f32")
    y, h = run_scan(dev)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


SHAPES = [(1, 1, 1, 1), (2, 17, 5, 3), (1, 64, 16, 4), (2, 130, 33, 16), (3, 77, 40, 17),
          (1, 50, 20, 33), (2, 40, 18, 64), (1, 300, 64, 16), (2, 1000, 48, 16),
          (2, 97, 30, 8), (1, 161, 52, 32), (1, 95, 7, 4), (2, 33, 16, 16)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_shapes(oracle_mod, shape, dtype):
    b, L, D, N = shape
    rng = np.random.default_rng(hash(shape) % 2**32)
    inp = wl.m1_inputs(rng, b, L, D, N, dt_mu=-2.0, h0_sd=0.5,
                       A=-rng.uniform(0.05, 4.0, (D, N)))
    dev, ref = prepare(inp, dtype)
    y, h = run_scan(dev)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert y.dtype == dev["x"].dtype
    assert_close(y, yr, dtype, "y")
    assert_close(h, hr, dtype, "h")


def test_scan_unaligned_inputs(oracle_mod):
    """x, dt, B, C at 4-byte (not 16-byte) aligned addresses take the general scan."""
    b, L, D, N = 2, 90, 24, 16
    inp = wl.m1_inputs(np.random.default_rng(11), b, L, D, N, h0_sd=0.1)
    dev, ref = prepare(inp, "f32")
    shifted = {}
    for k in ("x", "dt", "B", "C"):
        t = dev[k]
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        shifted[k] = v
    y, h = mb.mb_selective_scan(shifted["x"], shifted["dt"], dev["A"], shifted["B"], shifted["C"],
                                dev.get("D"), dev.get("h0"))
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


def test_scan_without_skip_and_state(oracle_mod):
    rng = np.random.default_rng(5)
    inp = wl.m1_inputs(rng, 2, 45, 24, 16, with_D=False)
    dev, ref = prepare(inp, "f32")
    y, h = run_scan(dev)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


def test_scan_state_in_place(oracle_mod):
    rng = np.random.default_rng(6)
    inp = wl.m1_inputs(rng, 2, 33, 20, 16, h0_sd=1.0)
    dev, ref = prepare(inp, "f32")
    h = dev["h0"].clone()
    y, h2 = mb.mb_selective_scan(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h, h_out=h)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert h2.data_ptr() == h.data_ptr()
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


def test_scan_split_sequence_chains(oracle_mod):
    rng = np.random.default_rng(7)
    inp = wl.m1_inputs(rng, 2, 100, 32, 16, h0_sd=0.5)
    dev, ref = prepare(inp, "f32")
    s = 37
    part = lambda k, sl: dev[k][:, sl].contiguous()
    ya, ha = mb.mb_selective_scan(part("x", slice(0, s)), part("dt", slice(0, s)), dev["A"],
                                  part("B", slice(0, s)), part("C", slice(0, s)), dev["D"], dev["h0"])
    yb, hb = mb.mb_selective_scan(part("x", slice(s, None)), part("dt", slice(s, None)), dev["A"],
                                  part("B", slice(s, None)), part("C", slice(s, None)), dev["D"], ha)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(torch.cat([ya, yb], 1), yr, "f32", "y")
    assert_close(hb, hr, "f32", "h")


def test_scan_zero_length_copies_state():
    h0 = torch.randn(2, 8, 4, device="cuda")
    x = torch.empty(2, 0, 8, device="cuda")
    B = torch.empty(2, 0, 4, device="cuda")
    A = -torch.ones(8, 4, device="cuda")
    y, h = mb.mb_selective_scan(x, x, A, B, B, None, h0)
    assert y.shape == (2, 0, 8)
    assert torch.equal(h, h0)
    y, h = mb.mb_selective_scan(x, x, A, B, B, None, None)
    assert torch.count_nonzero(h).item() == 0


def test_scan_deterministic():
    rng = np.random.default_rng(8)
    dev, _ = prepare(wl.m1_inputs(rng, 2, 200, 64, 16), "f32")
    y1, h1 = run_scan(dev)
    y2, h2 = run_scan(dev)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_workload_full(oracle_mod, dtype):
    """batch 8, L 2048, D 1536, N 16 -- the bench configuration, whole tensors."""
    dev, ref = prepare(wl.m1_block(), dtype)
    y, h = run_scan(dev)
    torch.cuda.synchronize()
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, dtype, "y")
    assert_close(h, hr, dtype, "h")
    # and per (batch, channel): every channel to its own scale
    assert_close_slices(y, yr, dtype, "y per channel", (0, 2))
    assert_close_slices(h, hr, dtype, "h per channel", (0, 1))


# ------------------------------------------------------- sequence blocks ----
def _blocks(b, L, D, N):
    return mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN, b, L, D, 1, 1, N) > 0


BLOCK_SHAPES = [(1, 8192, 64, 16),   # one channel group: 128 blocks of 64 steps
                (2, 3000, 100, 16),  # ragged channels and last block
                (1, 2000, 30, 8),    # D not a multiple of 4 (4-byte copies), N = 8
                (3, 1111, 64, 4)]    # N = 4


@pytest.mark.parametrize("shape", BLOCK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_scan_sequence_blocks(oracle_mod, shape):
    """The sequence cut into blocks (carry pass, then each block from the
    composed carries) against the oracle and against the one-block scan."""
    b, L, D, N = shape
    assert _blocks(b, L, D, N)
    rng = np.random.default_rng(sum(shape))
    inp = wl.m1_inputs(rng, b, L, D, N, h0_sd=0.5, A=-rng.uniform(0.01, 2.0, (D, N)))
    dev, ref = prepare(inp, "f32")
    y, h = run_scan(dev)
    y1, h1 = run_scan(dev, seq_blocks=False)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")
    assert torch.max(torch.abs(y - y1)).item() <= 1e-5 * torch.max(torch.abs(y1)).item()
    assert torch.max(torch.abs(h - h1)).item() <= 1e-5 * torch.max(torch.abs(h1)).item()


def test_scan_sequence_blocks_state_in_place(oracle_mod):
    """h_out == h0 with sequence blocks: the carry pass keeps its own copy of h0."""
    b, L, D, N = 1, 4000, 64, 16
    assert _blocks(b, L, D, N)
    rng = np.random.default_rng(21)
    inp = wl.m1_inputs(rng, b, L, D, N, h0_sd=1.0, A=-rng.uniform(0.001, 0.05, (D, N)))
    dev, ref = prepare(inp, "f32")
    h = dev["h0"].clone()
    y, h2 = mb.mb_selective_scan(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h, h_out=h)
    yr, hr = oracle_mod.m1_scan(**ref)
    assert h2.data_ptr() == h.data_ptr()
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.slow
def test_long_sequence_blocks_with_state(oracle_mod):
    """One sequence of the block model's width (batch 1, L 16384, D 1536, N 16:
    as many (t, c, n) elements as the block workload) runs in 32 sequence
    blocks; with h0 != 0 and a weak decay the initial state reaches every block."""
    assert _blocks(1, 16384, 1536, 16)
    rng = np.random.default_rng(22)
    inp = wl.m1_block(batch=1, L=16384)
    inp["h0"] = rng.normal(0.0, 0.5, size=(1, 1536, 16))
    inp["A"] = inp["A"] * 0.01
    dev, ref = prepare(inp, "f32")
    y, h = run_scan(dev)
    torch.cuda.synchronize()
    yr, hr = oracle_mod.m1_scan(**ref)
    assert np.max(np.abs(yr[:, -1])) > 1e-2 * np.max(np.abs(yr))
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


# ------------------------------------------------------------------- step ----
STEP_SHAPES = [(1, 1, 1), (3, 7, 4), (5, 33, 8), (4, 70, 16), (2, 40, 32), (2, 20, 64),
               (3, 9, 5), (2, 11, 13), (7, 129, 16)]


@pytest.mark.parametrize("shape", STEP_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_shapes(oracle_mod, shape, dtype):
    b, D, N = shape
    rng = np.random.default_rng(sum(shape) * 31)
    inp = dict(x=rng.standard_normal((b, D)), dt=np.logaddexp(0, rng.normal(-2, 1, (b, D))),
               A=-rng.uniform(0.1, 3.0, (D, N)), B=rng.standard_normal((b, N)),
               C=rng.standard_normal((b, N)), D=rng.standard_normal(D),
               h=rng.normal(0, 0.5, (b, D, N)))
    dev, ref = prepare(inp, dtype)
    h = dev["h"].clone()
    y, h2 = mb.mb_ssm_step(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h)
    yr, hr = oracle_mod.m1_step(ref["x"], ref["dt"], ref["A"], ref["B"], ref["C"], ref["D"], ref["h"])
    assert h2.data_ptr() == h.data_ptr()
    assert_close(y, yr, dtype, "y")
    assert_close(h, hr, dtype, "h")


def test_step_out_of_place_keeps_input(oracle_mod):
    inp = wl.m1_decode(batch=8, D=64)
    dev, ref = prepare(inp, "f32")
    h_in = dev["h"].clone()
    out = torch.empty_like(h_in)
    y, h = mb.mb_ssm_step(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h_in, h_out=out)
    yr, hr = oracle_mod.m1_step(ref["x"], ref["dt"], ref["A"], ref["B"], ref["C"], ref["D"], ref["h"])
    assert torch.equal(h_in, dev["h"])
    assert_close(y, yr, "f32", "y")
    assert_close(out, hr, "f32", "h")


def test_decode_workload_full(oracle_mod):
    """256 sequences, D 1536, N 16: one batched in-place step."""
    dev, ref = prepare(wl.m1_decode(), "f32")
    h = dev["h"].clone()
    y, _ = mb.mb_ssm_step(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h)
    yr, hr = oracle_mod.m1_step(ref["x"], ref["dt"], ref["A"], ref["B"], ref["C"], ref["D"], ref["h"])
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


def test_step_unrolled_matches_scan():
    """forward over a sequence == the step unrolled token by token (both on GPU)."""
    rng = np.random.default_rng(9)
    inp = wl.m1_inputs(rng, 3, 40, 48, 16, h0_sd=0.3)
    dev, _ = prepare(inp, "f32")
    y, h = run_scan(dev)
    hs = dev["h0"].clone()
    ys = []
    for t in range(40):
        yt, _ = mb.mb_ssm_step(dev["x"][:, t].contiguous(), dev["dt"][:, t].contiguous(), dev["A"],
                               dev["B"][:, t].contiguous(), dev["C"][:, t].contiguous(), dev["D"], hs)
        ys.append(yt)
    ys = torch.stack(ys, 1)
    assert torch.max(torch.abs(ys - y)).item() <= 1e-4 * torch.max(torch.abs(y)).item()
    assert torch.max(torch.abs(hs - h)).item() <= 1e-4 * torch.max(torch.abs(h)).item()
