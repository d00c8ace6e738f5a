"""GPU parity of the chunkwise SSD family (Mamba-2 SSD, Mamba-3 SISO, Mamba-3
MIMO) against the fp64 oracle, through the C ABI."""
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


def _seed(*xs):
    return int(abs(hash(tuple(xs)))) % (2 ** 32)


# -------------------------------------------------------------------- SSD ----
SSD_SHAPES = [  # batch, L, H, P, N, G
    (1, 1, 1, 16, 4, 1), (2, 65, 2, 16, 8, 1), (1, 64, 3, 32, 16, 3), (2, 130, 4, 16, 128, 2),
    (1, 200, 2, 64, 128, 1), (2, 333, 3, 48, 64, 1), (1, 129, 6, 16, 32, 2),
    (1, 700, 2, 128, 64, 1),   # two column groups, two sequence segments
    (1, 150, 2, 32, 96, 1),    # state rows padded to 128
    (1, 90, 2, 16, 12, 1)]     # N not a multiple of 8


@pytest.mark.parametrize("shape", SSD_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_shapes(oracle_mod, shape, dtype):
    b, L, H, P, N, G = shape
    inp = wl.ssd_inputs(np.random.default_rng(_seed(shape, 1)), b, L, H, P, N, G=G, h0_sd=0.05)
    dev, ref = prepare(inp, dtype)
    Y, h = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h0"])
    Yr, hr = oracle_mod.ssd(**ref)
    assert Y.dtype == dev["X"].dtype
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


def test_ssd_split_chaining(oracle_mod):
    inp = wl.ssd_inputs(np.random.default_rng(3), 2, 300, 2, 32, 64, h0_sd=0.05)
    dev, ref = prepare(inp, "f32")
    s = 100
    cut = lambda k, sl: dev[k][:, sl].contiguous()
    Ya, ha = mb.mb_ssd_chunked(cut("X", slice(0, s)), cut("logdecay", slice(0, s)),
                               cut("B", slice(0, s)), cut("C", slice(0, s)), dev["h0"])
    Yb, hb = mb.mb_ssd_chunked(cut("X", slice(s, None)), cut("logdecay", slice(s, None)),
                               cut("B", slice(s, None)), cut("C", slice(s, None)), ha)
    Yr, hr = oracle_mod.ssd(**ref)
    assert_close(torch.cat([Ya, Yb], 1), Yr, "f32", "Y")
    assert_close(hb, hr, "f32", "h")


SEG_SHAPES = [  # batch, L, H, P, N, G: long enough for several sequence segments
    (2, 1500, 4, 48, 128, 2),   # 128 state rows; a column tile half past P
    (1, 2600, 3, 16, 64, 1),    # 64 state rows: two of the four waves past P
    (2, 1800, 2, 96, 32, 1),    # 32 state rows: two of the four waves past N
    (1, 2100, 4, 64, 96, 4),    # one head per group; one wave past N
    (1, 2049, 2, 128, 12, 2),   # two column tiles, N = 12, a one-step last chunk
    (1, 1700, 2, 16, 4, 1),     # N = 4: one lane row of four in range
    (2, 1600, 3, 32, 8, 3)]     # N = 8, one head per group


@pytest.mark.parametrize("shape", SEG_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_segment_states(oracle_mod, shape, dtype):
    """The state-only pass (the segments' local end states as weighted
    products over their steps; fp32 and bf16 inputs) at the tile edges,
    through the sequences' outputs and final states."""
    b, L, H, P, N, G = shape
    inp = wl.ssd_inputs(np.random.default_rng(_seed(shape, 5)), b, L, H, P, N, G=G, h0_sd=0.05)
    dev, ref = prepare(inp, dtype)
    Y, h = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h0"])
    Yr, hr = oracle_mod.ssd(**ref)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")
    assert_close_slices(h, hr, dtype, "h per head", (0, 1))


def test_ssd_zero_length_and_in_place_state():
    X = torch.empty(2, 0, 2, 16, device="cuda")
    ld = torch.empty(2, 0, 2, device="cuda")
    B = torch.empty(2, 0, 1, 8, device="cuda")
    h0 = torch.randn(2, 2, 8, 16, device="cuda")
    Y, h = mb.mb_ssd_chunked(X, ld, B, B, h0)
    assert torch.equal(h, h0)
    hh = h0.clone()
    Y, h = mb.mb_ssd_chunked(X, ld, B, B, hh, h_out=hh)
    assert torch.equal(hh, h0)


def test_ssd_deterministic():
    dev, _ = prepare(wl.ssd_inputs(np.random.default_rng(4), 2, 257, 3, 32, 128), "f32")
    r1 = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"])
    r2 = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"])
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_block_workload_full(oracle_mod, dtype):
    """batch 4, L 4096, H 24, P 64, N 128, G 1 -- the bench configuration."""
    dev, ref = prepare(wl.ssd_block(), dtype)
    Y, h = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"])
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.ssd(**ref)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")
    # and per (batch, head): every head to its own scale
    assert_close_slices(Y, Yr, dtype, "Y per head", (0, 2))
    assert_close_slices(h, hr, dtype, "h per head", (0, 1))


# ------------------------------------------------------------------- SISO ----
TRAP_SHAPES = [  # batch, L, H, P, N, G
    (1, 1, 1, 16, 4, 1), (2, 65, 2, 16, 8, 2), (1, 64, 3, 32, 16, 1), (2, 130, 4, 16, 128, 2),
    (1, 333, 2, 64, 128, 1), (2, 97, 3, 32, 32, 3),
    (1, 700, 2, 128, 64, 1)]   # two column groups, two sequence segments


@pytest.mark.parametrize("shape", TRAP_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("rotate", [True, False])
def test_siso_shapes(oracle_mod, shape, rotate):
    b, L, H, P, N, G = shape
    inp = wl.trap_inputs(np.random.default_rng(_seed(shape, rotate)), b, L, H, P, N, G=G,
                         h0_sd=0.05, rotate=rotate)
    dev, ref = prepare(inp, "f32")
    Y, h = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], dev["h0"])
    Yr, hr = oracle_mod.trap(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


TRAP_SEG_SHAPES = [  # batch, L, H, P, N, G: several sequence segments
    (2, 1500, 4, 48, 128, 2),   # 128 state rows; a column tile half past P
    (1, 2600, 3, 16, 64, 1),    # 64 state rows, P = 16
    (2, 1800, 2, 96, 32, 1),    # 32 state rows (16 pairs)
    (1, 2100, 4, 64, 96, 4),    # one head per group; the second row block half past N
    (1, 2049, 2, 128, 12, 2),   # two column tiles, N = 12, a one-step last chunk
    (1, 1700, 2, 16, 4, 1),     # N = 4: two pairs
    (2, 1600, 3, 32, 8, 3)]     # N = 8, one head per group


@pytest.mark.parametrize("shape", TRAP_SEG_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("rotate", [True, False])
def test_siso_segment_states(oracle_mod, shape, rotate):
    """The SISO state-only pass (each quarter of a segment a weighted, turned
    product, carried to the segment's end) at the tile edges, through the
    outputs and final states."""
    b, L, H, P, N, G = shape
    inp = wl.trap_inputs(np.random.default_rng(_seed(shape, 7 + rotate)), b, L, H, P, N, G=G,
                         h0_sd=0.05, rotate=rotate)
    dev, ref = prepare(inp, "f32")
    Y, h = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], dev["h0"])
    Yr, hr = oracle_mod.trap(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    assert_close_slices(h, hr, "f32", "h per head", (0, 1))


def test_siso_bf16(oracle_mod):
    inp = wl.trap_inputs(np.random.default_rng(5), 2, 200, 3, 32, 64, h0_sd=0.05)
    dev, ref = prepare(inp, "bf16")
    Y, h = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], dev["h0"])
    Yr, hr = oracle_mod.trap(**ref)
    assert_close(Y, Yr, "bf16", "Y")
    assert_close(h, hr, "bf16", "h")


def _split_call(fn, dev, s, **kw):
    """Two chunked calls split at step s; the second gets the first's final state
    and the token before the split."""
    cut = lambda sl: {k: (v[:, sl].contiguous() if k != "h0" and v is not None else v) for k, v in dev.items()}
    a, b = cut(slice(0, s)), cut(slice(s, None))
    args = lambda d: (d["X"], d["logdecay"], d["B"], d["C"], d["beta"], d["gamma"], d["theta"])
    Ya, ha = fn(*args(a), dev["h0"])
    Yb, hb = fn(*args(b), ha, X_prev=dev["X"][:, s - 1].contiguous(), B_prev=dev["B"][:, s - 1].contiguous())
    return torch.cat([Ya, Yb], 1), hb


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rotate", [True, False])
def test_siso_split_with_previous_token(oracle_mod, dtype, rotate):
    """A sequence split at a step that is not a chunk boundary, with a nonzero
    cross-boundary weight, chains exactly through h0 and (X_prev, B_prev); the
    second part is long enough for several sequence segments."""
    inp = wl.trap_inputs(np.random.default_rng(41 + rotate), 2, 900, 3, 32, 64, G=1, h0_sd=0.05, rotate=rotate)
    dev, ref = prepare(inp, dtype)
    Yr, hr = oracle_mod.trap(**ref)
    Y, h = _split_call(mb.mb_trap_ssd, dev, 301)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


@pytest.mark.parametrize("R", [2, 4])
def test_mimo_split_with_previous_token(oracle_mod, R):
    inp = wl.mimo_inputs(np.random.default_rng(43 + R), 1, 600, 2, 32, 64, R, h0_sd=0.05)
    dev, ref = prepare(inp, "f32")
    Yr, hr = oracle_mod.mimo(**ref)
    Y, h = _split_call(mb.mb_mimo_ssd, dev, 133)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


def test_siso_large_angles(oracle_mod):
    """Accumulated angles of several hundred radians (long sequence, large theta):
    the chunk-local angles keep fp32 accurate."""
    inp = wl.trap_inputs(np.random.default_rng(6), 1, 2000, 2, 16, 32)
    inp["theta"] = inp["theta"] * 8.0
    dev, ref = prepare(inp, "f32")
    Y, h = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], None)
    Yr, hr = oracle_mod.trap(**ref)
    assert np.max(np.cumsum(ref["theta"], axis=1)) > 300
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.slow
def test_siso_block_workload_full(oracle_mod):
    """batch 4, L 4096, H 24, P 64, N 128 with rotations -- the bench configuration."""
    dev, ref = prepare(wl.siso_block(), "f32")
    Y, h = mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], None)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.trap(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    assert_close_slices(Y, Yr, "f32", "Y per head", (0, 2))
    assert_close_slices(h, hr, "f32", "h per head", (0, 1))


# ------------------------------------------------------------------- MIMO ----
MIMO_SHAPES = [  # batch, L, H, P, N, R
    (1, 1, 1, 16, 4, 1), (2, 37, 2, 16, 8, 2), (1, 70, 2, 32, 16, 4), (2, 50, 2, 16, 128, 4),
    (1, 33, 3, 16, 32, 8), (1, 21, 2, 16, 16, 16), (2, 130, 2, 32, 64, 1)]


@pytest.mark.parametrize("shape", MIMO_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("rotate", [True, False])
def test_mimo_shapes(oracle_mod, shape, rotate):
    b, L, H, P, N, R = shape
    inp = wl.mimo_inputs(np.random.default_rng(_seed(shape, rotate)), b, L, H, P, N, R,
                         h0_sd=0.05, rotate=rotate)
    dev, ref = prepare(inp, "f32")
    Y, h = mb.mb_mimo_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], dev["h0"])
    Yr, hr = oracle_mod.mimo(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


def test_mimo_rank_one_matches_siso():
    """R = 1 MIMO equals SISO with one group per head (both on the GPU)."""
    inp = wl.mimo_inputs(np.random.default_rng(7), 2, 100, 3, 32, 64, 1, h0_sd=0.05)
    dev, _ = prepare(inp, "f32")
    Ym, hm = mb.mb_mimo_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                            dev["theta"], dev["h0"])
    Ys, hs = mb.mb_trap_ssd(dev["X"][..., 0].contiguous(), dev["logdecay"], dev["B"][..., 0].contiguous(),
                            dev["C"][..., 0].contiguous(), dev["beta"], dev["gamma"], dev["theta"], dev["h0"])
    scale = torch.max(torch.abs(Ys)).item()
    assert torch.max(torch.abs(Ym[..., 0] - Ys)).item() <= 1e-4 * scale
    assert torch.max(torch.abs(hm - hs)).item() <= 1e-4 * torch.max(torch.abs(hs)).item()


@pytest.mark.slow
def test_mimo_block_workload_full(oracle_mod):
    """batch 2, L 8192, H 16, P 64, N 128, R 4 -- the bench configuration."""
    dev, ref = prepare(wl.mimo_block(), "f32")
    Y, h = mb.mb_mimo_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], None)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.mimo(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    assert_close_slices(Y, Yr, "f32", "Y per head", (0, 2))
    assert_close_slices(h, hr, "f32", "h per head", (0, 1))
