"""GPU parity in the degenerate regimes of the recurrences, against the fp64
oracle through the C ABI:

* no decay (log-decay 0 everywhere, Mamba-1 A = 0): the state is a running sum
  of every input (TorchMamba README, Math notes M2: a_t = 1);
* very strong decay (log-decay about -60 per step): the state holds little
  more than the current step, and the chunk-local cumulative log-decay reaches
  thousands below zero, where exp(cum_i) and exp(-cum_j) separately over- or
  underflow;
* no input (X = 0) from a non-zero initial state under a weak decay and the
  data-dependent rotations: the output is the initial state carried by the
  composed (decay, angle) of every earlier step, across every sequence segment
  (Math notes M3 SISO, rotations compose additively);
* Mamba-1 with dt = 0 (y = D x, the state untouched) and with A = 0 (prefix
  sums);
* SISO with beta = 0 and no rotation against the oracle's Mamba-2 SSD of
  gamma X (the reduction of the TorchMamba README, Models table: the exact
  two-term path).

Every case runs at a length that spans several sequence segments of the
chunked walk (its planner splits long sequences), so the segment composition
runs too."""
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


def _ssd(dev):
    return mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h0"])


def _trap(dev):
    return mb.mb_trap_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], dev["h0"])


def _mimo(dev):
    return mb.mb_mimo_ssd(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["beta"], dev["gamma"],
                          dev["theta"], dev["h0"])


# --------------------------------------------------------------- no decay ----
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_no_decay_long(oracle_mod, dtype):
    """Mamba-2, logdecay = 0 at L = 4096: S_t = h0 + sum_{s<=t} B_s X_s^T."""
    inp = wl.ssd_inputs(np.random.default_rng(201), 2, 4096, 8, 64, 128, h0_sd=0.05)
    inp["logdecay"] = np.zeros_like(inp["logdecay"])
    dev, ref = prepare(inp, dtype)
    Y, h = _ssd(dev)
    Yr, hr = oracle_mod.ssd(**ref)
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


def test_siso_no_decay_long(oracle_mod):
    """SISO with rotations, logdecay = 0 at L = 4096."""
    inp = wl.trap_inputs(np.random.default_rng(202), 2, 4096, 8, 64, 128, h0_sd=0.05)
    inp["logdecay"] = np.zeros_like(inp["logdecay"])
    dev, ref = prepare(inp, "f32")
    Y, h = _trap(dev)
    Yr, hr = oracle_mod.trap(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


def test_mimo_no_decay_long(oracle_mod):
    inp = wl.mimo_inputs(np.random.default_rng(203), 1, 2048, 4, 64, 128, 4, h0_sd=0.05)
    inp["logdecay"] = np.zeros_like(inp["logdecay"])
    dev, ref = prepare(inp, "f32")
    Y, h = _mimo(dev)
    Yr, hr = oracle_mod.mimo(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


# --------------------------------------------------------- strong decay ----
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_strong_decay(oracle_mod, dtype):
    """logdecay ~ -60 per step: a chunk's cumulative log-decay reaches about -3800."""
    rng = np.random.default_rng(204)
    inp = wl.ssd_inputs(rng, 2, 1500, 4, 64, 128, h0_sd=0.05)
    inp["logdecay"] = -rng.uniform(50.0, 70.0, size=inp["logdecay"].shape)
    dev, ref = prepare(inp, dtype)
    Y, h = _ssd(dev)
    Yr, hr = oracle_mod.ssd(**ref)
    assert np.all(np.isfinite(Y.float().cpu().numpy()))
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")
    assert_close_slices(Y, Yr, dtype, "Y per head", (0, 2))


def test_siso_strong_decay(oracle_mod):
    rng = np.random.default_rng(205)
    inp = wl.trap_inputs(rng, 2, 1500, 4, 64, 128, h0_sd=0.05)
    inp["logdecay"] = -rng.uniform(50.0, 70.0, size=inp["logdecay"].shape)
    # beta carries alpha = exp(logdecay) of its step (the trapezoid recipe)
    inp["beta"] = inp["beta"] * 0.0 + 0.3 * np.exp(inp["logdecay"])
    dev, ref = prepare(inp, "f32")
    Y, h = _trap(dev)
    Yr, hr = oracle_mod.trap(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    assert_close_slices(Y, Yr, "f32", "Y per head", (0, 2))


def test_mimo_strong_decay(oracle_mod):
    rng = np.random.default_rng(206)
    inp = wl.mimo_inputs(rng, 1, 1200, 4, 64, 128, 4, h0_sd=0.05)
    inp["logdecay"] = -rng.uniform(50.0, 70.0, size=inp["logdecay"].shape)
    dev, ref = prepare(inp, "f32")
    Y, h = _mimo(dev)
    Yr, hr = oracle_mod.mimo(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    assert_close_slices(Y, Yr, "f32", "Y per head", (0, 2))


# ------------------------------------------ no input, carried initial state ----
def _weak_decay(rng, shape):
    # about -0.0005 per step: the initial state survives the whole sequence
    return -rng.uniform(0.0, 0.001, size=shape)


@pytest.mark.parametrize("L", [700, 4096])
def test_ssd_zero_input_carried_state(oracle_mod, L):
    rng = np.random.default_rng(207)
    inp = wl.ssd_inputs(rng, 2, L, 6, 64, 128, h0_sd=0.5)
    inp["X"] = np.zeros_like(inp["X"])
    inp["logdecay"] = _weak_decay(rng, inp["logdecay"].shape)
    dev, ref = prepare(inp, "f32")
    Y, h = _ssd(dev)
    Yr, hr = oracle_mod.ssd(**ref)
    assert np.max(np.abs(Yr[:, -1])) > 1e-2 * np.max(np.abs(Yr))   # the state reaches the end
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.parametrize("L", [700, 4096])
def test_siso_zero_input_carried_state(oracle_mod, L):
    """X = 0 (and no previous token), h0 != 0, theta != 0: Y_t =
    exp(sum_{s<=t} ld_s) C_t^T R(-Theta_t) h0 -- only the composed decay and
    angle of the earlier steps and segments act."""
    rng = np.random.default_rng(208)
    inp = wl.trap_inputs(rng, 2, L, 6, 64, 128, h0_sd=0.5)
    inp["X"] = np.zeros_like(inp["X"])
    inp["logdecay"] = _weak_decay(rng, inp["logdecay"].shape)
    dev, ref = prepare(inp, "f32")
    Y, h = _trap(dev)
    Yr, hr = oracle_mod.trap(**ref)
    assert np.max(np.abs(Yr[:, -1])) > 1e-2 * np.max(np.abs(Yr))
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


def test_mimo_zero_input_carried_state(oracle_mod):
    rng = np.random.default_rng(209)
    inp = wl.mimo_inputs(rng, 1, 2048, 4, 64, 128, 4, h0_sd=0.5)
    inp["X"] = np.zeros_like(inp["X"])
    inp["logdecay"] = _weak_decay(rng, inp["logdecay"].shape)
    dev, ref = prepare(inp, "f32")
    Y, h = _mimo(dev)
    Yr, hr = oracle_mod.mimo(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


# ----------------------------------------------------------------- Mamba-1 ----
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_m1_zero_step(oracle_mod, dtype):
    """dt = 0: y = D x exactly and the state is h0."""
    inp = wl.m1_inputs(np.random.default_rng(210), 2, 2048, 192, 16, h0_sd=0.3)
    inp["dt"] = np.zeros_like(inp["dt"])
    dev, ref = prepare(inp, dtype)
    y, h = mb.mb_selective_scan(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"])
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, dtype, "y")
    assert torch.equal(h, dev["h0"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_m1_no_decay(oracle_mod, dtype):
    """A = 0: h_t = h0 + sum_{s<=t} dt_s B_s x_s (no decay over 2048 steps)."""
    inp = wl.m1_inputs(np.random.default_rng(211), 2, 2048, 192, 16, h0_sd=0.3)
    inp["A"] = np.zeros_like(inp["A"])
    dev, ref = prepare(inp, dtype)
    y, h = mb.mb_selective_scan(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"])
    yr, hr = oracle_mod.m1_scan(**ref)
    assert_close(y, yr, dtype, "y")
    assert_close(h, hr, dtype, "h")


def test_m1_zero_input_carried_state(oracle_mod):
    """x = 0 from h0 != 0 under a weak decay: h_T = exp(A sum dt) h0 and y_t =
    C_t . (exp(A cum_t) h0), across the whole sequence."""
    rng = np.random.default_rng(212)
    inp = wl.m1_inputs(rng, 2, 2048, 192, 16, h0_sd=0.5)
    inp["x"] = np.zeros_like(inp["x"])
    inp["A"] = -rng.uniform(0.0, 0.02, size=inp["A"].shape)
    dev, ref = prepare(inp, "f32")
    y, h = mb.mb_selective_scan(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"])
    yr, hr = oracle_mod.m1_scan(**ref)
    assert np.max(np.abs(yr[:, -1])) > 1e-2 * np.max(np.abs(yr))
    assert_close(y, yr, "f32", "y")
    assert_close(h, hr, "f32", "h")


# ------------------------------------------------- SISO -> Mamba-2 reduction ----
@pytest.mark.parametrize("L", [333, 4096])
def test_siso_without_beta_and_rotation_is_ssd_of_gamma_x(oracle_mod, L):
    """beta = 0, theta = None: the trapezoid is the Mamba-2 SSD of gamma X."""
    inp = wl.trap_inputs(np.random.default_rng(213), 2, L, 6, 64, 128, h0_sd=0.05, rotate=False)
    inp["beta"] = np.zeros_like(inp["beta"])
    dev, ref = prepare(inp, "f32")
    Y, h = _trap(dev)
    Xg = ref["X"] * ref["gamma"][..., None]
    Yr, hr = oracle_mod.ssd(Xg, ref["logdecay"], ref["B"], ref["C"], ref["h0"])
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
