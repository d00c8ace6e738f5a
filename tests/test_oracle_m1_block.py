"""Pins of the oracle's Mamba-1 scan with the block prologue and epilogue
(causal conv1d + SiLU, softplus(dt + bias), SiLU(z) gate): it equals the
pinned scan applied to inputs built with library routines (scipy.signal.lfilter
for the causal filter, numpy.logaddexp for softplus, scipy.special.expit for
the sigmoid), and a sequence split across calls chains exactly through h0 and
the raw-input history."""
import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

from selective_state_space_amd import workloads as wl

RTOL, ATOL = 1e-10, 1e-12


def close(a, b, rtol=RTOL, atol=ATOL):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def _reference(o, inp):
    x, w = inp["x"], inp["conv_w"]
    b, L, D = x.shape
    K = w.shape[1]
    hist = inp.get("x_hist")
    if hist is None:
        hist = np.zeros((b, K - 1, D))
    ext = np.concatenate([hist, x], axis=1)                  # (b, K-1+L, D)
    pre = np.empty_like(x)
    for c in range(D):
        # lfilter gives out[t] = sum_j f[j] ext[t - j]; with f = w reversed, f[j] = w[K-1-j]
        # multiplies x_{t-j}, i.e. tap k = K-1-j multiplies x_{t-K+1+k}
        pre[:, :, c] = lfilter(w[c, ::-1], [1.0], ext[:, :, c], axis=1)[:, K - 1:]
    pre = pre + (inp["conv_b"] if inp.get("conv_b") is not None else 0.0)
    xc = pre * expit(pre)
    dtv = np.logaddexp(0.0, inp["dt"] + (inp["dt_bias"] if inp.get("dt_bias") is not None else 0.0))
    y, h = o.m1_scan(xc, dtv, inp["A"], inp["B"], inp["C"], inp["D"], inp.get("h0"))
    if inp.get("z") is not None:
        y = y * (inp["z"] * expit(inp["z"]))
    return y, h


@pytest.mark.parametrize("K,hist,h0", [(4, False, 0.0), (4, True, 0.5), (3, True, 0.0), (1, False, 0.3), (2, False, 0.0)])
def test_block_equals_library_composition(oracle_mod, K, hist, h0):
    inp = wl.m1_block_inputs(np.random.default_rng(8100 + K + 10 * hist), 2, 37, 5, 4, K=K, h0_sd=h0, hist=hist)
    y, h = oracle_mod.m1_block(**inp)
    yr, hr = _reference(oracle_mod, inp)
    close(y, yr)
    close(h, hr)


def test_block_optional_terms(oracle_mod):
    """No bias, no gate, no skip: the composition without those terms."""
    inp = wl.m1_block_inputs(np.random.default_rng(8200), 1, 20, 3, 2)
    for k in ("conv_b", "dt_bias", "z", "D"):
        inp[k] = None
    y, h = oracle_mod.m1_block(**inp)
    yr, hr = _reference(oracle_mod, inp)
    close(y, yr)
    close(h, hr)


def test_block_split_chaining(oracle_mod):
    inp = wl.m1_block_inputs(np.random.default_rng(8300), 2, 60, 4, 4, K=4, h0_sd=0.2)
    y, h = oracle_mod.m1_block(**inp)
    s = 23
    a = dict(inp, x=inp["x"][:, :s], dt=inp["dt"][:, :s], B=inp["B"][:, :s], C=inp["C"][:, :s], z=inp["z"][:, :s])
    ya, ha = oracle_mod.m1_block(**a)
    b = dict(inp, x=inp["x"][:, s:], dt=inp["dt"][:, s:], B=inp["B"][:, s:], C=inp["C"][:, s:], z=inp["z"][:, s:],
             h0=ha, x_hist=inp["x"][:, s - 3:s])
    yb, hb = oracle_mod.m1_block(**b)
    close(np.concatenate([ya, yb], 1), y)
    close(hb, h)
