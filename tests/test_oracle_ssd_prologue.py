"""Pins of the Mamba-2 block prologue oracle against what the mathematics fixes:
the causal convolution is scipy's FIR filter along time; one tap is a per-channel
affine map; softplus satisfies softplus(v) - softplus(-v) = v; a sequence split
in two with the history carried gives the unsplit result; the outputs are the
SiLU'd channels split and scaled as stated."""
import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

H, P, G, N = 2, 4, 1, 4
CIN = H * P + 2 * G * N


def _inputs(rng, b=2, L=23, K=4):
    return dict(xBC=rng.standard_normal((b, L, CIN)), conv_w=rng.standard_normal((CIN, K)),
                dt=rng.standard_normal((b, L, H)), A=-np.exp(rng.standard_normal(H)),
                conv_b=rng.standard_normal(CIN), dt_bias=rng.standard_normal(H))


def test_conv_is_fir_filter(oracle_mod):
    rng = np.random.default_rng(1)
    i = _inputs(rng)
    X, B, C, ld, dtp = oracle_mod.ssd_prologue(**i, H=H, P=P, G=G, N=N)
    pre = np.empty(i["xBC"].shape)
    for c in range(CIN):
        pre[:, :, c] = lfilter(i["conv_w"][c, ::-1], [1.0], i["xBC"][:, :, c], axis=1) + i["conv_b"][c]
    v = pre * expit(pre)
    d = np.logaddexp(0.0, i["dt"] + i["dt_bias"])
    assert np.allclose(X, v[..., :H * P].reshape(2, 23, H, P) * d[..., None], rtol=1e-12, atol=1e-14)
    assert np.allclose(B, v[..., H * P:H * P + G * N].reshape(2, 23, G, N), rtol=1e-12, atol=1e-14)
    assert np.allclose(C, v[..., H * P + G * N:].reshape(2, 23, G, N), rtol=1e-12, atol=1e-14)
    assert np.allclose(ld, d * i["A"], rtol=1e-13)


def test_one_tap_and_softplus_identity(oracle_mod):
    rng = np.random.default_rng(2)
    i = _inputs(rng, K=1)
    _, B, _, _, dtp = oracle_mod.ssd_prologue(**i, H=H, P=P, G=G, N=N)
    pre = i["xBC"][..., H * P:H * P + G * N] * i["conv_w"][H * P:H * P + G * N, 0] + i["conv_b"][H * P:H * P + G * N]
    assert np.allclose(B.reshape(pre.shape), pre / (1.0 + np.exp(-pre)), rtol=1e-13, atol=1e-15)
    i2 = dict(i, dt=-i["dt"] - 2 * i["dt_bias"])      # u -> -u
    dtn = oracle_mod.ssd_prologue(**i2, H=H, P=P, G=G, N=N)[4]
    assert np.allclose(dtp - dtn, i["dt"] + i["dt_bias"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_split_with_history(oracle_mod, K):
    rng = np.random.default_rng(3 + K)
    i = _inputs(rng, L=30, K=K)
    whole = oracle_mod.ssd_prologue(**i, H=H, P=P, G=G, N=N)
    s = 11
    a = dict(i, xBC=i["xBC"][:, :s], dt=i["dt"][:, :s])
    bb = dict(i, xBC=i["xBC"][:, s:], dt=i["dt"][:, s:], x_hist=i["xBC"][:, s - K + 1:s])
    first = oracle_mod.ssd_prologue(**a, H=H, P=P, G=G, N=N)
    second = oracle_mod.ssd_prologue(**bb, H=H, P=P, G=G, N=N)
    for w, f, g in zip(whole, first, second):
        assert np.allclose(w, np.concatenate([f, g], axis=1), rtol=1e-13, atol=1e-15)


def _block_inputs(rng, b=2, L=29, K=4):
    i = _inputs(rng, b, L, K)
    i.update(x_hist=rng.standard_normal((b, K - 1, CIN)), h0=0.3 * rng.standard_normal((b, H, N, P)),
             D=rng.standard_normal(H), z=rng.standard_normal((b, L, H, P)))
    return i


def test_block_is_prologue_then_gated_ssd(oracle_mod):
    """ssd_block = ssd_prologue, then the SSD on its X, B, C, logdecay, then the
    skip term on the convolved activation (SiLU of the FIR-filtered x channels,
    not yet scaled by dt') and the SiLU(z) gate: checked against scipy's FIR
    filter and logistic sigmoid, with the history carried."""
    rng = np.random.default_rng(9)
    i = _block_inputs(rng)
    Y, h = oracle_mod.ssd_block(**i, H=H, P=P, G=G, N=N)
    full = np.concatenate([i["x_hist"], i["xBC"]], axis=1)
    pre = np.empty(full.shape)
    for c in range(CIN):
        pre[:, :, c] = lfilter(i["conv_w"][c, ::-1], [1.0], full[:, :, c], axis=1) + i["conv_b"][c]
    v = (pre * expit(pre))[:, 3:]
    d = np.logaddexp(0.0, i["dt"] + i["dt_bias"])
    xs = v[..., :H * P].reshape(2, 29, H, P)
    Bv = v[..., H * P:H * P + G * N].reshape(2, 29, G, N)
    Cv = v[..., H * P + G * N:].reshape(2, 29, G, N)
    Ys, hs = oracle_mod.ssd(xs * d[..., None], d * i["A"], Bv, Cv, i["h0"])
    ref = (Ys + i["D"][None, None, :, None] * xs) * i["z"] * expit(i["z"])
    assert np.allclose(Y, ref, rtol=1e-11, atol=1e-13) and np.allclose(h, hs, rtol=1e-11, atol=1e-13)


def test_block_split_chains_through_history_and_state(oracle_mod):
    """A sequence split in two calls chains exactly with the state and the last
    K - 1 raw xBC rows of the first call as the second's history."""
    rng = np.random.default_rng(10)
    i = _block_inputs(rng, L=40)
    Y, h = oracle_mod.ssd_block(**i, H=H, P=P, G=G, N=N)
    s = 17
    a = dict(i, xBC=i["xBC"][:, :s], dt=i["dt"][:, :s], z=i["z"][:, :s])
    Ya, ha = oracle_mod.ssd_block(**a, H=H, P=P, G=G, N=N)
    bb = dict(i, xBC=i["xBC"][:, s:], dt=i["dt"][:, s:], z=i["z"][:, s:], x_hist=i["xBC"][:, s - 3:s], h0=ha)
    Yb, hb = oracle_mod.ssd_block(**bb, H=H, P=P, G=G, N=N)
    assert np.allclose(np.concatenate([Ya, Yb], 1), Y, rtol=1e-11, atol=1e-13)
    assert np.allclose(hb, h, rtol=1e-11, atol=1e-13)
