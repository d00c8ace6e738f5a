"""Pins of the Mamba-3 SISO backward oracle: its gradients are the derivatives
of the (separately pinned) forward oracle, checked by central finite
differences in fp64, element by element on small inputs (with rotations, the
previous token and grouped heads) and along random directions on longer ones."""
import numpy as np
import pytest

from selective_state_space_amd import workloads as wl

NAMES = ("X", "logdecay", "B", "C", "beta", "gamma", "theta", "h0", "X_prev", "B_prev")


def case(seed, b, L, H, P, N, G, rot=True, prev=True, dh=True):
    rng = np.random.default_rng(seed)
    inp = wl.trap_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.3)
    if not rot:
        inp["theta"] = None
    inp["X_prev"] = rng.standard_normal((b, H, P)) * 0.3 if prev else None
    inp["B_prev"] = rng.standard_normal((b, G, N)) * 0.3 if prev else None
    dY = rng.standard_normal((b, L, H, P))
    dhv = rng.standard_normal((b, H, N, P)) if dh else None
    return inp, dY, dhv


def loss(oracle_mod, inp, dY, dh):
    Y, h = oracle_mod.trap(**inp)
    v = float(np.sum(Y * dY))
    if dh is not None:
        v += float(np.sum(h * dh))
    return v


def grads(oracle_mod, inp, dY, dh):
    g = oracle_mod.trap_bwd(inp["X"], inp["logdecay"], inp["B"], inp["C"], inp["beta"], inp["gamma"], dY,
                            inp["theta"], inp["h0"], dh, inp["X_prev"], inp["B_prev"])
    return dict(zip(NAMES, g))


@pytest.mark.parametrize("rot,prev,dh", [(True, True, True), (False, True, True), (True, False, False)])
def test_every_element_by_central_differences(oracle_mod, rot, prev, dh):
    inp, dY, dhv = case(2, 2, 5, 2, 3, 4, 1 if rot else 2, rot, prev, dh)
    g = grads(oracle_mod, inp, dY, dhv)
    eps = 1e-6
    for name in NAMES:
        base = inp[name]
        if base is None:
            continue
        fd = np.empty_like(base)
        for i in range(base.size):
            up = base.copy()
            up.flat[i] += eps
            dn = base.copy()
            dn.flat[i] -= eps
            fd.flat[i] = (loss(oracle_mod, dict(inp, **{name: up}), dY, dhv) -
                          loss(oracle_mod, dict(inp, **{name: dn}), dY, dhv)) / (2 * eps)
        err = np.max(np.abs(fd - g[name])) / max(np.max(np.abs(fd)), 1e-300)
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("shape", [(1, 70, 2, 4, 8, 1), (2, 33, 4, 3, 6, 2), (1, 1, 2, 2, 4, 1)])
def test_directional_derivatives(oracle_mod, shape):
    b, L, H, P, N, G = shape
    inp, dY, dhv = case(21 + L, b, L, H, P, N, G)
    g = grads(oracle_mod, inp, dY, dhv)
    rng = np.random.default_rng(L + 1)
    eps = 1e-6
    for name in NAMES:
        v = rng.standard_normal(inp[name].shape)
        up = loss(oracle_mod, dict(inp, **{name: inp[name] + eps * v}), dY, dhv)
        dn = loss(oracle_mod, dict(inp, **{name: inp[name] - eps * v}), dY, dhv)
        fd = (up - dn) / (2 * eps)
        an = float(np.sum(g[name] * v))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_reduces_to_the_ssd_backward(oracle_mod):
    """beta = 0, gamma = 1, theta = 0: the Mamba-2 SSD, so the gradients are the
    SSD backward's (and dgamma = X . dX)."""
    inp, dY, dhv = case(5, 1, 30, 2, 3, 4, 1, rot=True, prev=False)
    inp["beta"] = np.zeros_like(inp["beta"])
    inp["gamma"] = np.ones_like(inp["gamma"])
    inp["theta"] = np.zeros_like(inp["theta"])
    g = grads(oracle_mod, inp, dY, dhv)
    r = oracle_mod.ssd_bwd(inp["X"], inp["logdecay"], inp["B"], inp["C"], dY, inp["h0"], dhv)
    for name, ref in zip(("X", "logdecay", "B", "C", "h0"), r):
        assert np.allclose(g[name], ref, rtol=1e-11, atol=1e-13), name
    assert np.allclose(g["gamma"], np.sum(inp["X"] * g["X"], axis=-1), rtol=1e-11, atol=1e-13)
