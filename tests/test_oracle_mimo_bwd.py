"""Pins of the Mamba-3 MIMO backward oracle: its gradients are the derivatives
of the (separately pinned) forward oracle, by central finite differences in
fp64, element by element on small inputs and along random directions on longer
ones; rank 1 is the SISO backward."""
import numpy as np
import pytest

from selective_state_space_amd import workloads as wl

NAMES = ("X", "logdecay", "B", "C", "beta", "gamma", "theta", "h0", "X_prev", "B_prev")


def case(seed, b, L, H, P, N, R, rot=True, prev=True, dh=True):
    rng = np.random.default_rng(seed)
    inp = wl.mimo_inputs(rng, b, L, H, P, N, R, h0_sd=0.3, rotate=rot)
    inp["X_prev"] = rng.standard_normal((b, H, P, R)) * 0.3 if prev else None
    inp["B_prev"] = rng.standard_normal((b, H, N, R)) * 0.3 if prev else None
    dY = rng.standard_normal((b, L, H, P, R))
    dhv = rng.standard_normal((b, H, N, P)) if dh else None
    return inp, dY, dhv


def loss(oracle_mod, inp, dY, dh):
    Y, h = oracle_mod.mimo(**inp)
    v = float(np.sum(Y * dY))
    if dh is not None:
        v += float(np.sum(h * dh))
    return v


def grads(oracle_mod, inp, dY, dh):
    g = oracle_mod.mimo_bwd(inp["X"], inp["logdecay"], inp["B"], inp["C"], inp["beta"], inp["gamma"], dY,
                            inp["theta"], inp["h0"], dh, inp["X_prev"], inp["B_prev"])
    return dict(zip(NAMES, g))


@pytest.mark.parametrize("rot,prev,dh", [(True, True, True), (False, True, False)])
def test_every_element_by_central_differences(oracle_mod, rot, prev, dh):
    inp, dY, dhv = case(3, 1, 4, 2, 3, 4, 2, rot, prev, dh)
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


@pytest.mark.parametrize("shape", [(1, 40, 2, 4, 6, 4), (2, 17, 1, 3, 4, 3)])
def test_directional_derivatives(oracle_mod, shape):
    inp, dY, dhv = case(31 + shape[1], *shape)
    g = grads(oracle_mod, inp, dY, dhv)
    rng = np.random.default_rng(shape[1])
    eps = 1e-6
    for name in NAMES:
        v = rng.standard_normal(inp[name].shape)
        fd = (loss(oracle_mod, dict(inp, **{name: inp[name] + eps * v}), dY, dhv) -
              loss(oracle_mod, dict(inp, **{name: inp[name] - eps * v}), dY, dhv)) / (2 * eps)
        an = float(np.sum(g[name] * v))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_rank_one_is_the_siso_backward(oracle_mod):
    inp, dY, dhv = case(7, 1, 12, 2, 3, 4, 1)
    g = grads(oracle_mod, inp, dY, dhv)
    s = {k: (v[..., 0] if v is not None and k in ("X", "B", "C", "X_prev", "B_prev") else v) for k, v in inp.items()}
    r = oracle_mod.trap_bwd(s["X"], s["logdecay"], s["B"].reshape(1, 12, 2, 4), s["C"].reshape(1, 12, 2, 4),
                            s["beta"], s["gamma"], dY[..., 0], s["theta"], s["h0"], dhv, s["X_prev"], s["B_prev"])
    # SISO with one group per head: B (b, L, G = H, N)
    for name, ref in zip(NAMES, r):
        got = g[name]
        if name in ("X", "B", "C", "X_prev", "B_prev"):
            got = got[..., 0]
        assert np.allclose(got, ref.reshape(got.shape), rtol=1e-11, atol=1e-13), name
