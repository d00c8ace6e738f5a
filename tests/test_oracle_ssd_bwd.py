"""Pins of the Mamba-2 SSD backward oracle: its gradients are the derivatives of
the (separately pinned) forward oracle, checked by central finite differences
in fp64, element by element on small inputs and along random directions on
longer ones."""
import numpy as np
import pytest

from selective_state_space_amd import workloads as wl

NAMES = ("X", "logdecay", "B", "C", "h0")


def loss(oracle_mod, inp, dY, dh):
    Y, h = oracle_mod.ssd(inp["X"], inp["logdecay"], inp["B"], inp["C"], inp["h0"])
    v = float(np.sum(Y * dY))
    if dh is not None:
        v += float(np.sum(h * dh))
    return v


def grads(oracle_mod, inp, dY, dh):
    dX, dld, dB, dC, dh0 = oracle_mod.ssd_bwd(inp["X"], inp["logdecay"], inp["B"], inp["C"], dY, inp["h0"], dh)
    return dict(X=dX, logdecay=dld, B=dB, C=dC, h0=dh0)


def case(seed, b, L, H, P, N, G, dh=True):
    rng = np.random.default_rng(seed)
    inp = wl.ssd_inputs(rng, b, L, H, P, N, G=G, h0_sd=0.3)
    dY = rng.standard_normal((b, L, H, P))
    dhv = rng.standard_normal((b, H, N, P)) if dh else None
    return inp, dY, dhv


@pytest.mark.parametrize("dh", [True, False])
def test_every_element_by_central_differences(oracle_mod, dh):
    inp, dY, dhv = case(1, 2, 6, 4, 3, 5, 2, dh)
    g = grads(oracle_mod, inp, dY, dhv)
    eps = 1e-5
    for name in NAMES:
        base = inp[name]
        fd = np.empty_like(base)
        for i in range(base.size):
            for sgn, slot in ((1, 0), (-1, 1)):
                pert = base.copy()
                pert.flat[i] += sgn * eps
                v = loss(oracle_mod, dict(inp, **{name: pert}), dY, dhv)
                if slot == 0:
                    up = v
                else:
                    fd.flat[i] = (up - v) / (2 * eps)
        err = np.max(np.abs(fd - g[name])) / max(np.max(np.abs(fd)), 1e-300)
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("shape", [(1, 130, 2, 8, 16, 1), (2, 67, 4, 5, 6, 2), (1, 1, 3, 4, 2, 3)])
def test_directional_derivatives(oracle_mod, shape):
    b, L, H, P, N, G = shape
    inp, dY, dhv = case(7 + L, b, L, H, P, N, G)
    g = grads(oracle_mod, inp, dY, dhv)
    rng = np.random.default_rng(L)
    eps = 1e-6
    for name in NAMES:
        v = rng.standard_normal(inp[name].shape)
        up = loss(oracle_mod, dict(inp, **{name: inp[name] + eps * v}), dY, dhv)
        dn = loss(oracle_mod, dict(inp, **{name: inp[name] - eps * v}), dY, dhv)
        fd = (up - dn) / (2 * eps)
        an = float(np.sum(g[name] * v))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_group_gradients_sum_over_heads(oracle_mod):
    """With G groups shared by H / G heads, dB and dC of a group are the sums of
    the per-head gradients obtained with each head alone in its own group."""
    inp, dY, dhv = case(3, 1, 20, 4, 3, 5, 1)
    g = grads(oracle_mod, inp, dY, dhv)
    dB_sum = np.zeros_like(g["B"])
    dC_sum = np.zeros_like(g["C"])
    for h in range(4):
        sub = dict(X=inp["X"][:, :, h:h + 1], logdecay=inp["logdecay"][:, :, h:h + 1], B=inp["B"], C=inp["C"],
                   h0=inp["h0"][:, h:h + 1])
        gh = grads(oracle_mod, sub, dY[:, :, h:h + 1], dhv[:, h:h + 1])
        dB_sum += gh["B"]
        dC_sum += gh["C"]
        assert np.allclose(gh["X"], g["X"][:, :, h:h + 1], rtol=1e-12, atol=1e-14)
    assert np.allclose(dB_sum, g["B"], rtol=1e-12, atol=1e-13)
    assert np.allclose(dC_sum, g["C"], rtol=1e-12, atol=1e-13)


def test_final_state_only(oracle_mod):
    """dY = 0: only the final state carries gradient.  Then dX_t = B_t . (decay
    from t+1 to the end) dh_out and dh0 = (total decay) dh_out."""
    inp, dY, dhv = case(5, 1, 9, 2, 3, 4, 1)
    dY[:] = 0.0
    g = grads(oracle_mod, inp, dY, dhv)
    ld = inp["logdecay"][0]                        # (L, H)
    L = ld.shape[0]
    for h in range(2):
        tot = np.exp(ld[:, h].sum())
        assert np.allclose(g["h0"][0, h], tot * dhv[0, h], rtol=1e-12)
        for t in range(L):
            w = np.exp(ld[t + 1:, h].sum())
            ref = w * (inp["B"][0, t, 0] @ dhv[0, h])
            assert np.allclose(g["X"][0, t, h], ref, rtol=1e-12, atol=1e-15)
    assert np.all(g["C"] == 0.0)
