"""Pins of the oracle's MIMO block composition (mimo_block): the B / C prologue
per rank row against torch's RMS normalisation, rank 1 against the SISO
block, invariance to a positive rescaling of any rank row, the epilogue's
special cases, and split-sequence chaining through the previous token's raw B."""
import numpy as np
import pytest

from selective_state_space_amd import workloads as wl


def test_prologue_per_rank_against_library_rms_norm(oracle_mod):
    """With z = None, D = None and no rotation, mimo_block is mimo on rows that
    torch's rms_norm over the state axis (per batch, step, head and rank) plus the
    head's bias produce."""
    import torch
    rng = np.random.default_rng(61)
    inp = wl.mimo_block_inputs(rng, 1, 9, 3, 4, 6, 3, h0_sd=0.2, rotate=False)
    D, z = inp.pop("D"), inp.pop("z")
    nb, nc, bb, bc = inp.pop("normB_w"), inp.pop("normC_w"), inp.pop("biasB"), inp.pop("biasC")
    Y, h = oracle_mod.mimo_block(**inp, normB_w=nb, normC_w=nc, biasB=bb, biasC=bc, eps=1e-3)

    def ref_rows(V, w, bias):
        t = torch.from_numpy(np.moveaxis(V, -1, -2).copy())          # (b, L, H, R, N)
        r = torch.nn.functional.rms_norm(t, (V.shape[-2],), torch.from_numpy(w), eps=1e-3).numpy()
        r = r + bias[None, None, :, None, :]
        return np.moveaxis(r, -1, -2)
    Yr, hr = oracle_mod.mimo(inp["X"], inp["logdecay"], ref_rows(inp["B"], nb, bb), ref_rows(inp["C"], nc, bc),
                             inp["beta"], inp["gamma"], None, inp["h0"])
    assert np.allclose(Y, Yr, rtol=1e-12, atol=1e-14) and np.allclose(h, hr, rtol=1e-12, atol=1e-14)


def test_rank_one_is_the_siso_block(oracle_mod):
    """R = 1 (the rank axis squeezed) is the SISO block with one group per head."""
    rng = np.random.default_rng(62)
    inp = wl.mimo_block_inputs(rng, 2, 70, 3, 8, 10, 1, h0_sd=0.2, prev=True)
    Y, h = oracle_mod.mimo_block(**inp, eps=1e-4)
    sq = {k: (v[..., 0] if k in ("X", "B", "C", "X_prev", "B_prev", "z") else v) for k, v in inp.items()}
    Ys, hs = oracle_mod.trap_block(**sq, eps=1e-4)
    assert np.allclose(Y[..., 0], Ys, rtol=1e-11, atol=1e-13) and np.allclose(h, hs, rtol=1e-11, atol=1e-13)


def test_rank_row_scale_invariance(oracle_mod):
    """Without bias and with eps -> 0, a positive rescaling of any (step, head,
    rank) row of B or C, and of the previous token's B, changes nothing."""
    rng = np.random.default_rng(63)
    inp = wl.mimo_block_inputs(rng, 1, 40, 2, 4, 8, 4, h0_sd=0.2, prev=True)
    inp.update(biasB=None, biasC=None, eps=1e-30)
    Y, h = oracle_mod.mimo_block(**inp)
    s1 = np.exp(rng.standard_normal((1, 40, 2, 1, 4)))
    s2 = np.exp(rng.standard_normal((1, 40, 2, 1, 4)))
    s3 = np.exp(rng.standard_normal((1, 2, 1, 4)))
    Y2, h2 = oracle_mod.mimo_block(**dict(inp, B=inp["B"] * s1, C=inp["C"] * s2, B_prev=inp["B_prev"] * s3))
    assert np.allclose(Y2, Y, rtol=1e-10, atol=1e-12) and np.allclose(h2, h, rtol=1e-10, atol=1e-12)
    # the bias comes after the norm: still invariant, and it matters
    bias = rng.standard_normal((2, 8))
    Yb, _ = oracle_mod.mimo_block(**dict(inp, biasB=bias))
    Yb2, _ = oracle_mod.mimo_block(**dict(inp, biasB=bias, B=inp["B"] * s1, B_prev=inp["B_prev"] * s3))
    assert np.allclose(Yb2, Yb, rtol=1e-10, atol=1e-12)
    assert not np.allclose(Yb, Y)


def test_epilogue_special_cases(oracle_mod):
    """z = 0 closes the gate (state unchanged); without z the skip term adds
    D[h] X_r to every rank; the gate matches scipy's logistic sigmoid times z."""
    from scipy.special import expit
    rng = np.random.default_rng(64)
    inp = wl.mimo_block_inputs(rng, 1, 20, 3, 4, 6, 2, h0_sd=0.2)
    D, z = inp.pop("D"), inp.pop("z")
    Y, h = oracle_mod.mimo_block(**inp)
    Yz, hz = oracle_mod.mimo_block(**inp, D=D, z=np.zeros_like(z))
    assert np.all(Yz == 0.0) and np.array_equal(hz, h)
    Yd, _ = oracle_mod.mimo_block(**inp, D=D)
    assert np.allclose(Yd - Y, D[None, None, :, None, None] * inp["X"], rtol=1e-13, atol=1e-15)
    Yg, _ = oracle_mod.mimo_block(**inp, D=D, z=z)
    assert np.allclose(Yg, (Y + D[None, None, :, None, None] * inp["X"]) * z * expit(z), rtol=1e-12, atol=1e-15)


def test_split_chains_through_the_raw_previous_token(oracle_mod):
    """A sequence split in two calls chains exactly when the second call gets
    h0 = the first's h_out and X_prev, B_prev = the first call's last X and raw
    (not normalised) B: the prologue runs on the previous token inside the call."""
    rng = np.random.default_rng(65)
    inp = wl.mimo_block_inputs(rng, 2, 50, 2, 4, 8, 4, h0_sd=0.3, prev=True)
    Y, h = oracle_mod.mimo_block(**inp, eps=1e-4)
    s = 23
    cut = lambda v, sl: v[:, sl]
    seq = ("X", "logdecay", "B", "C", "beta", "gamma", "theta", "z")
    a = {k: (cut(v, slice(0, s)) if k in seq else v) for k, v in inp.items()}
    Ya, ha = oracle_mod.mimo_block(**a, eps=1e-4)
    bpart = {k: (cut(v, slice(s, None)) if k in seq else v) for k, v in inp.items()}
    bpart.update(h0=ha, X_prev=inp["X"][:, s - 1], B_prev=inp["B"][:, s - 1])
    Yb, hb = oracle_mod.mimo_block(**bpart, eps=1e-4)
    assert np.allclose(np.concatenate([Ya, Yb], 1), Y, rtol=1e-11, atol=1e-13)
    assert np.allclose(hb, h, rtol=1e-11, atol=1e-13)
