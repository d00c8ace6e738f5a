"""Seeded synthetic inputs for the scans (shared by the tests and the bench).

This module only draws random numbers and applies the input recipes of the
workloads (softplus for step sizes, sigmoid for the trapezoid mix, the
alpha/beta/gamma coefficients the Mamba-3 configurations are defined with).  It
holds none of the scans' arithmetic.  Draws use ``numpy.random.default_rng``
(PCG64) in float64, in the order written in each function, so a seed fixes every
value; callers cast to the run dtype.

Workload recipes (shapes are the ones the pages' blocks use: d_model 768 with
expand 2 for Mamba-1, d_head 64 / d_state 128 for the SSD family):

* m1_tiny     seed 101: batch 1, L 64, D 16, N 4.
* m1_block    seed 102: batch 8, L 2048, D 1536, N 16.
* m1_decode   seed 106: batch 256, D 1536, N 16 (state ~ N(0, 0.1)).
* ssd_block   seed 103: batch 4, L 4096, H 24, P 64, N 128, G 1.
* siso_block  seed 104: as ssd_block, with trapezoid mix and rotary angles.
* mimo_block  seed 105: batch 2, L 8192, H 16, P 64, N 128, R 4.
* ssd_decode  seeds 107 (Mamba-2), 108 (SISO), 109 (MIMO): one token for 256
              sequences on the block shapes, state ~ N(0, 0.1).
* m1_fused    seed 110: the Mamba-1 block shapes with the block's prologue and
              epilogue inputs (conv1d width 4, dt bias, gate z).
* mimo_block_full  seed 118: the MIMO block shape with the block's B / C norm
              weights and biases, skip weight and gate.
"""
from __future__ import annotations

import numpy as np


def _softplus(v):
    return np.logaddexp(0.0, v)


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def s4d_real_A(D: int, N: int) -> np.ndarray:
    """A[c, n] = -(n + 1) for every channel (S4D-real initialisation)."""
    return -np.tile(np.arange(1, N + 1, dtype=np.float64), (D, 1))


# --------------------------------------------------------------------------
# Mamba-1
# --------------------------------------------------------------------------
def m1_inputs(rng, batch, L, D, N, dt_mu=-3.0, dt_sd=1.0, with_D=True,
              h0_sd=0.0, A=None):
    """Order: Dskip, x, B, C, dt, (h0)."""
    Dskip = rng.standard_normal(D) if with_D else None
    x = rng.standard_normal((batch, L, D))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    dt = _softplus(rng.normal(dt_mu, dt_sd, size=(batch, L, D)))
    h0 = rng.normal(0.0, h0_sd, size=(batch, D, N)) if h0_sd > 0 else None
    if A is None:
        A = s4d_real_A(D, N)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=Dskip, h0=h0)


def m1_tiny(seed=101):
    """batch 1, L 64, D 16, N 4; dt = softplus(N(-2, 0.5)).
    Order: x, B, C, dt, Dskip.  h0 = 0."""
    rng = np.random.default_rng(seed)
    b, L, D, N = 1, 64, 16, 4
    x = rng.standard_normal((b, L, D))
    B = rng.standard_normal((b, L, N))
    C = rng.standard_normal((b, L, N))
    dt = _softplus(rng.normal(-2.0, 0.5, size=(b, L, D)))
    Dskip = rng.standard_normal(D)
    return dict(x=x, dt=dt, A=s4d_real_A(D, N), B=B, C=C, D=Dskip, h0=None)


def m1_block(seed=102, batch=8, L=2048, D=1536, N=16):
    """batch 8, L 2048, D 1536, N 16; dt = softplus(N(-3, 1)).
    Order: Dskip (drawn first), x, B, C, dt.  h0 = 0."""
    rng = np.random.default_rng(seed)
    Dskip = rng.standard_normal(D)
    x = rng.standard_normal((batch, L, D))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    dt = _softplus(rng.normal(-3.0, 1.0, size=(batch, L, D)))
    return dict(x=x, dt=dt, A=s4d_real_A(D, N), B=B, C=C, D=Dskip, h0=None)


def m1_decode(seed=106, batch=256, D=1536, N=16, model_seed=102):
    """One batched decode step on the block model: A = -(n+1) and Dskip is the
    first draw of the block seed.  From `seed`: state ~ N(0, 0.1) (batch, D, N),
    x (batch, D), B, C (batch, N), dt = softplus(N(-3, 1)) (batch, D)."""
    Dskip = np.random.default_rng(model_seed).standard_normal(D)
    rng = np.random.default_rng(seed)
    h = rng.normal(0.0, 0.1, size=(batch, D, N))
    x = rng.standard_normal((batch, D))
    B = rng.standard_normal((batch, N))
    C = rng.standard_normal((batch, N))
    dt = _softplus(rng.normal(-3.0, 1.0, size=(batch, D)))
    return dict(x=x, dt=dt, A=s4d_real_A(D, N), B=B, C=C, D=Dskip, h=h)


# --------------------------------------------------------------------------
# Mamba-2 / Mamba-3
# --------------------------------------------------------------------------
def ssd_inputs(rng, batch, L, H, P, N, G=1, h0_sd=0.0):
    """X, B, C ~ N(0,1)/sqrt(N); A_h = -U(1,16); dt = softplus(N(-3,1));
    logdecay = dt * A_h.  Order: X, B, C, A_h, dt, (h0)."""
    s = 1.0 / np.sqrt(N)
    X = rng.standard_normal((batch, L, H, P)) * s
    B = rng.standard_normal((batch, L, G, N)) * s
    C = rng.standard_normal((batch, L, G, N)) * s
    A_h = -rng.uniform(1.0, 16.0, size=H)
    dt = _softplus(rng.normal(-3.0, 1.0, size=(batch, L, H)))
    ld = dt * A_h
    h0 = rng.normal(0.0, h0_sd, size=(batch, H, N, P)) if h0_sd > 0 else None
    return dict(X=X, logdecay=ld, B=B, C=C, h0=h0)


def ssd_block(seed=103, batch=4, L=4096, H=24, P=64, N=128, G=1):
    return ssd_inputs(np.random.default_rng(seed), batch, L, H, P, N, G)


def ssd_bwd_block(seed=111, batch=4, L=4096, H=24, P=64, N=128, G=1):
    """The Mamba-2 block inputs (seed 103) with the incoming gradients of the
    backward: dY ~ N(0,1) like X and dh_out ~ N(0,1) like the state."""
    d = ssd_block(batch=batch, L=L, H=H, P=P, N=N, G=G)
    rng = np.random.default_rng(seed)
    d["dY"] = rng.standard_normal((batch, L, H, P))
    d["dh_out"] = rng.standard_normal((batch, H, N, P))
    return d


def _trap_coeffs(rng, batch, L, H, N):
    """dt = softplus(N(-3,1)); A_h = -U(1,16); alpha = exp(dt*A_h);
    lambda = sigmoid(N(0,1)); gamma = lambda*dt; beta = (1-lambda)*dt*alpha;
    theta = U(0, pi) * dt (dt broadcast over N/2).  Order: dt, A_h, lambda,
    theta-uniforms."""
    dt = _softplus(rng.normal(-3.0, 1.0, size=(batch, L, H)))
    A_h = -rng.uniform(1.0, 16.0, size=H)
    ld = dt * A_h
    alpha = np.exp(ld)
    lam = _sigmoid(rng.standard_normal((batch, L, H)))
    gamma = lam * dt
    beta = (1.0 - lam) * dt * alpha
    theta = rng.uniform(0.0, np.pi, size=(batch, L, H, N // 2)) * dt[..., None]
    return ld, beta, gamma, theta


def trap_inputs(rng, batch, L, H, P, N, G=1, h0_sd=0.0, rotate=True):
    """Order: X, B, C, then the coefficients of _trap_coeffs, then (h0)."""
    s = 1.0 / np.sqrt(N)
    X = rng.standard_normal((batch, L, H, P)) * s
    B = rng.standard_normal((batch, L, G, N)) * s
    C = rng.standard_normal((batch, L, G, N)) * s
    ld, beta, gamma, theta = _trap_coeffs(rng, batch, L, H, N)
    h0 = rng.normal(0.0, h0_sd, size=(batch, H, N, P)) if h0_sd > 0 else None
    return dict(X=X, logdecay=ld, B=B, C=C, beta=beta, gamma=gamma,
                theta=theta if rotate else None, h0=h0)


def siso_block(seed=104, batch=4, L=4096, H=24, P=64, N=128, G=1):
    return trap_inputs(np.random.default_rng(seed), batch, L, H, P, N, G)


def siso_gated(seed=115, batch=4, L=4096, H=24, P=64, N=128, G=1):
    """The SISO block with its output epilogue: the skip weight D (H,) ~ N(0,1)
    and the gate z (b,L,H,P) ~ N(0,1), drawn after the scan inputs."""
    rng = np.random.default_rng(seed)
    inp = trap_inputs(rng, batch, L, H, P, N, G)
    inp["D"] = rng.standard_normal(H)
    inp["z"] = rng.standard_normal((batch, L, H, P))
    return inp


def siso_block_full(seed=116, batch=4, L=4096, H=24, P=64, N=128, G=1):
    """The SISO block with both ends: the scan inputs, then the B / C norm
    weights ~ 1 + N(0, 0.3^2) (N,), the biases ~ N(0, 0.5^2) (H, N), the skip
    weight D ~ N(0,1) (H,) and the gate z ~ N(0,1) like X."""
    rng = np.random.default_rng(seed)
    inp = trap_inputs(rng, batch, L, H, P, N, G)
    inp["normB_w"] = 1.0 + 0.3 * rng.standard_normal(N)
    inp["normC_w"] = 1.0 + 0.3 * rng.standard_normal(N)
    inp["biasB"] = 0.5 * rng.standard_normal((H, N))
    inp["biasC"] = 0.5 * rng.standard_normal((H, N))
    inp["D"] = rng.standard_normal(H)
    inp["z"] = rng.standard_normal((batch, L, H, P))
    return inp


def m2_prologue_inputs(rng, batch, L, H, P, G, N, K=4, hist=True):
    """The Mamba-2 block's projected channels xBC ~ N(0,1) (b, L, H P + 2 G N);
    conv_w ~ N(0, 1/K) (channels, K); conv_b ~ N(0, 0.1); raw dt ~ N(0, 0.5)
    (b, L, H); dt_bias = softplus^-1(U(0.001, 0.1)); A = -U(1, 16) per head;
    x_hist ~ N(0,1) (b, K-1, channels) or None."""
    cin = H * P + 2 * G * N
    xBC = rng.standard_normal((batch, L, cin))
    conv_w = rng.standard_normal((cin, K)) / np.sqrt(K)
    conv_b = rng.normal(0.0, 0.1, cin)
    dt = rng.normal(0.0, 0.5, (batch, L, H))
    dt_bias = np.log(np.expm1(rng.uniform(0.001, 0.1, H)))
    A = -rng.uniform(1.0, 16.0, H)
    x_hist = rng.standard_normal((batch, K - 1, cin)) if hist and K > 1 else None
    return dict(xBC=xBC, conv_w=conv_w, dt=dt, A=A, conv_b=conv_b, dt_bias=dt_bias, x_hist=x_hist)


def m2_block_full(seed=120, batch=4, L=4096, H=24, P=64, G=1, N=128, K=4):
    """The Mamba-2 layer at the block shape: the prologue inputs (m2_prologue_inputs,
    no history), then the skip weight D ~ N(0,1) (H,) and the gate z ~ N(0,1)
    (b, L, H, P); h0 = 0."""
    rng = np.random.default_rng(seed)
    i = m2_prologue_inputs(rng, batch, L, H, P, G, N, K, hist=False)
    i["D"] = rng.standard_normal(H)
    i["z"] = rng.standard_normal((batch, L, H, P))
    i["h0"] = None
    return i


def m2_prologue_block(seed=117, batch=4, L=4096, H=24, P=64, G=1, N=128, K=4):
    return m2_prologue_inputs(np.random.default_rng(seed), batch, L, H, P, G, N, K, hist=False)


def mimo_inputs(rng, batch, L, H, P, N, R, h0_sd=0.0, rotate=True):
    """Xr (b,L,H,P,R), Br, Cr (b,L,H,N,R) ~ N(0,1)/sqrt(N*R); then the SISO
    coefficients.  Order: X, B, C, coefficients, (h0)."""
    s = 1.0 / np.sqrt(N * R)
    X = rng.standard_normal((batch, L, H, P, R)) * s
    B = rng.standard_normal((batch, L, H, N, R)) * s
    C = rng.standard_normal((batch, L, H, N, R)) * s
    ld, beta, gamma, theta = _trap_coeffs(rng, batch, L, H, N)
    h0 = rng.normal(0.0, h0_sd, size=(batch, H, N, P)) if h0_sd > 0 else None
    return dict(X=X, logdecay=ld, B=B, C=C, beta=beta, gamma=gamma,
                theta=theta if rotate else None, h0=h0)


def mimo_block(seed=105, batch=2, L=8192, H=16, P=64, N=128, R=4):
    return mimo_inputs(np.random.default_rng(seed), batch, L, H, P, N, R)


def mimo_block_inputs(rng, batch, L, H, P, N, R, h0_sd=0.0, rotate=True, prev=False):
    """The MIMO inputs (mimo_inputs), then the block's parameters: B / C norm
    weights ~ 1 + N(0, 0.3^2) (N,), biases ~ N(0, 0.5^2) (H, N), the skip weight
    D ~ N(0,1) (H,), the gate z ~ N(0,1) like X, and with `prev` the previous
    token's X (b, H, P, R) and raw B (b, H, N, R) at the scale of X and B."""
    inp = mimo_inputs(rng, batch, L, H, P, N, R, h0_sd=h0_sd, rotate=rotate)
    inp["normB_w"] = 1.0 + 0.3 * rng.standard_normal(N)
    inp["normC_w"] = 1.0 + 0.3 * rng.standard_normal(N)
    inp["biasB"] = 0.5 * rng.standard_normal((H, N))
    inp["biasC"] = 0.5 * rng.standard_normal((H, N))
    inp["D"] = rng.standard_normal(H)
    inp["z"] = rng.standard_normal((batch, L, H, P, R))
    if prev:
        s = 1.0 / np.sqrt(N * R)
        inp["X_prev"] = rng.standard_normal((batch, H, P, R)) * s
        inp["B_prev"] = rng.standard_normal((batch, H, N, R)) * s
    return inp


def mimo_block_full(seed=118, batch=2, L=8192, H=16, P=64, N=128, R=4):
    """The MIMO block shape with both ends of the block (mimo_block_inputs)."""
    return mimo_block_inputs(np.random.default_rng(seed), batch, L, H, P, N, R)


def ssd_step_inputs(rng, batch, H, P, G, N, R, kind, h_sd=0.1):
    """One decode token of the SSD family.  kind "m2": X, B, C, logdecay and the
    state; "trap": also beta, gamma and the previous token's X, B; "rot": also
    the angle increments theta.  X, B, C ~ N(0,1)/sqrt(N R); dt = softplus(N(-3,1)),
    A_h = -U(1,16), logdecay = dt A_h; lambda = sigmoid(N(0,1)), beta = (1-lambda)
    dt alpha, gamma = lambda dt; theta = U(0, pi) dt; state ~ N(0, h_sd).
    Order: X, B, C, dt, A_h, state, then lambda, X_prev, B_prev, theta.  With
    R = 1 the rank axis is dropped."""
    s = 1.0 / np.sqrt(N * R)
    shp_x, shp_b = (batch, H, P, R), (batch, G, N, R)
    d = dict(X=rng.standard_normal(shp_x) * s, B=rng.standard_normal(shp_b) * s,
             C=rng.standard_normal(shp_b) * s)
    dt = _softplus(rng.normal(-3.0, 1.0, (batch, H)))
    ld = dt * -rng.uniform(1.0, 16.0, H)
    d["logdecay"] = ld
    d["h"] = rng.normal(0.0, h_sd, (batch, H, N, P))
    if kind != "m2":
        lam = _sigmoid(rng.standard_normal((batch, H)))
        d["beta"] = (1.0 - lam) * dt * np.exp(ld)
        d["gamma"] = lam * dt
        d["X_prev"] = rng.standard_normal(shp_x) * s
        d["B_prev"] = rng.standard_normal(shp_b) * s
        if kind == "rot":
            d["theta"] = rng.uniform(0.0, np.pi, (batch, H, N // 2)) * dt[..., None]
    if R == 1:
        for k in ("X", "B", "C", "X_prev", "B_prev"):
            if k in d:
                d[k] = d[k][..., 0]
    return d


def ssd_decode(model):
    """The decode workloads: 256 sequences on the block shapes.  "m2": H 24,
    P 64, N 128, G 1; "siso": the same with trapezoid and rotation; "mimo": H 16,
    P 64, N 128, R 4, with trapezoid and rotation."""
    if model == "m2":
        return ssd_step_inputs(np.random.default_rng(107), 256, 24, 64, 1, 128, 1, "m2")
    if model == "siso":
        return ssd_step_inputs(np.random.default_rng(108), 256, 24, 64, 1, 128, 1, "rot")
    if model == "mimo":
        return ssd_step_inputs(np.random.default_rng(109), 256, 16, 64, 16, 128, 4, "rot")
    raise ValueError(model)


def m1_block_inputs(rng, batch, L, D, N, K=4, h0_sd=0.0, hist=False):
    """Inputs of the Mamba-1 scan with the block prologue and epilogue: raw x ~
    N(0,1); conv_w ~ N(0, 1/K) (D, K); conv_b ~ N(0, 0.1); raw dt ~ N(0, 0.5) with
    dt_bias = softplus^-1(U(0.001, 0.1)) (so softplus(dt + bias) starts near the
    usual step sizes); B, C ~ N(0,1); D ~ N(0,1); gate z ~ N(0,1); A = -(n+1).
    Order: x, conv_w, conv_b, dt, dt_bias, B, C, D, z, (h0), (x_hist)."""
    x = rng.standard_normal((batch, L, D))
    conv_w = rng.normal(0.0, 1.0 / np.sqrt(K), (D, K))
    conv_b = rng.normal(0.0, 0.1, D)
    dt = rng.normal(0.0, 0.5, (batch, L, D))
    u = rng.uniform(0.001, 0.1, D)
    dt_bias = np.log(np.expm1(u))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    Dskip = rng.standard_normal(D)
    z = rng.standard_normal((batch, L, D))
    d = dict(x=x, conv_w=conv_w, conv_b=conv_b, dt=dt, dt_bias=dt_bias, A=s4d_real_A(D, N), B=B, C=C,
             D=Dskip, z=z, h0=None, x_hist=None)
    if h0_sd > 0:
        d["h0"] = rng.normal(0.0, h0_sd, (batch, D, N))
    if hist and K > 1:
        d["x_hist"] = rng.standard_normal((batch, K - 1, D))
    return d


def siso_bwd_block(seed=113):
    """The Mamba-3 SISO block inputs (seed 104) with the incoming gradients of
    the backward: dY ~ N(0,1) like X and dh_out ~ N(0,1) like the state."""
    d = siso_block()
    rng = np.random.default_rng(seed)
    b, L, H, P = d["X"].shape
    N = d["B"].shape[3]
    d["dY"] = rng.standard_normal((b, L, H, P))
    d["dh_out"] = rng.standard_normal((b, H, N, P))
    return d


def mimo_bwd_block(seed=114):
    """The Mamba-3 MIMO block inputs (seed 105) with the incoming gradients of
    the backward: dY ~ N(0,1) like X and dh_out ~ N(0,1) like the state."""
    d = mimo_block()
    rng = np.random.default_rng(seed)
    b, L, H, P, R = d["X"].shape
    N = d["B"].shape[3]
    d["dY"] = rng.standard_normal((b, L, H, P, R))
    d["dh_out"] = rng.standard_normal((b, H, N, P))
    return d


def m1_bwd_block(seed=112):
    """The Mamba-1 block inputs (seed 102) with the incoming gradients of the
    backward: dy ~ N(0,1) like x and dh_out ~ N(0,1) like the state."""
    d = m1_block()
    rng = np.random.default_rng(seed)
    b, L, D = d["x"].shape
    N = d["A"].shape[1]
    d["dy"] = rng.standard_normal((b, L, D))
    d["dh_out"] = rng.standard_normal((b, D, N))
    return d


def m1_fused(seed=110, batch=8, L=2048, D=1536, N=16, K=4):
    return m1_block_inputs(np.random.default_rng(seed), batch, L, D, N, K)
