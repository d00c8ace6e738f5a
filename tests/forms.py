"""Alternate fp64 numpy forms used only to pin the oracle.

Each form computes the same result as an oracle loop by a different route that
the pages name: the matrix (quadratic / dual) forms, the chunkwise form, the
two-SSD decomposition, the physical-frame step, the R^2-SISO expansion of MIMO,
and the zero-order-hold alternative that must *differ* from the
exponential-Euler scan.  None of these forms is part of the oracle, and none is
used against the GPU.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Mamba-1
# --------------------------------------------------------------------------
def m1_matrix(x, dt, A, B, C, D=None, h0=None):
    """Dense lower-triangular form of the Mamba-1 scan (TorchMamba README,
    `selective_scan_matrix`; guarded at L <= 32 like the original):
        y_t[c] = sum_{s<=t} sum_n C_t[n] exp(A[c,n] (cum_t - cum_s)) dt_s B_s[n] x_s
               + sum_n C_t[n] exp(A[c,n] cum_t) h0[c,n] + D[c] x_t
    with cum_t = sum_{r<=t} dt_r (inclusive)."""
    b, L, Dm = x.shape
    if L > 32:
        raise ValueError("matrix form is limited to L <= 32")
    N = A.shape[1]
    y = np.zeros((b, L, Dm))
    h = np.zeros((b, Dm, N))
    tri = np.tril(np.ones((L, L)))
    for bb in range(b):
        cum = np.cumsum(dt[bb], axis=0)                       # (L, D)
        diff = cum[:, None, :] - cum[None, :, :]              # (t, s, D)
        dec = np.exp(diff[..., None] * A[None, None, :, :])   # (t, s, D, N)
        dec *= tri[:, :, None, None]
        u = dt[bb][:, :, None] * B[bb][:, None, :] * x[bb][:, :, None]  # (s, D, N)
        y[bb] = np.einsum("tn,tsdn,sdn->td", C[bb], dec, u)
        h[bb] = np.einsum("sdn,sdn->dn", dec[L - 1], u)
        if h0 is not None:
            g = np.exp(cum[:, :, None] * A[None])            # (t, D, N)
            y[bb] += np.einsum("tn,tdn,dn->td", C[bb], g, h0[bb])
            h[bb] += g[L - 1] * h0[bb]
        if D is not None:
            y[bb] += D[None, :] * x[bb]
    return y, h


def m1_zoh(x, dt, A, B, C, D=None):
    """Zero-order-hold alternative: Bbar = (exp(dt A) - 1) / A * B.  The pages
    name it as the documented alternative that the exponential-Euler scan must
    not silently become (TorchMamba README, Math notes M1)."""
    b, L, Dm = x.shape
    N = A.shape[1]
    y = np.zeros((b, L, Dm))
    h = np.zeros((b, Dm, N))
    for t in range(L):
        a = np.exp(dt[:, t, :, None] * A[None])
        bbar = (a - 1.0) / A[None] * B[:, t, None, :]
        h = a * h + bbar * x[:, t, :, None]
        y[:, t] = np.einsum("bdn,bn->bd", h, C[:, t])
        if D is not None:
            y[:, t] += D[None] * x[:, t]
    return y, h


# --------------------------------------------------------------------------
# Mamba-2
# --------------------------------------------------------------------------
def _group_index(H, G):
    return np.arange(H) // (H // G)


def ssd_quadratic(X, logdecay, B, C, h0=None):
    """Quadratic dual form (TorchMamba README, Math notes M2 citing the SSD
    paper's Eq. 16; `ssd_quadratic`, guarded at L <= 512):
        Y = (Lmask o C B^T) X + diag(exp(cum)) C h0,
        Lmask[i, j] = exp(cum_i - cum_j) for i >= j, else 0."""
    ld = logdecay
    b, L, H, P = X.shape
    if L > 512:
        raise ValueError("quadratic form is limited to L <= 512")
    G, N = B.shape[2], B.shape[3]
    gi = _group_index(H, G)
    Y = np.zeros_like(X)
    h = np.zeros((b, H, N, P))
    tri = np.tril(np.ones((L, L), dtype=bool))
    for bb in range(b):
        for hh in range(H):
            g = gi[hh]
            cum = np.cumsum(ld[bb, :, hh])
            Lm = np.where(tri, np.exp(np.where(tri, cum[:, None] - cum[None, :], 0.0)), 0.0)
            Bg, Cg, Xh = B[bb, :, g], C[bb, :, g], X[bb, :, hh]
            Y[bb, :, hh] = (Lm * (Cg @ Bg.T)) @ Xh
            w = np.exp(cum[-1] - cum) if L else np.zeros(0)
            h[bb, hh] = (Bg * w[:, None]).T @ Xh
            if h0 is not None:
                Y[bb, :, hh] += np.exp(cum)[:, None] * (Cg @ h0[bb, hh])
                h[bb, hh] += (np.exp(cum[-1]) if L else 1.0) * h0[bb, hh]
    return Y, h


def ssd_chunkwise(X, logdecay, B, C, h0=None, Q=64):
    """Chunkwise form (TorchMamba README, Math notes M2: intra-chunk quadratic
    plus an inter-chunk carry factored through B, the decay and C):
    for each chunk of Q steps (the last may be shorter)
        intra:  Y_c = (Lmask_c o C_c B_c^T) X_c
        state:  S_c = sum_j exp(cum_last - cum_j) B_j (x) X_j
        carry:  H_{c+1} = exp(cum_last) H_c + S_c,   H_0 = h0
        output: Y_c += diag(exp(cum)) C_c H_c
    with cum restarting at 0 in every chunk."""
    ld = logdecay
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    gi = _group_index(H, G)
    Y = np.zeros_like(X)
    hout = np.zeros((b, H, N, P))
    for bb in range(b):
        for hh in range(H):
            g = gi[hh]
            Hs = np.zeros((N, P)) if h0 is None else h0[bb, hh].copy()
            for c0 in range(0, L, Q):
                c1 = min(c0 + Q, L)
                cum = np.cumsum(ld[bb, c0:c1, hh])
                n = c1 - c0
                tri = np.tril(np.ones((n, n), dtype=bool))
                Lm = np.where(tri, np.exp(np.where(tri, cum[:, None] - cum[None, :], 0.0)), 0.0)
                Bc, Cc, Xc = B[bb, c0:c1, g], C[bb, c0:c1, g], X[bb, c0:c1, hh]
                Yc = (Lm * (Cc @ Bc.T)) @ Xc
                Yc += np.exp(cum)[:, None] * (Cc @ Hs)
                Y[bb, c0:c1, hh] = Yc
                w = np.exp(cum[-1] - cum)
                Hs = np.exp(cum[-1]) * Hs + (Bc * w[:, None]).T @ Xc
            hout[bb, hh] = Hs
    return Y, hout


def ssd_step(X_t, ld_t, B_t, C_t, S):
    """One SSD step: S <- exp(ld) S + B (x) X; Y = S^T C.  X_t (b,H,P),
    ld_t (b,H), B_t, C_t (b,G,N), S (b,H,N,P)."""
    b, H, P = X_t.shape
    G = B_t.shape[1]
    gi = _group_index(H, G)
    Bh, Ch = B_t[:, gi], C_t[:, gi]                     # (b, H, N)
    S = np.exp(ld_t)[..., None, None] * S + Bh[..., :, None] * X_t[..., None, :]
    Y = np.einsum("bhnp,bhn->bhp", S, Ch)
    return Y, S


# --------------------------------------------------------------------------
# Mamba-3 SISO
# --------------------------------------------------------------------------
def rot_pairs(v, phi, sign=1.0):
    """Rotate consecutive pairs of the last axis of v by phi (broadcast over
    leading axes, phi has shape v.shape[:-1] + (N/2,))."""
    c, s = np.cos(phi), sign * np.sin(phi)
    v0, v1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = c * v0 - s * v1
    out[..., 1::2] = s * v0 + c * v1
    return out


def rotated_BC(B, C, theta, H):
    """Per-head rotated B~, C~ (b, L, H, N) with Theta = inclusive cumsum."""
    G = B.shape[2]
    gi = _group_index(H, G)
    Bh, Ch = B[:, :, gi], C[:, :, gi]
    if theta is None:
        return Bh.copy(), Ch.copy(), None
    Th = np.cumsum(theta, axis=1)
    return rot_pairs(Bh, Th), rot_pairs(Ch, Th), Th


def trap_matrix(X, logdecay, B, C, beta, gamma, theta=None, h0=None):
    """Parallel mask form of the SISO recurrence (TorchMamba README, Math notes
    M3 SISO: the mask is the product of the 1-semiseparable decay matrix with a
    two-band matrix; `trap_rope_matrix`, guarded at L <= 16):
        M[t, u] = A(t,u) gamma_u + [u < t] A(t,u+1) beta_{u+1},
        A(t,u) = exp(sum_{r=u+1..t} ld_r),
        Y_t = sum_u M[t,u] (C~_t . B~_u) X_u + exp(cum_t) h0^T C~_t."""
    ld = logdecay
    b, L, H, P = X.shape
    if L > 16:
        raise ValueError("matrix form is limited to L <= 16")
    N = B.shape[3]
    Bt, Ct, Th = rotated_BC(B, C, theta, H)
    Y = np.zeros_like(X)
    hout = np.zeros((b, H, N, P))
    for bb in range(b):
        for hh in range(H):
            cum = np.cumsum(ld[bb, :, hh])
            Adec = np.zeros((L, L + 1))
            for t in range(L):
                for u in range(t + 1):
                    Adec[t, u] = np.exp(cum[t] - cum[u])
            # one-semiseparable decay times the two-band (gamma, beta) matrix
            band = np.zeros((L, L))
            for u in range(L):
                band[u, u] = gamma[bb, u, hh]
                if u + 1 < L:
                    band[u + 1, u] = beta[bb, u + 1, hh]
            M = Adec[:, :L] @ band
            M = np.tril(M)
            Sc = Ct[bb, :, hh] @ Bt[bb, :, hh].T
            Y[bb, :, hh] = (M * Sc) @ X[bb, :, hh]
            Sfin = (Bt[bb, :, hh] * M[L - 1][:, None]).T @ X[bb, :, hh]
            if h0 is not None:
                Y[bb, :, hh] += np.exp(cum)[:, None] * (Ct[bb, :, hh] @ h0[bb, hh])
                Sfin += np.exp(cum[-1]) * h0[bb, hh]
            if Th is not None:
                Sfin = rot_pairs(Sfin.T, Th[bb, L - 1, hh], -1.0).T
            hout[bb, hh] = Sfin
    return Y, hout


def trap_two_ssd(X, logdecay, B, C, beta, gamma, theta=None, h0=None, Q=None):
    """Two-SSD decomposition (mamba3-minimal README, "Two-SSD Decomposition"):
    Y = ssd(gamma X, ld, B~, C~; h0) + ssd(beta X_prev, ld, B~_prev, C~; 0)
    with X_prev, B~_prev shifted by one step over the whole sequence (zero at
    t = 0) before any chunking.  The states add; the sum is de-rotated."""
    ld = logdecay
    b, L, H, P = X.shape
    Bt, Ct, Th = rotated_BC(B, C, theta, H)
    Xg = X * gamma[..., None]
    Xp = np.zeros_like(X)
    Xp[:, 1:] = X[:, :-1]
    Xp *= beta[..., None]
    Bp = np.zeros_like(Bt)
    Bp[:, 1:] = Bt[:, :-1]
    run = (lambda *a: ssd_chunkwise(*a, Q=Q)) if Q else ssd_quadratic
    Y1, h1 = run(Xg, ld, Bt, Ct, h0)
    Y2, h2 = run(Xp, ld, Bp, Ct, None)
    S = h1 + h2
    if Th is not None and L:
        S = np.swapaxes(rot_pairs(np.swapaxes(S, -1, -2), Th[:, L - 1][:, :, None, :], -1.0), -1, -2)
    return Y1 + Y2, S


def trap_physical_step_loop(X, logdecay, B, C, beta, gamma, theta=None, h0=None):
    """Physical-frame SISO loop with unrotated B, C and no cumulative angle:
        S_t = R(-theta_t) (alpha_t S_{t-1} + beta_t B_{t-1} (x) X_{t-1})
              + gamma_t B_t (x) X_t,        Y_t = S_t^T C_t.
    Equal to the rotated-frame loop because rotations compose additively."""
    ld = logdecay
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    gi = _group_index(H, G)
    S = np.zeros((b, H, N, P)) if h0 is None else h0.copy()
    Bprev = np.zeros((b, H, N))
    Xprev = np.zeros((b, H, P))
    Y = np.zeros_like(X)
    for t in range(L):
        Bt, Ct, Xt = B[:, t][:, gi], C[:, t][:, gi], X[:, t]
        a = np.exp(ld[:, t])[..., None, None]
        inner = a * S + beta[:, t][..., None, None] * Bprev[..., :, None] * Xprev[..., None, :]
        if theta is not None:
            inner = np.swapaxes(rot_pairs(np.swapaxes(inner, -1, -2), theta[:, t][:, :, None, :], -1.0), -1, -2)
        S = inner + gamma[:, t][..., None, None] * Bt[..., :, None] * Xt[..., None, :]
        Y[:, t] = np.einsum("bhnp,bhn->bhp", S, Ct)
        Bprev, Xprev = Bt, Xt
    return Y, S


# --------------------------------------------------------------------------
# Mamba-3 MIMO
# --------------------------------------------------------------------------
def mimo_physical_step_loop(X, logdecay, B, C, beta, gamma, theta=None, h0=None):
    """Physical-frame MIMO loop: the rank sums enter like the SISO terms,
        S_t = R(-theta_t)(alpha S + beta sum_r B_{t-1,r} (x) X_{t-1,r})
              + gamma sum_r B_{t,r} (x) X_{t,r},     Y_{t,r} = S_t^T C_{t,r}."""
    ld = logdecay
    b, L, H, P, R = X.shape
    N = B.shape[3]
    S = np.zeros((b, H, N, P)) if h0 is None else h0.copy()
    prev = np.zeros((b, H, N, P))
    Y = np.zeros_like(X)
    for t in range(L):
        cur = np.einsum("bhnr,bhpr->bhnp", B[:, t], X[:, t])
        a = np.exp(ld[:, t])[..., None, None]
        inner = a * S + beta[:, t][..., None, None] * prev
        if theta is not None:
            inner = np.swapaxes(rot_pairs(np.swapaxes(inner, -1, -2), theta[:, t][:, :, None, :], -1.0), -1, -2)
        S = inner + gamma[:, t][..., None, None] * cur
        Y[:, t] = np.einsum("bhnp,bhnr->bhpr", S, C[:, t])
        prev = cur
    return Y, S
