#!/usr/bin/env python3
"""Benchmark of the selective state-space scans on one MI355X.

One *step* runs every scan of the library once on its workload, with inputs
already resident in HBM:

  m1_scan    Mamba-1 selective scan, batch 8, L 2048, D 1536, N 16, fp32
  m1_step    Mamba-1 decode step, 256 sequences, D 1536, N 16, fp32, in place
  ssd_f32    Mamba-2 SSD, batch 4, L 4096, H 24, P 64, N 128, G 1, fp32
  ssd_bf16   the same with bf16 X/B/C/Y (bf16 matrix operands, fp32
             accumulation and state)
  siso       Mamba-3 SISO trapezoid + rotations, shapes of ssd_f32, fp32
  mimo       Mamba-3 MIMO rank 4, batch 2, L 8192, H 16, P 64, N 128, fp32

The printed metric is scanned tokens per second over the whole step (a token
is one (batch, time) position of a workload; the decode step counts its 256
sequences).  Per-workload times come from HIP events recorded on the stream the
kernels run on, over the same timed steps.  The `roofline` object is for the
workload whose kernels take the largest share of the step; `kernels` lists
every workload.  `cpu_baseline` times the fp64 oracle on a bounded sample of the
same workloads on the host cores.  `next` times, beside the step and outside its
token count, the decode steps of the SSD family (one token for 256 sequences:
Mamba-2, SISO and MIMO on the block shapes; bound by HBM).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only a,b] [--no-cpu] [--no-next]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 (vector and MFMA)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
VALU_F32_LANE_OPS = 256 * 2.4e9 * 64   # non-packed fp32 VALU lane-ops/s (256 CU x 2.4 GHz x 64 lanes)
# Minimal VALU issue slots per Mamba-1 (t, c, n) element: dt*A (1), exp (2: the
# transcendental unit runs at half rate), (dt*x)*B (1), a*h + u (1), y += C*h (1).
M1_SLOTS_PER_ELEM = 6


# ----------------------------------------------------------------------------
# algorithmic work per workload (bytes: each input read once, each output
# written once; flops at the canonical chunk length 64, causal half only)
# ----------------------------------------------------------------------------
def m1_scan_work(b, L, D, N, es=4):
    nbytes = es * (3 * b * L * D + 2 * b * L * N) + 4 * (D * N + D + b * D * N)
    return nbytes, b * L * D * N      # (bytes, exp count)


# Minimal VALU issue slots per (t, c, n) element of the Mamba-1 backward: the
# recomputed forward (6) and the adjoint step: G += C dy, dB and dC products,
# U += G B, exp (2) and its argument, G a h_prev (2), V += A w, dA += dt w,
# G *= a (12).
M1_BWD_SLOTS_PER_ELEM = 18


def m1_bwd_work(b, L, D, N):
    """x, dt, dy, B, C, A, Dskip, dh_out read and dx, ddt, dB, dC, dA, dDskip, dh0
    written once; (bytes, elements)."""
    nbytes = 4 * (5 * b * L * D + 4 * b * L * N + 2 * b * D * N + 2 * D * N + 2 * D)
    return nbytes, b * L * D * N


def m1_step_work(b, D, N, es=4):
    nbytes = 4 * (2 * b * D * N) + es * (3 * b * D + 2 * b * N) + 4 * (D * N + D)
    return nbytes, b * D * N


def ssd_work(b, L, H, P, N, G, es=4, Q=64):
    nbytes = es * (2 * b * L * H * P + 2 * b * L * G * N) + 4 * (b * L * H + b * H * N * P)
    flops = b * L * H * (4 * N * P + P * (Q + 1) + N * (Q + 1) * G / H)
    return nbytes, flops


def siso_work(b, L, H, P, N, G, Q=64):
    nbytes = 4 * (2 * b * L * H * P + 2 * b * L * G * N + 3 * b * L * H + b * L * H * N // 2 + b * H * N * P)
    flops = b * L * H * (4 * N * P + P * (Q + 1) + N * (Q + 1))
    return nbytes, flops


def mimo_work(b, L, H, P, N, R, Q=64):
    Qt = Q // R
    nbytes = 4 * (2 * b * L * H * P * R + 2 * b * L * H * N * R + 3 * b * L * H + b * L * H * N // 2 + b * H * N * P)
    flops = b * L * H * (4 * N * P * R + R * R * (Qt + 1) * (N + P))
    return nbytes, flops


def ssd_bwd_work(b, L, H, P, N, G, Q=64):
    """Backward of the Mamba-2 SSD: inputs X, dY, logdecay, B, C, dh_out read and
    dX, dlogdecay, dB, dC, dh0 written once; flops of the chunkwise form at
    Q = 64 (causal halves): the chunk-local states U and V (4NP), the state
    products dY H^T, B G, X G^T (6NP), dY X^T and its two uses (2P(Q+1) + 2N(Q+1)
    less the shared C B^T, N(Q+1) G/H)."""
    nbytes = 4 * (2 * 2 * b * L * H * P + 2 * 2 * b * L * G * N + 2 * b * L * H + 2 * b * H * N * P)
    flops = b * L * H * (10 * N * P + 2 * P * (Q + 1) + 2 * N * (Q + 1) + N * (Q + 1) * G / H)
    return nbytes, flops


def siso_bwd_work(b, L, H, P, N, G, Q=64):
    """Backward of the Mamba-3 SISO recurrence: inputs X, dY, B, C, logdecay,
    beta, gamma, theta, dh_out read and their gradients written once; flops of
    the chunkwise form of the two-term (trapezoid) SSD at Q = 64: local states
    (6NP), the state products for both terms (10NP), the scores and masked
    products of both terms (4P(Q+1) + 6N(Q+1)).  The library runs it as a
    one-term SSD over 2L interleaved steps (about 17% more flops)."""
    nbytes = 4 * (4 * b * L * H * P + 4 * b * L * G * N + 6 * b * L * H + b * L * H * N + 2 * b * H * N * P)
    flops = b * L * H * (16 * N * P + 4 * P * (Q + 1) + 6 * N * (Q + 1))
    return nbytes, flops


def mimo_bwd_work(b, L, H, P, N, R, Q=64):
    """Backward of the Mamba-3 MIMO recurrence: inputs and their gradients moved
    once; flops of the chunkwise two-term rank-R form (Q rows, Q/R steps per
    chunk): 16NPR for the local states and the state products, R^2 (Q/R + 1)
    (4P + 6N) for the scores and masked products.  With R = 1 this is the SISO
    count.  The library runs it as a one-term SSD over (3R - 1) L rows."""
    Qt = Q // R
    nbytes = 4 * (3 * b * L * H * P * R + 4 * b * L * H * N * R + 6 * b * L * H + b * L * H * N + 2 * b * H * N * P)
    flops = b * L * H * (16 * N * P * R + R * R * (Qt + 1) * (4 * P + 6 * N))
    return nbytes, flops


def ssd_step_work(b, H, P, N, G, R, trap, rot, es=4):
    """One decode token: the fp32 state read and written once, plus the token's
    inputs and output."""
    nbytes = 4 * 2 * b * H * N * P + es * (2 * b * H * P * R + 2 * b * G * N * R) + 4 * b * H
    if trap:
        nbytes += es * (b * H * P * R + b * G * N * R) + 4 * 2 * b * H
    if rot:
        nbytes += 4 * b * H * (N // 2)
    return nbytes


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
class Workload:
    name = ""
    tokens = 0
    bound = "hbm"

    def run(self):
        raise NotImplementedError


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


class M1Scan(Workload):
    name = "m1_scan"
    kernel = "k_m1_scan"
    bound = "alu"
    source = "selective_state_space_amd/csrc/m1.hip"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, D, N = 8, 2048, 1536, 16
        self.shape = dict(batch=b, L=L, D=D, N=N)
        inp = wl.m1_block()
        self.inp = inp
        f = torch.float32
        self.x, self.dt, self.B, self.C = (_dev(inp[k], f) for k in ("x", "dt", "B", "C"))
        self.A, self.D = _dev(inp["A"], f), _dev(inp["D"], f)
        self.y = torch.empty_like(self.x)
        self.h = torch.empty((b, D, N), dtype=f, device="cuda")
        self.tokens = b * L
        self.bytes, self.exps = m1_scan_work(b, L, D, N)
        self.flops = None

    def run(self):
        self.mb.mb_selective_scan(self.x, self.dt, self.A, self.B, self.C, self.D, None, y=self.y, h_out=self.h)


class M1Fused(Workload):
    """The Mamba-1 scan with the block prologue and epilogue in the same kernel
    (conv1d + SiLU, softplus of dt plus bias, SiLU gate); outside the step,
    measured beside it.  Its ALU count is the scan's alone (the prologue adds a
    few operations per (t, c), not per state), so the fraction is a lower bound."""
    name = "m1_fused"
    kernel = "k_m1_scan_w"
    bound = "alu"
    source = "selective_state_space_amd/csrc/m1.hip"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        inp = wl.m1_fused()
        self.inp = inp
        b, L, D = inp["x"].shape
        N, K = inp["A"].shape[1], inp["conv_w"].shape[1]
        self.shape = dict(batch=b, L=L, D=D, N=N, K=K)
        f = torch.float32
        self.t = {k: (_dev(v, f) if v is not None else None) for k, v in inp.items()}
        self.y = torch.empty_like(self.t["x"])
        self.h = torch.empty((b, D, N), dtype=f, device="cuda")
        self.tokens = b * L
        nbytes, self.exps = m1_scan_work(b, L, D, N)
        self.bytes = nbytes + 4 * (b * L * D + D * (K + 2))   # the gate z, conv_w, conv_b, dt_bias
        self.flops = None

    def run(self):
        t = self.t
        self.mb.mb_selective_scan_fused(t["x"], t["conv_w"], t["dt"], t["A"], t["B"], t["C"], t["D"], None,
                                        conv_b=t["conv_b"], dt_bias=t["dt_bias"], z=t["z"], y=self.y,
                                        h_out=self.h)


class M1Step(Workload):
    name = "m1_step"
    kernel = "k_m1_step_q"
    source = "selective_state_space_amd/csrc/m1.hip"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, D, N = 256, 1536, 16
        self.shape = dict(batch=b, D=D, N=N)
        inp = wl.m1_decode()
        self.inp = inp
        f = torch.float32
        self.x, self.dt, self.B, self.C = (_dev(inp[k], f) for k in ("x", "dt", "B", "C"))
        self.A, self.D = _dev(inp["A"], f), _dev(inp["D"], f)
        self.h = _dev(inp["h"], f)
        self.y = torch.empty_like(self.x)
        self.tokens = b
        self.bytes, self.exps = m1_step_work(b, D, N)
        self.flops = None

    def run(self):
        self.mb.mb_ssm_step(self.x, self.dt, self.A, self.B, self.C, self.D, self.h, y=self.y)


class SSD(Workload):
    kernel = "k_scores + k_walk (state-only pass) + k_walk_m2s (full pass)"
    source = "selective_state_space_amd/csrc/ssd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch, dtype):
        self.mb = mb
        self.name = "ssd_" + dtype
        b, L, H, P, N, G = 4, 4096, 24, 64, 128, 1
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, G=G)
        inp = wl.ssd_block()
        self.inp = inp
        act = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.X, self.B, self.C = (_dev(inp[k], act) for k in ("X", "B", "C"))
        self.ld = _dev(inp["logdecay"], torch.float32)
        self.Y = torch.empty_like(self.X)
        self.h = torch.empty((b, H, N, P), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, b, L, H, P, G, N, 1, 0),
                              dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        es = 2 if dtype == "bf16" else 4
        self.bytes, self.flops = ssd_work(b, L, H, P, N, G, es)
        self.exps = None
        self.dtype = dtype
        if dtype == "bf16":
            self.bound = "hbm"
            self.kernel = "k_scores + k_walk_bf (state-only pass) + k_walk_bf (full pass)"

    def run(self):
        self.mb.mb_ssd_chunked(self.X, self.ld, self.B, self.C, None, Y=self.Y, h_out=self.h, ws=self.ws)


class M1Bwd(Workload):
    """Backward of the Mamba-1 scan at the block shape (outside the step,
    measured beside it)."""
    name = "m1_bwd"
    kernel = "k_m1_scan_w (checkpoints) + k_m1_bwd + k_m1_bwd_reduce"
    source = "selective_state_space_amd/csrc/m1.hip"
    bound = "alu"
    slots = M1_BWD_SLOTS_PER_ELEM

    def __init__(self, mb, wl, torch):
        self.mb = mb
        inp = wl.m1_bwd_block()
        self.inp = inp
        b, L, D = inp["x"].shape
        N = inp["A"].shape[1]
        self.shape = dict(batch=b, L=L, D=D, N=N)
        self.t = {k: _dev(v, torch.float32) for k, v in inp.items() if v is not None}
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN_BWD, b, L, D, 1, 1, N),
                              dtype=torch.uint8, device="cuda")
        t = self.t
        self.out = dict(dx=torch.empty_like(t["x"]), ddt=torch.empty_like(t["x"]), dA=torch.empty_like(t["A"]),
                        dB=torch.empty_like(t["B"]), dC=torch.empty_like(t["C"]), dD=torch.empty_like(t["D"]),
                        dh0=torch.empty_like(t["dh_out"]))
        self.tokens = b * L
        self.bytes, self.exps = m1_bwd_work(b, L, D, N)
        self.flops = None

    def run(self):
        t = self.t
        self.mb.mb_selective_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["dy"], t["D"], None, t["dh_out"],
                                      ws=self.ws, **self.out)


class SSDBwd(Workload):
    """Backward of the Mamba-2 SSD at the block shape (outside the step, measured
    beside it)."""
    name = "ssd_bwd"
    kernel = "k_bwd_local + k_bwd_pass + k_bwd_grad + k_bwd_ld"
    source = "selective_state_space_amd/csrc/ssd_bwd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, N, G = 4, 4096, 24, 64, 128, 1
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, G=G)
        inp = wl.ssd_bwd_block()
        self.inp = inp
        self.t = {k: _dev(v, torch.float32) for k, v in inp.items() if v is not None}
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED_BWD, b, L, H, P, G, N),
                              dtype=torch.uint8, device="cuda")
        t = self.t
        self.out = dict(dX=torch.empty_like(t["X"]), dlogdecay=torch.empty_like(t["logdecay"]),
                        dB=torch.empty_like(t["B"]), dC=torch.empty_like(t["C"]), dh0=torch.empty_like(t["dh_out"]))
        self.tokens = b * L
        self.bytes, self.flops = ssd_bwd_work(b, L, H, P, N, G)
        self.exps = None

    def run(self):
        t = self.t
        self.mb.mb_ssd_chunked_bwd(t["X"], t["logdecay"], t["B"], t["C"], t["dY"], None, t["dh_out"], ws=self.ws,
                                   **self.out)


class SISOBwd(Workload):
    """Backward of the Mamba-3 SISO recurrence at the block shape (outside the
    step, measured beside it)."""
    name = "siso_bwd"
    kernel = "angle and interleave kernels + the SSD backward over 2L steps + the mapping back"
    source = "selective_state_space_amd/csrc/ssd_bwd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, N, G = 4, 4096, 24, 64, 128, 1
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, G=G, trapezoid=True, rotation=True)
        inp = wl.siso_bwd_block()
        self.inp = inp
        self.t = {k: _dev(v, torch.float32) for k, v in inp.items() if v is not None}
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_TRAP_SSD_BWD, b, L, H, P, G, N),
                              dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        self.bytes, self.flops = siso_bwd_work(b, L, H, P, N, G)
        self.exps = None

    def run(self):
        t = self.t
        self.mb.mb_trap_ssd_bwd(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["dY"], t["theta"],
                                None, t["dh_out"], ws=self.ws)


class MIMOBwd(Workload):
    """Backward of the Mamba-3 MIMO recurrence at the block shape (outside the
    step, measured beside it)."""
    name = "mimo_bwd"
    kernel = "angle and row kernels + the SSD backward over (3R - 1) L rows + the mapping back"
    source = "selective_state_space_amd/csrc/ssd_bwd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, N, R = 2, 8192, 16, 64, 128, 4
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, R=R, trapezoid=True, rotation=True)
        inp = wl.mimo_bwd_block()
        self.inp = inp
        self.t = {k: _dev(v, torch.float32) for k, v in inp.items() if v is not None}
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_MIMO_SSD_BWD, b, L, H, P, 1, N, R),
                              dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        self.bytes, self.flops = mimo_bwd_work(b, L, H, P, N, R)
        self.exps = None

    def run(self):
        t = self.t
        self.mb.mb_mimo_ssd_bwd(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["dY"], t["theta"],
                                None, t["dh_out"], ws=self.ws)


class SISO(Workload):
    name = "siso"
    kernel = "k_walk (state-only pass) + k_walk (full pass)"
    source = "selective_state_space_amd/csrc/ssd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, N, G = 4, 4096, 24, 64, 128, 1
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, G=G)
        inp = wl.siso_block()
        self.inp = inp
        f = torch.float32
        self.t = {k: _dev(inp[k], f) for k in ("X", "logdecay", "B", "C", "beta", "gamma", "theta")}
        self.Y = torch.empty_like(self.t["X"])
        self.h = torch.empty((b, H, N, P), dtype=f, device="cuda")
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_TRAP_SSD, b, L, H, P, G, N, 1, 0),
                              dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        self.bytes, self.flops = siso_work(b, L, H, P, N, G)
        self.exps = None

    def run(self):
        t = self.t
        self.mb.mb_trap_ssd(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["theta"], None,
                            Y=self.Y, h_out=self.h, ws=self.ws)


class SISOGated(SISO):
    """Mamba-3 SISO with the block's output epilogue (skip term D[h] X and the
    SiLU(z) gate) fused into the scan's store; outside the step, measured beside
    it.  Bytes add the gate z; flops are the scan's (the epilogue adds a few
    operations per output)."""
    name = "siso_gated"

    def __init__(self, mb, wl, torch):
        super().__init__(mb, wl, torch)
        inp = wl.siso_gated()
        self.inp = inp
        f = torch.float32
        self.t = {k: _dev(inp[k], f) for k in ("X", "logdecay", "B", "C", "beta", "gamma", "theta", "D", "z")}
        b, L, H, P = inp["X"].shape
        self.bytes += 4 * (b * L * H * P + H)

    def run(self):
        t = self.t
        self.mb.mb_trap_ssd_gated(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["theta"],
                                  None, D=t["D"], z=t["z"], Y=self.Y, h_out=self.h, ws=self.ws)


class SISOBlock(SISO):
    """Mamba-3 SISO with both ends of its block fused into the scan: BCNorm +
    bias on B, C before the rotations, skip term and SiLU gate at the store;
    outside the step, measured beside it.  Bytes add z and the parameters;
    flops are the scan's."""
    name = "siso_block"

    def __init__(self, mb, wl, torch):
        super().__init__(mb, wl, torch)
        inp = wl.siso_block_full()
        self.inp = inp
        f = torch.float32
        self.t = {k: _dev(inp[k], f) for k in ("X", "logdecay", "B", "C", "beta", "gamma", "theta", "normB_w",
                                               "normC_w", "biasB", "biasC", "D", "z")}
        b, L, H, P = inp["X"].shape
        N = inp["B"].shape[3]
        self.bytes += 4 * (b * L * H * P + H + 2 * N + 2 * H * N)

    def run(self):
        t = self.t
        self.mb.mb_trap_ssd_block(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["theta"],
                                  None, normB_w=t["normB_w"], normC_w=t["normC_w"], biasB=t["biasB"],
                                  biasC=t["biasC"], D=t["D"], z=t["z"], Y=self.Y, h_out=self.h, ws=self.ws)


class M2Prologue(Workload):
    """The Mamba-2 block prologue in one pass (conv1d + SiLU over the x, B, C
    channels, softplus of dt, split into the SSD's inputs) at the Mamba-2 block
    shape; outside the step, measured beside it.  HBM-bound: xBC and dt read
    once, X, B, C, logdecay written once."""
    name = "m2_prologue"
    kernel = "k_ssd_prologue"
    source = "selective_state_space_amd/csrc/ssd_prologue.hip"
    bound = "hbm"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, G, N, K = 4, 4096, 24, 64, 1, 128, 4
        self.dims = (H, P, G, N)
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, G=G, K=K)
        inp = wl.m2_prologue_block()
        self.inp = inp
        f = torch.float32
        self.t = {k: (_dev(v, f) if v is not None else None) for k, v in inp.items()}
        self.out = (torch.empty((b, L, H, P), dtype=f, device="cuda"), torch.empty((b, L, G, N), dtype=f, device="cuda"),
                    torch.empty((b, L, G, N), dtype=f, device="cuda"), torch.empty((b, L, H), dtype=f, device="cuda"))
        cin = H * P + 2 * G * N
        self.tokens = b * L
        self.bytes = 4 * (2 * b * L * cin + 2 * b * L * H + cin * (K + 1) + 2 * H)
        self.flops = None
        self.exps = None

    def run(self):
        t = self.t
        H, P, G, N = self.dims
        X, B, C, ld = self.out
        self.mb.mb_ssd_prologue(t["xBC"], t["conv_w"], t["dt"], t["A"], H, P, G, N, conv_b=t["conv_b"],
                                dt_bias=t["dt_bias"], X=X, B=B, C=C, logdecay=ld)


class MIMO(Workload):
    name = "mimo"
    kernel = "k_walk (state-only pass) + k_walk (full pass)"
    source = "selective_state_space_amd/csrc/ssd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, N, R = 2, 8192, 16, 64, 128, 4
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, R=R)
        inp = wl.mimo_block()
        self.inp = inp
        f = torch.float32
        self.t = {k: _dev(inp[k], f) for k in ("X", "logdecay", "B", "C", "beta", "gamma", "theta")}
        self.Y = torch.empty_like(self.t["X"])
        self.h = torch.empty((b, H, N, P), dtype=f, device="cuda")
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_MIMO_SSD, b, L, H, P, 1, N, R, 0),
                              dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        self.bytes, self.flops = mimo_work(b, L, H, P, N, R)
        self.exps = None

    def run(self):
        t = self.t
        self.mb.mb_mimo_ssd(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["theta"], None,
                            Y=self.Y, h_out=self.h, ws=self.ws)


class SSDDecode(Workload):
    """Decode step of the SSD family (outside the timed step: measured next to it)."""
    kernel = "k_ssd_step"
    source = "selective_state_space_amd/csrc/ssd_step.hip"

    def __init__(self, mb, wl, torch, model):
        self.mb = mb
        self.name = model + "_decode"
        inp = wl.ssd_decode(model)
        self.inp = inp
        f = torch.float32
        self.t = {k: (_dev(v, f) if v is not None else None) for k, v in inp.items()}
        X, B = inp["X"], inp["B"]
        b, H, P = X.shape[:3]
        R = X.shape[3] if X.ndim == 4 else 1
        G, N = B.shape[1], B.shape[2]
        self.shape = dict(batch=b, H=H, P=P, N=N, G=G, R=R, trapezoid=model != "m2", rotation=model != "m2")
        self.tokens = b
        self.bytes = ssd_step_work(b, H, P, N, G, R, model != "m2", model != "m2")
        self.flops = self.exps = None
        self.Y = torch.empty_like(self.t["X"])

    def run(self):
        t = self.t
        self.mb.mb_ssd_step(t["X"], t["logdecay"], t["B"], t["C"], t["h"], beta=t.get("beta"),
                            gamma=t.get("gamma"), theta=t.get("theta"), X_prev=t.get("X_prev"),
                            B_prev=t.get("B_prev"), Y=self.Y)


ALL = ["m1_scan", "m1_step", "ssd_f32", "ssd_bf16", "siso", "mimo"]
# measured beside the step, not part of it: the decode steps of the SSD family, the
# Mamba-1 scan with the block prologue and epilogue fused, the Mamba-2 block prologue, Mamba-3 SISO with its output
# epilogue and with both ends of its block fused, and the backwards of the
# Mamba-2 SSD, the Mamba-1 scan, Mamba-3 SISO and MIMO
NEXT = ["m2_decode", "siso_decode", "mimo_decode", "m1_fused", "m2_prologue", "siso_gated", "siso_block", "ssd_bwd", "m1_bwd", "siso_bwd", "mimo_bwd"]


def make(name, mb, wl, torch):
    if name == "m1_scan":
        return M1Scan(mb, wl, torch)
    if name == "m1_step":
        return M1Step(mb, wl, torch)
    if name == "m1_fused":
        return M1Fused(mb, wl, torch)
    if name == "m2_prologue":
        return M2Prologue(mb, wl, torch)
    if name == "siso_block":
        return SISOBlock(mb, wl, torch)
    if name == "siso_gated":
        return SISOGated(mb, wl, torch)
    if name == "ssd_bwd":
        return SSDBwd(mb, wl, torch)
    if name == "m1_bwd":
        return M1Bwd(mb, wl, torch)
    if name == "siso_bwd":
        return SISOBwd(mb, wl, torch)
    if name == "mimo_bwd":
        return MIMOBwd(mb, wl, torch)
    if name == "ssd_f32":
        return SSD(mb, wl, torch, "f32")
    if name == "ssd_bf16":
        return SSD(mb, wl, torch, "bf16")
    if name == "siso":
        return SISO(mb, wl, torch)
    if name == "mimo":
        return MIMO(mb, wl, torch)
    if name.endswith("_decode"):
        return SSDDecode(mb, wl, torch, name[:-len("_decode")])
    raise ValueError(name)


def roofline_of(w, ms, bound=None):
    """Achieved fraction of the roofline that bounds workload w at ms per call."""
    s = ms * 1e-3
    bound = bound or w.bound
    if bound == "alu":
        ach = w.exps * getattr(w, "slots", M1_SLOTS_PER_ELEM) / s / 1e9
        peak = VALU_F32_LANE_OPS / 1e9
        return {"bound": "alu", "achieved": ach, "peak": peak, "unit": "Gop/s", "frac": ach / peak}
    if bound == "mfma":
        peak = BF16_PEAK_TFLOPS if getattr(w, "dtype", "f32") == "bf16" else FP32_PEAK_TFLOPS
        ach = w.flops / s / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak}
    ach = w.bytes / s / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS}


def source_hash(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(w):
    """HBM bytes per call measured with rocprofv3 counters (profiles/traffic.json),
    or None when no measurement exists for the current kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(p)).get(w.name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_hash(w.source):
        return None
    return rec.get("bytes_per_call")


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of each workload
# ----------------------------------------------------------------------------
def cpu_baseline(ws):
    """Time the fp64 oracle on the host cores on the same inputs (bf16 inputs are
    timed with their fp32 values: the oracle's cost does not depend on them)."""
    import oracle
    oracle.build()
    threads = oracle.get_threads()
    total_tok, total_s, parts = 0, 0.0, []
    for w in ws:
        i = w.inp
        t0 = time.perf_counter()
        if w.name == "m1_scan":
            oracle.m1_scan(**i)
        elif w.name == "m1_step":
            oracle.m1_step(i["x"], i["dt"], i["A"], i["B"], i["C"], i["D"], i["h"])
        elif w.name.startswith("ssd"):
            oracle.ssd(**i)
        elif w.name == "siso":
            oracle.trap(**i)
        elif w.name == "mimo":
            oracle.mimo(**i)
        dt = time.perf_counter() - t0
        total_tok += w.tokens
        total_s += dt
        parts.append("%s full (%d tokens, %.2f s)" % (w.name, w.tokens, dt))
    return {"value": total_tok / total_s if total_s else None, "unit": "scanned tokens/s",
            "cores": threads, "kind": "oracle", "sample": "; ".join(parts)}


_FLUSH = []


def cold_ms(torch, w, reps=5):
    """Median time of one call of workload w after overwriting a 512 MiB buffer,
    which evicts the 256 MB last-level cache: every input comes from HBM."""
    if not _FLUSH:
        _FLUSH.append(torch.empty(128 << 20, dtype=torch.float32, device="cuda"))
    buf = _FLUSH[0]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for r in range(reps):
        buf.fill_(float(r))
        e0.record()
        w.run()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return float(np.median(ms))


def time_next(args, mb, wl, torch):
    """Decode steps of the SSD family, the fused Mamba-1 block scan and the
    backwards, timed with
    HIP events on the stream they run on, outside the step (they are not part of
    its token count)."""
    res = []
    for n in NEXT:
        print("# preparing %s" % n, file=sys.stderr, flush=True)
        w = make(n, mb, wl, torch)
        for _ in range(args.warmup):
            w.run()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record()
            w.run()
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
        r = roofline_of(w, ms)
        roof = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        roof["traffic"] = traffic_for(w)
        res.append({"workload": w.name, "kernel": w.kernel, "shape": w.shape, "ms": round(ms, 5),
                    "tokens_per_s": w.tokens / (ms * 1e-3), "roofline": roof})
        del w
    return res


def copy_calibration(torch, reps=5):
    """A plain device-to-device copy of 256 MiB, repeated: the reference that the
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    n = 64 << 20
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_call": n * 4, "copy_bytes_written_per_call": n * 4,
                      "calls": reps}))
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the per-workload timings after a last-level-cache flush")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the decode steps of the SSD family measured beside the step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU; this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch
    import selective_state_space_amd as mb
    from selective_state_space_amd import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(torch)
    mb.load_library()
    names = [n for n in (args.only.split(",") if args.only else ALL) if n]
    ws = []
    for n in names:
        print("# preparing %s" % n, file=sys.stderr, flush=True)
        ws.append(make(n, mb, wl, torch))
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for w in ws:
            w.run()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ws]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for i, w in enumerate(ws):
            ev[k][i][0].record()
            w.run()
            ev[k][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = []
    for i, w in enumerate(ws):
        ms = [ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)]
        per.append(float(np.mean(ms)))
    ms_per_step = wall * 1e3 / args.steps
    tokens = sum(w.tokens for w in ws)
    kernels = []
    for w, ms in zip(ws, per):
        r = roofline_of(w, ms)
        d = {"workload": w.name, "ms": round(ms, 5), "tokens_per_s": w.tokens / (ms * 1e-3),
             "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}}
        hbm = roofline_of(w, ms, "hbm")
        d["hbm_gbs"] = round(hbm["achieved"], 1)
        d["hbm_frac"] = round(hbm["frac"], 4)
        if w.exps:
            d["exp_per_s"] = w.exps / (ms * 1e-3)
        kernels.append(d)
    dom = int(np.argmax(per))
    w = ws[dom]
    r = roofline_of(w, per[dom])
    roof = {"bound": r["bound"], "achieved": round(r["achieved"], 3), "peak": r["peak"],
            "unit": r["unit"], "frac": round(r["frac"], 4), "traffic": traffic_for(w),
            "kernel": w.kernel, "workload": w.name}

    if not args.no_cold:
        print("# cold timings (last-level cache flushed before each call)", file=sys.stderr, flush=True)
        for w, d in zip(ws, kernels):
            cms = cold_ms(torch, w)
            d["cold_ms"] = round(cms, 5)
            d["cold_hbm_frac"] = round(w.bytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    out = {
        "metric": "scanned tokens/sec, SSD fwd L=4096 + M1 scan; % MFMA / % HBM roofline",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "scanned tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if all(getattr(w, "dtype", "f32") == "f32" for w in ws) else "f32+bf16",
        "data": "synthetic (seeded numpy inputs, recipes in selective_state_space_amd/workloads.py)",
        "config": {"workload": "+".join(names), "tokens_per_step": tokens,
                   "shapes": {w.name: w.shape for w in ws}},
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_next and not args.only:
        out["next"] = time_next(args, mb, wl, torch)
    if not args.no_cpu:
        print("# timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(ws)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
