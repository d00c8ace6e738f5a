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
sequences), the step timed back to back.  Per-workload times come from HIP
events recorded on the stream the kernels run on: the headline `ms` of each
workload is the mean over calls that each follow a flush of the last-level
cache (every input read from HBM), with the back-to-back mean (`warm_ms`)
beside it.  The `roofline` object is for the workload whose kernels take the
largest share of the step, `rooflines` for the two workloads the metric names,
and `kernels` lists every workload.  `cpu_baseline` times the fp64 oracle on
the same workloads on the host cores.  `next` times, beside the step and
outside its token count, the decode steps of the SSD family, the fused block
variants and the backwards.

The run has two phases, so that a rocprofv3 kernel trace of it splits cleanly:
every warm call (warm-up and back-to-back timing, the step's workloads and
then those beside it) comes before the first cache flush, and every flushed
call after it.  `--summarize DIR...` prints markdown tables of rocprofv3 csv
output directories (kernel trace split by phase; counter means per dispatch).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only a,b] [--no-cpu] [--no-next]
                    [--next a,b] [--no-cold] [--copy-calibration] [--summarize DIR...]
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
# fp32 vector issue slots per second without packed fp32 (disabled in this
# library): 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12, one FMA per lane
# per clock.  The published 157.3 TFLOP/s fp32 vector peak counts packed FMA
# (two per lane per clock, two flops each).  Measured on MI355X with a
# throughput probe (8 independent chains per lane, shader clock read at
# 2.32-2.39 GHz): v_fma_f32 takes 4.3-4.6 cycles per wave instruction per SIMD
# at 2 to 8 waves per SIMD (35.9 T lane-ops/s at 8 waves); one wave alone
# issues one only every ~8.6 cycles.
VALU_LANE_SLOTS = 256 * 4 * 16 * 2.4e9
PACKED_VALU_LANE_SLOTS = 2 * VALU_LANE_SLOTS   # the published peak, in FMA lane-slots
# v_exp_f32 throughput from the same probe: 9.2 cycles per wave instruction at
# 8 waves per SIMD, about two FMA slots; one exp beside four FMA chains takes
# the sum of their times (the two do not overlap), so an exp counts 2 slots.
EXP_SLOTS = 2
# Minimal VALU issue slots per Mamba-1 (t, c, n) element: dt*A, (dt*x)*B,
# a*h + u, y += C*h (one slot each) and one exp.
M1_SLOTS_PER_ELEM = 4 + EXP_SLOTS


# ----------------------------------------------------------------------------
# algorithmic work per workload (bytes: each input read once, each output
# written once; flops at the canonical chunk length 64, causal half only)
# ----------------------------------------------------------------------------
def m1_scan_work(b, L, D, N, es=4):
    nbytes = es * (3 * b * L * D + 2 * b * L * N) + 4 * (D * N + D + b * D * N)
    return nbytes, b * L * D * N      # (bytes, exp count)


# Minimal VALU issue slots per (t, c, n) element of the Mamba-1 backward: the
# recomputed forward (4 + an exp) and the adjoint step: G += C dy, dB and dC
# products, U += G B, the exp's argument and the exp, G a h_prev (2), V += A w,
# dA += dt w, G *= a (10 + an exp).
M1_BWD_SLOTS_PER_ELEM = 14 + 2 * EXP_SLOTS


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
    kernel = "k_m1_scan_w"
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


class M1Long(M1Scan):
    """One long sequence of the Mamba-1 block model's width (batch 1, L 16384,
    D 1536, N 16: as many (t, c, n) elements as the block workload, but 24
    channel groups for 256 compute units): the scan cut into sequence blocks
    with the carry pass (the default), or in one block (`m1_long_one_block`);
    outside the step, measured beside it."""
    name = "m1_long"
    kernel = "k_m1_scan_w (carry pass) + k_m1_scan_w (sequence blocks)"

    def __init__(self, mb, wl, torch, one_block=False):
        self.mb = mb
        b, L, D, N = 1, 16384, 1536, 16
        self.shape = dict(batch=b, L=L, D=D, N=N, sequence_blocks=not one_block)
        inp = wl.m1_block(batch=b, L=L)
        self.inp = inp
        f = torch.float32
        self.x, self.dt, self.B, self.C = (_dev(inp[k], f) for k in ("x", "dt", "B", "C"))
        self.A, self.D = _dev(inp["A"], f), _dev(inp["D"], f)
        self.y = torch.empty_like(self.x)
        self.h = torch.empty((b, D, N), dtype=f, device="cuda")
        self.one_block = one_block
        if one_block:
            self.name = "m1_long_one_block"
            self.kernel = "k_m1_scan_w"
            self.ws = None
        else:
            self.ws = torch.empty(max(256, mb.mb_workspace_size(mb.MB_OP_SELECTIVE_SCAN, b, L, D, 1, 1, N)),
                                  dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        self.bytes, self.exps = m1_scan_work(b, L, D, N)
        self.flops = None

    def run(self):
        self.mb.mb_selective_scan(self.x, self.dt, self.A, self.B, self.C, self.D, None, y=self.y, h_out=self.h,
                                  ws=self.ws, seq_blocks=not self.one_block)


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
    kernel = "k_scores + k_seg_state (state-only pass) + k_walk_m2s (full pass)"
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
            self.kernel = "k_scores + k_walk_bf (state-only pass) + k_walk_bfs (full pass)"

    def run(self):
        self.mb.mb_ssd_chunked(self.X, self.ld, self.B, self.C, None, Y=self.Y, h_out=self.h, ws=self.ws)


class SSDGated(SSD):
    """The Mamba-2 SSD with the block's output side (skip term D[h] X and SiLU(z)
    gate) fused into the store; outside the step, measured beside it.  Bytes add
    z and D; flops are the scan's."""

    def __init__(self, mb, wl, torch, dtype):
        super().__init__(mb, wl, torch, dtype)
        self.name = "ssd_gated_" + dtype
        rng = np.random.default_rng(119)
        act = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.D = _dev(rng.standard_normal(self.shape["H"]), torch.float32)
        self.z = _dev(rng.standard_normal(tuple(self.X.shape)), act)
        b, L, H, P = self.X.shape
        self.bytes += (2 if dtype == "bf16" else 4) * b * L * H * P + 4 * H
        self.kernel = self.kernel.replace("(full pass)", "(full pass, output side)")

    def run(self):
        self.mb.mb_ssd_chunked_gated(self.X, self.ld, self.B, self.C, None, D=self.D, z=self.z, Y=self.Y,
                                     h_out=self.h, ws=self.ws)


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
    kernel = "k_seg_trap (state-only pass) + k_walk (full pass)"
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


class MIMOBlock(Workload):
    """Mamba-3 MIMO with both ends of its block fused into the scan: BCNorm +
    bias on every rank row of B, C before the rotations, skip term and SiLU gate
    per rank at the store; outside the step, measured beside it.  Bytes add z and
    the parameters; flops are the scan's."""
    name = "mimo_block"
    kernel = "k_walk (state-only pass, prologue) + k_walk (full pass, both ends)"
    source = "selective_state_space_amd/csrc/ssd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch):
        self.mb = mb
        b, L, H, P, N, R = 2, 8192, 16, 64, 128, 4
        self.shape = dict(batch=b, L=L, H=H, P=P, N=N, R=R)
        inp = wl.mimo_block_full()
        self.inp = inp
        f = torch.float32
        self.t = {k: _dev(v, f) for k, v in inp.items() if v is not None}
        self.Y = torch.empty_like(self.t["X"])
        self.h = torch.empty((b, H, N, P), dtype=f, device="cuda")
        self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_MIMO_SSD, b, L, H, P, 1, N, R, 0),
                              dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        nbytes, self.flops = mimo_work(b, L, H, P, N, R)
        self.bytes = nbytes + 4 * (b * L * H * P * R + H + 2 * N + 2 * H * N)
        self.exps = None

    def run(self):
        t = self.t
        self.mb.mb_mimo_ssd_block(t["X"], t["logdecay"], t["B"], t["C"], t["beta"], t["gamma"], t["theta"], None,
                                  normB_w=t["normB_w"], normC_w=t["normC_w"], biasB=t["biasB"], biasC=t["biasC"],
                                  D=t["D"], z=t["z"], Y=self.Y, h_out=self.h, ws=self.ws)


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


class M2Block(Workload):
    """The Mamba-2 layer around its scan in one call (mb_ssd_block: conv1d + SiLU
    over xBC and softplus of dt fused into the chunked SSD, skip term and SiLU
    gate at the store) at the Mamba-2 block shape; with `unfused`, the same work
    as two calls, the prologue pass (mb_ssd_prologue) and then the SSD with its
    output side (mb_ssd_chunked_gated); outside the step, measured beside it.
    Bytes: xBC, dt, z read and Y written once plus the parameters; flops are the
    SSD's."""
    source = "selective_state_space_amd/csrc/ssd.hip"
    bound = "mfma"

    def __init__(self, mb, wl, torch, dtype, unfused=False):
        self.mb = mb
        b, L, H, P, G, N, K = 4, 4096, 24, 64, 1, 128, 4
        self.dims = (H, P, G, N)
        self.dtype = dtype
        self.unfused = unfused
        self.name = ("m2_unfused_" if unfused else "m2_block_") + dtype
        if dtype == "bf16":
            # bf16 runs on the bf16 matrix instruction, where the SSD is bound by HBM
            self.bound = "hbm"
            self.kernel = "k_ssd_prologue + k_scores + k_walk_bf (state-only) + k_walk_bfs (output side)"
        elif unfused:
            self.kernel = "k_ssd_prologue + k_scores + k_seg_state (state-only) + k_walk_m2s (output side)"
        else:
            self.kernel = ("k_scores (B, C prologue) + k_walk (state-only, x prologue) + "
                           "k_walk_m2s (x prologue, output side)")
        self.shape = dict(batch=b, L=L, H=H, P=P, G=G, N=N, K=K)
        inp = wl.m2_block_full()
        self.inp = inp
        act = torch.bfloat16 if dtype == "bf16" else torch.float32
        f = torch.float32
        self.t = {k: (_dev(v, act if k in ("xBC", "z") else f) if v is not None else None) for k, v in inp.items()}
        self.Y = torch.empty((b, L, H, P), dtype=act, device="cuda")
        self.h = torch.empty((b, H, N, P), dtype=f, device="cuda")
        es = 2 if dtype == "bf16" else 4
        cin = H * P + 2 * G * N
        if unfused:
            self.X = torch.empty((b, L, H, P), dtype=act, device="cuda")
            self.B = torch.empty((b, L, G, N), dtype=act, device="cuda")
            self.C = torch.empty((b, L, G, N), dtype=act, device="cuda")
            self.ld = torch.empty((b, L, H), dtype=f, device="cuda")
            self.ws = torch.empty(mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, b, L, H, P, G, N, 1, 0),
                                  dtype=torch.uint8, device="cuda")
        else:
            op = mb.MB_OP_SSD_BLOCK_BF16 if dtype == "bf16" else mb.MB_OP_SSD_BLOCK
            self.ws = torch.empty(mb.mb_workspace_size(op, b, L, H, P, G, N, 1, 0), dtype=torch.uint8, device="cuda")
        self.tokens = b * L
        self.bytes = es * (b * L * cin + 2 * b * L * H * P) + 4 * (b * L * H + cin * (K + 1) + 3 * H + b * H * N * P)
        _, self.flops = ssd_work(b, L, H, P, N, G, es)
        self.exps = None

    def run(self):
        t = self.t
        H, P, G, N = self.dims
        if self.unfused:
            self.mb.mb_ssd_prologue(t["xBC"], t["conv_w"], t["dt"], t["A"], H, P, G, N, conv_b=t["conv_b"],
                                    dt_bias=t["dt_bias"], X=self.X, B=self.B, C=self.C, logdecay=self.ld)
            self.mb.mb_ssd_chunked_gated(self.X, self.ld, self.B, self.C, None, D=t["D"], z=t["z"], Y=self.Y,
                                         h_out=self.h, ws=self.ws)
        else:
            self.mb.mb_ssd_block(t["xBC"], t["conv_w"], t["dt"], t["A"], H, P, G, N, conv_b=t["conv_b"],
                                 dt_bias=t["dt_bias"], D=t["D"], z=t["z"], Y=self.Y, h_out=self.h, ws=self.ws)


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
NEXT = ["m2_decode", "siso_decode", "mimo_decode", "m1_long", "m1_long_one_block", "m1_fused", "m2_prologue", "m2_block_f32", "m2_unfused_f32", "m2_block_bf16", "m2_unfused_bf16", "ssd_gated_f32", "ssd_gated_bf16", "siso_gated", "siso_block", "mimo_block", "ssd_bwd", "m1_bwd", "siso_bwd", "mimo_bwd"]


def make(name, mb, wl, torch):
    if name == "m1_scan":
        return M1Scan(mb, wl, torch)
    if name == "m1_step":
        return M1Step(mb, wl, torch)
    if name == "m1_fused":
        return M1Fused(mb, wl, torch)
    if name == "m1_long":
        return M1Long(mb, wl, torch)
    if name == "m1_long_one_block":
        return M1Long(mb, wl, torch, one_block=True)
    if name == "m2_prologue":
        return M2Prologue(mb, wl, torch)
    if name == "siso_block":
        return SISOBlock(mb, wl, torch)
    if name.startswith("m2_block_"):
        return M2Block(mb, wl, torch, name[len("m2_block_"):])
    if name.startswith("m2_unfused_"):
        return M2Block(mb, wl, torch, name[len("m2_unfused_"):], unfused=True)
    if name.startswith("ssd_gated_"):
        return SSDGated(mb, wl, torch, name[len("ssd_gated_"):])
    if name == "mimo_block":
        return MIMOBlock(mb, wl, torch)
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
        peak = VALU_LANE_SLOTS / 1e9
        return {"bound": "alu", "achieved": ach, "peak": peak, "unit": "G lane-slots/s", "frac": ach / peak,
                "peak_note": "fp32 FMA without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz",
                "frac_of_packed_peak": ach / (PACKED_VALU_LANE_SLOTS / 1e9)}
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


TRAFFIC_REPS = 3


def traffic_run(mb, wl, torch):
    """The calls the byte counters are read on: every workload in turn, called
    TRAFFIC_REPS times between two one-element fills (marker kernels; the set-up
    and first call of each workload fall outside them).  Prints the order, with
    each workload's kernel source and algorithmic bytes, as one JSON line."""
    order = []
    for n in ALL + NEXT:
        print("# traffic run: %s" % n, file=sys.stderr, flush=True)
        w = make(n, mb, wl, torch)
        w.run()   # first call outside the measured ones (library set-up, first-touch)
        torch.cuda.synchronize()
        torch.full((1,), 1.0, device="cuda")
        for _ in range(TRAFFIC_REPS):
            w.run()
        torch.full((1,), 2.0, device="cuda")
        torch.cuda.synchronize()
        order.append({"name": n, "source": w.source, "bytes": getattr(w, "bytes", None)})
        del w
        torch.cuda.empty_cache()
    print(json.dumps({"traffic_order": order, "reps": TRAFFIC_REPS}))
    return 0


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def traffic(run_log, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """profiles/traffic.json and a markdown table from four rocprofv3 counter
    passes: FETCH_SIZE and WRITE_SIZE over `bench.py --traffic-run` (run_log: the
    output of one such run, with its JSON line), and the same two over `bench.py
    --copy-calibration` (a plain 256 MiB copy, whose bytes are known: the counters
    are scaled so that they read them).  The traffic run's dispatches are split
    into workloads at the marker fills (the segments after the first, third, ...
    fill are the measured calls); a workload's bytes per call are the sum over
    its dispatches divided by the number of calls."""
    spec = None
    for line in open(run_log):
        if line.startswith("{") and "traffic_order" in line:
            spec = json.loads(line)["traffic_order"]
    if spec is None:
        raise SystemExit("no traffic_order line in %s" % run_log)

    def kib_by_kernel(rows):
        return [(_short(r["Kernel_Name"]), float(r["Counter_Value"])) for r in rows]

    def copy_kib(d):
        v = [x for n, x in kib_by_kernel(_counter_rows(d)) if "copyBuffer" in n or "copy" in n.lower()]
        return float(np.median(v))

    copy_bytes = 256 << 20
    ff = copy_bytes / 1024.0 / copy_kib(cfetch_dir)
    wf = copy_bytes / 1024.0 / copy_kib(cwrite_dir)

    def segments(d):
        segs, cur = [], None
        for n, v in kib_by_kernel(_counter_rows(d)):
            if "FillFunctor" in n:
                cur = []
                segs.append(cur)
            elif cur is not None:
                cur.append((n, v))
        return segs

    order = [d["name"] for d in spec]
    fs, ws_ = segments(fetch_dir)[0::2], segments(write_dir)[0::2]
    if len(fs) != len(order) or len(ws_) != len(order):
        raise SystemExit("counter runs hold %d / %d measured segments, expected %d" % (len(fs), len(ws_), len(order)))
    out = {"_calibration": {"fetch_factor": ff, "write_factor": wf, "copy_bytes": copy_bytes,
                            "copy_fetch_kib": copy_kib(cfetch_dir), "copy_write_kib": copy_kib(cwrite_dir)}}
    lines = ["| workload | kernels | read MB | written MB | total MB | algorithmic MB | ratio |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for d, f, w in zip(spec, fs, ws_):
        n = d["name"]
        rd = sum(v for _, v in f) * 1024 * ff / TRAFFIC_REPS
        wr = sum(v for _, v in w) * 1024 * wf / TRAFFIC_REPS
        kern = []
        for k, _ in f:
            if k not in kern:
                kern.append(k)
        alg = d["bytes"]
        out[n] = {"bytes_per_call": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr),
                  "source": d["source"], "source_sha": source_hash(d["source"]), "kernels": kern}
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %s | %s |" % (
            n, " + ".join("`%s`" % k for k in kern), rd / 1e6, wr / 1e6, (rd + wr) / 1e6,
            "%.1f" % (alg / 1e6) if alg else "", "%.2f" % ((rd + wr) / alg) if alg else ""))
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print("Calibration: the plain 256 MiB device copy reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB per "
          "dispatch, so FETCH_SIZE is scaled by %.4f and WRITE_SIZE by %.4f (bytes = KiB x 1024 x factor).\n"
          % (copy_kib(cfetch_dir), copy_kib(cwrite_dir), ff, wf))
    print("\n".join(lines))
    return 0


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores
# ----------------------------------------------------------------------------
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(ws, wl):
    """Time the fp64 oracle on the host cores on the same inputs (bf16 inputs are
    timed with their fp32 values: the oracle's cost does not depend on them),
    in passes over the step's workloads until about 10 s of host time (a bounded
    sample), then the two small workloads (Mamba-1 tiny, Mamba-1 decode) on one
    thread."""
    import oracle
    oracle.build()
    threads = oracle.get_threads()
    total_tok, total_s, passes = 0, 0.0, 0
    per = {w.name: 0.0 for w in ws}
    while True:
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
            per[w.name] += dt
        passes += 1
        if total_s >= 10.0 or passes >= 50:
            break
    sample = "%d passes over the full workloads of the step, %.1f s in all; per pass: %s" % (
        passes, total_s, ", ".join("%s %d tokens %.3f s" % (w.name, w.tokens, per[w.name] / passes) for w in ws))
    single = {}
    oracle.set_threads(1)
    try:
        tiny = wl.m1_tiny()
        dec = wl.m1_decode()
        for name, fn, tok in (("m1_tiny", lambda: oracle.m1_scan(**tiny), 64),
                              ("m1_step", lambda: oracle.m1_step(dec["x"], dec["dt"], dec["A"], dec["B"],
                                                                 dec["C"], dec["D"], dec["h"]), 256)):
            reps, t0 = 0, time.perf_counter()
            while True:
                fn()
                reps += 1
                el = time.perf_counter() - t0
                if el > 0.5 or reps >= 1000:
                    break
            single[name] = {"tokens_per_s": tok * reps / el, "ms_per_call": el * 1e3 / reps}
    finally:
        oracle.set_threads(threads)
    return {"value": total_tok / total_s if total_s else None, "unit": "scanned tokens/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": sample, "single_thread": single}


_FLUSH = {}


def flush(torch):
    """Read a 512 MiB buffer (a sum over it): evicts the 256 MB last-level cache,
    so the next call reads every input from HBM.  A read rather than a write:
    overwriting the buffer leaves dirty lines whose write-back then competes
    with the measured call (the Mamba-1 decode step measured 0.5-0.8 us slower
    after a fill than after a read)."""
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    _FLUSH["sum"] = _FLUSH["buf"].sum()


def time_flushed(torch, w, reps):
    """Event times (ms) of `reps` calls of workload w, each after a cache flush."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        flush(torch)
        e0.record()
        w.run()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def time_warm(torch, w, warmup, reps):
    """Event times (ms) of `reps` back-to-back calls after `warmup` calls."""
    for _ in range(warmup):
        w.run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        w.run()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def _roof(w, ms):
    r = roofline_of(w, ms)
    roof = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
    roof["traffic"] = traffic_for(w)
    return roof


def entry(w, flushed, warm):
    """One workload's record: the headline time is the mean over calls after a
    cache flush; the warm (back-to-back) mean beside it."""
    ms = float(np.mean(flushed))
    d = {"workload": w.name, "kernel": w.kernel, "shape": w.shape, "ms": round(ms, 5),
         "ms_median": round(float(np.median(flushed)), 5), "ms_min": round(float(np.min(flushed)), 5),
         "warm_ms": round(float(np.mean(warm)), 5) if warm else None,
         "tokens_per_s": w.tokens / (ms * 1e-3), "roofline": _roof(w, ms)}
    hbm = roofline_of(w, ms, "hbm")
    d["hbm_gbs"] = round(hbm["achieved"], 1)
    d["hbm_frac"] = round(hbm["frac"], 4)
    if w.exps:
        d["exp_per_s"] = w.exps / (ms * 1e-3)
    return d


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


# ----------------------------------------------------------------------------
# rocprofv3 summaries (markdown) of this script's own runs
# ----------------------------------------------------------------------------
def _short(name):
    n = name.replace("mb::(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    k = n.find("(")
    return n[:k] if k > 0 else n


def summarize(paths):
    """Markdown tables from rocprofv3 csv output directories of bench.py runs.

    Kernel trace: every dispatch before the first cache flush (a reduction over
    the 512 MiB flush buffer) is in the warm phase (warm-up and back-to-back
    calls); every dispatch after it is in the flushed phase (each workload call
    follows a flush).  Dispatches are grouped by kernel and launch size
    (workgroups), which tells apart the workloads that share a kernel.  The
    flush kernels and torch's fills are left out.
    Counter collection: the mean per dispatch of each counter, with the MFMA
    busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 XCDs x
    1024 SIMDs), the VALU busy fraction of a wave's life (SQ_ACTIVE_INST_VALU /
    SQ_WAVE_CYCLES) and the LDS bank-conflict share (SQ_LDS_BANK_CONFLICT /
    SQ_LDS_IDX_ACTIVE)."""
    import csv
    import glob
    out = []
    for d in paths:
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            rows = list(csv.DictReader(open(f)))
            rows.sort(key=lambda r: int(r["Start_Timestamp"]))
            phase, stats = "warm", {}
            for r in rows:
                name = _short(r["Kernel_Name"])
                if "reduce_kernel" in name:
                    phase = "flushed"
                    continue
                if "FillFunctor" in name:
                    continue
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                wg = 1
                for ax in "XYZ":
                    wg *= max(1, int(r["Grid_Size_" + ax]) // max(1, int(r["Workgroup_Size_" + ax])))
                stats.setdefault((name, wg, phase), []).append(us)
            out.append("Kernel trace `%s`\n" % os.path.relpath(f, d))
            out.append("| kernel | workgroups | phase | calls | avg µs | median µs | min µs | max µs |")
            out.append("|---|---:|---|---:|---:|---:|---:|---:|")
            for (name, wg, ph), v in sorted(stats.items(), key=lambda kv: (kv[0][0], kv[0][1], kv[0][2] != "flushed")):
                out.append("| `%s` | %d | %s | %d | %.2f | %.2f | %.2f | %.2f |" % (
                    name, wg, ph, len(v), np.mean(v), np.median(v), np.min(v), np.max(v)))
            out.append("")
    # counters: every counter file of every directory in one table (one pass per
    # directory; a kernel's mean per dispatch in each)
    acc, files = {}, []
    for d in paths:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            files.append(os.path.basename(f))
            for r in csv.DictReader(open(f)):
                name = _short(r["Kernel_Name"])
                if "FillFunctor" in name or "copyBuffer" in name or "reduce_kernel" in name:
                    continue
                acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if acc:
        cnames = sorted({c for v in acc.values() for c in v})
        out.append("Counters from %s (mean per dispatch)\n" % ", ".join("`%s`" % f for f in files))
        extra = []
        if {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"} <= set(cnames):
            extra.append("MFMA busy")
        if {"SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"} <= set(cnames):
            extra.append("VALU busy")
        if {"SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"} <= set(cnames):
            extra.append("LDS conflict")
        out.append("| kernel | dispatches | " + " | ".join(cnames + extra) + " |")
        out.append("|---|---:|" + "---:|" * (len(cnames) + len(extra)))
        for name, cv in acc.items():
            m = {c: float(np.mean(v)) for c, v in cv.items()}
            cells = ["%.0f" % m[c] if c in m else "" for c in cnames]
            if "MFMA busy" in extra:
                cells.append("%.1f%%" % (100 * m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) /
                                         max(1.0, m.get("GRBM_GUI_ACTIVE", 0) / 8 * 1024)))
            if "VALU busy" in extra:
                cells.append("%.1f%%" % (100 * m.get("SQ_ACTIVE_INST_VALU", 0) / max(1.0, m.get("SQ_WAVE_CYCLES", 0))))
            if "LDS conflict" in extra:
                cells.append("%.1f%%" % (100 * m.get("SQ_LDS_BANK_CONFLICT", 0) / max(1.0, m.get("SQ_LDS_IDX_ACTIVE", 0))))
            n = len(next(iter(cv.values())))
            out.append("| `%s` | %d | %s |" % (name, n, " | ".join(cells)))
        out.append("")
    print("\n".join(out))
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
                    help="skip the workloads measured beside the step")
    ap.add_argument("--next", default="", help="comma-separated subset of the workloads beside the step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for rocprofv3 byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print markdown summaries of rocprofv3 csv output directories and exit")
    ap.add_argument("--traffic-run", action="store_true",
                    help="only run every workload behind a marker fill (the calls the byte counters read)")
    ap.add_argument("--traffic", nargs=5, metavar=("RUN_LOG", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/traffic.json from the byte-counter passes and print a table")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args.summarize)
    if args.traffic:
        return traffic(*args.traffic)
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
    if args.traffic_run:
        return traffic_run(mb, wl, torch)
    names = [n for n in (args.only.split(",") if args.only else ALL) if n]
    ws = []
    for n in names:
        print("# preparing %s" % n, file=sys.stderr, flush=True)
        ws.append(make(n, mb, wl, torch))
    torch.cuda.synchronize()

    # ---- warm phase: the step, back to back --------------------------------------
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
    warm = [[ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)] for i in range(len(ws))]
    ms_per_step = wall * 1e3 / args.steps
    tokens = sum(w.tokens for w in ws)

    if args.no_next:
        nxt_names = []
    elif args.next:
        nxt_names = [n for n in args.next.split(",") if n]
    else:
        nxt_names = [] if args.only else NEXT
    nxt_warm = []
    for n in nxt_names:
        print("# preparing %s" % n, file=sys.stderr, flush=True)
        w = make(n, mb, wl, torch)
        nxt_warm.append((w, time_warm(torch, w, args.warmup, args.steps)))
        if not args.no_cold:
            w.inp = None   # keep the device tensors only
        else:
            del w

    # ---- flushed phase: every call after a last-level-cache flush -----------------
    if not args.no_cold:
        print("# flushed timings (last-level cache flushed before each call)", file=sys.stderr, flush=True)
        flushed = [time_flushed(torch, w, args.steps) for w in ws]
        nxt = [entry(w, time_flushed(torch, w, args.steps), t) for w, t in nxt_warm]
    else:
        flushed = warm
        nxt = [entry(w, t, t) for w, t in nxt_warm]
    del nxt_warm

    kernels = [entry(w, f, t) for w, f, t in zip(ws, flushed, warm)]
    dom = int(np.argmax([np.mean(t) for t in warm]))
    roof = dict(kernels[dom]["roofline"])
    roof.update({"kernel": ws[dom].kernel, "workload": ws[dom].name,
                 "timing": "mean event time per call after a last-level-cache flush" if not args.no_cold
                 else "mean event time per call, back to back"})

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
        # the two workloads the metric names, beside the dominant one
        "rooflines": {d["workload"]: d["roofline"] for d in kernels if d["workload"] in ("ssd_f32", "m1_scan")},
        "kernels": kernels,
    }
    if nxt:
        out["next"] = nxt
    if not args.no_cpu:
        print("# timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(ws, wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
