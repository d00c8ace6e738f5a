"""GPU parity of the SSD-family decode step (mb_ssd_step: Mamba-2, Mamba-3
SISO and MIMO, state in the physical frame) against the fp64 oracle step,
through the C ABI; and decode after a chunked prefill against the oracle's
forward loop."""
import zlib

import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import assert_close, prepare, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _step_inputs(rng, b, H, P, G, N, R, kind, h_sd=0.3):
    return wl.ssd_step_inputs(rng, b, H, P, G, N, R, kind, h_sd=h_sd)


def _run(dev):
    args = {k: dev.get(k) for k in ("beta", "gamma", "theta", "X_prev", "B_prev")}
    return mb.mb_ssd_step(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h"], **args,
                          h_out=torch.empty_like(dev["h"]))


CASES = [  # batch, H, P, G, N, R, kind
    (3, 4, 64, 2, 128, 1, "m2"), (2, 3, 16, 3, 8, 1, "m2"), (4, 6, 64, 1, 128, 1, "rot"),
    (2, 2, 32, 1, 16, 1, "trap"), (2, 4, 64, 4, 128, 4, "rot"), (1, 3, 12, 3, 6, 2, "rot"),
    (2, 2, 4, 2, 2, 1, "rot"), (1, 2, 1024, 2, 10, 1, "rot"), (1, 2, 20, 2, 34, 16, "trap"),
    (2, 2, 64, 2, 64, 8, "rot")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_step_parity(oracle_mod, case, dtype):
    b, H, P, G, N, R, kind = case
    inp = _step_inputs(np.random.default_rng(zlib.crc32(repr(case).encode())), b, H, P, G, N, R, kind)
    dev, ref = prepare(inp, dtype)
    Y, h = _run(dev)
    Yr, hr = oracle_mod.ssd_step(**ref)
    assert Y.dtype == dev["X"].dtype
    assert_close(Y, Yr, dtype, "Y")
    assert_close(h, hr, dtype, "h")


def test_ssd_step_in_place_and_no_state(oracle_mod):
    inp = _step_inputs(np.random.default_rng(11), 2, 3, 32, 3, 16, 1, "rot")
    dev, ref = prepare(inp, "f32")
    Yr, hr = oracle_mod.ssd_step(**ref)
    h = dev["h"].clone()
    Y, h2 = mb.mb_ssd_step(dev["X"], dev["logdecay"], dev["B"], dev["C"], h, beta=dev["beta"],
                           gamma=dev["gamma"], theta=dev["theta"], X_prev=dev["X_prev"], B_prev=dev["B_prev"])
    assert h2.data_ptr() == h.data_ptr()
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
    # a zero state and no previous token (the first token of a sequence)
    Y0, h0 = mb.mb_ssd_step(dev["X"], dev["logdecay"], dev["B"], dev["C"], torch.zeros_like(h),
                            beta=dev["beta"], gamma=dev["gamma"], theta=dev["theta"])
    Yz, hz = oracle_mod.ssd_step(ref["X"], ref["logdecay"], ref["B"], ref["C"], None, ref["beta"], ref["gamma"],
                                 ref["theta"])
    assert_close(Y0, Yz, "f32", "Y")
    assert_close(h0, hz, "f32", "h")


@pytest.mark.parametrize("model", ["m2", "siso", "mimo"])
def test_decode_after_chunked_prefill(oracle_mod, model):
    """Prefill L0 tokens with the chunked entry point, then decode the rest with
    the step, passing the previous token's B and X; compare with the oracle's
    forward loop over the whole sequence."""
    rng = np.random.default_rng({"m2": 21, "siso": 22, "mimo": 23}[model])
    L, L0 = 150, 130
    if model == "m2":
        inp = wl.ssd_inputs(rng, 2, L, 4, 32, 64, G=2, h0_sd=0.2)
    elif model == "siso":
        inp = wl.trap_inputs(rng, 2, L, 3, 32, 64, G=1, h0_sd=0.2)
    else:
        inp = wl.mimo_inputs(rng, 1, L, 2, 32, 64, 4, h0_sd=0.2)
    dev, ref = prepare(inp, "f32")
    Yr, hr = getattr(oracle_mod, {"m2": "ssd", "siso": "trap", "mimo": "mimo"}[model])(**ref)
    pre = {k: (v[:, :L0].contiguous() if k != "h0" and v is not None else v) for k, v in dev.items()}
    if model == "m2":
        _, h = mb.mb_ssd_chunked(pre["X"], pre["logdecay"], pre["B"], pre["C"], pre["h0"])
    elif model == "siso":
        _, h = mb.mb_trap_ssd(pre["X"], pre["logdecay"], pre["B"], pre["C"], pre["beta"], pre["gamma"],
                              pre["theta"], pre["h0"])
    else:
        _, h = mb.mb_mimo_ssd(pre["X"], pre["logdecay"], pre["B"], pre["C"], pre["beta"], pre["gamma"],
                              pre["theta"], pre["h0"])
    ys = []
    for t in range(L0, L):
        kw = {}
        if model != "m2":
            kw = dict(beta=dev["beta"][:, t].contiguous(), gamma=dev["gamma"][:, t].contiguous(),
                      theta=dev["theta"][:, t].contiguous(), X_prev=dev["X"][:, t - 1].contiguous(),
                      B_prev=dev["B"][:, t - 1].contiguous())
        y, h = mb.mb_ssd_step(dev["X"][:, t].contiguous(), dev["logdecay"][:, t].contiguous(),
                              dev["B"][:, t].contiguous(), dev["C"][:, t].contiguous(), h, **kw)
        ys.append(y)
    assert_close(torch.stack(ys, 1), Yr[:, L0:], "f32", "Y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.parametrize("model", ["m2", "siso", "mimo"])
def test_ssd_step_decode_workloads(oracle_mod, model):
    """The measured decode workloads: 256 sequences on the block shapes."""
    dev, ref = prepare(wl.ssd_decode(model), "f32")
    Y, h = _run(dev)
    torch.cuda.synchronize()
    Yr, hr = oracle_mod.ssd_step(**ref)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")
