"""GPU parity of the Mamba-2 block prologue (conv1d + SiLU over the x, B, C
channels, softplus of dt, split into the SSD's inputs) against the fp64 oracle,
through the C ABI; and the prologue followed by the chunked SSD against the
oracle's composition."""
import numpy as np
import pytest
import torch

import selective_state_space_amd as mb
from selective_state_space_amd import workloads as wl
from gpu_util import assert_close, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _dev(v):
    return None if v is None else torch.from_numpy(np.ascontiguousarray(v)).float().cuda()


def _ref(v):
    return None if v is None else np.asarray(v, np.float32).astype(np.float64)


SHAPES = [  # batch, L, H, P, G, N, K
    (1, 1, 1, 4, 1, 4, 4), (2, 37, 2, 16, 1, 8, 4), (1, 100, 4, 16, 2, 16, 3), (2, 65, 3, 32, 3, 32, 2),
    (1, 17, 2, 64, 1, 128, 1), (1, 300, 24, 64, 1, 128, 4)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("opt", [True, False], ids=["bias_hist", "plain"])
def test_prologue_parity(oracle_mod, shape, opt):
    b, L, H, P, G, N, K = shape
    i = wl.m2_prologue_inputs(np.random.default_rng(sum(shape) + opt), b, L, H, P, G, N, K, hist=opt)
    if not opt:
        i["conv_b"], i["dt_bias"] = None, None
    got = mb.mb_ssd_prologue(_dev(i["xBC"]), _dev(i["conv_w"]), _dev(i["dt"]), _dev(i["A"]), H, P, G, N,
                             conv_b=_dev(i["conv_b"]), x_hist=_dev(i["x_hist"]), dt_bias=_dev(i["dt_bias"]),
                             dt_out=True)
    torch.cuda.synchronize()
    ref = oracle_mod.ssd_prologue(**{k: _ref(v) for k, v in i.items()}, H=H, P=P, G=G, N=N)
    for name, g, r in zip(("X", "B", "C", "logdecay", "dt'"), got, ref):
        assert_close(g, r, "f32", name)


def test_prologue_split_chains_exactly():
    b, L, H, P, G, N, K = 2, 90, 2, 16, 1, 16, 4
    i = wl.m2_prologue_inputs(np.random.default_rng(9), b, L, H, P, G, N, K, hist=False)
    d = {k: _dev(v) for k, v in i.items()}
    whole = mb.mb_ssd_prologue(d["xBC"], d["conv_w"], d["dt"], d["A"], H, P, G, N, conv_b=d["conv_b"],
                               dt_bias=d["dt_bias"])
    s = 37
    f = mb.mb_ssd_prologue(d["xBC"][:, :s].contiguous(), d["conv_w"], d["dt"][:, :s].contiguous(), d["A"], H, P,
                           G, N, conv_b=d["conv_b"], dt_bias=d["dt_bias"])
    g = mb.mb_ssd_prologue(d["xBC"][:, s:].contiguous(), d["conv_w"], d["dt"][:, s:].contiguous(), d["A"], H, P,
                           G, N, conv_b=d["conv_b"], dt_bias=d["dt_bias"],
                           x_hist=d["xBC"][:, s - K + 1:s].contiguous())
    torch.cuda.synchronize()
    for w, a, c in zip(whole, f, g):
        assert torch.equal(w, torch.cat([a, c], dim=1))


def test_prologue_then_ssd(oracle_mod):
    b, L, H, P, G, N, K = 1, 200, 2, 32, 1, 64, 4
    i = wl.m2_prologue_inputs(np.random.default_rng(11), b, L, H, P, G, N, K, hist=True)
    d = {k: _dev(v) for k, v in i.items()}
    X, B, C, ld = mb.mb_ssd_prologue(d["xBC"], d["conv_w"], d["dt"], d["A"], H, P, G, N, conv_b=d["conv_b"],
                                     x_hist=d["x_hist"], dt_bias=d["dt_bias"])
    Y, h = mb.mb_ssd_chunked(X, ld, B, C, None)
    torch.cuda.synchronize()
    Xr, Br, Cr, ldr, _ = oracle_mod.ssd_prologue(**{k: _ref(v) for k, v in i.items()}, H=H, P=P, G=G, N=N)
    Yr, hr = oracle_mod.ssd(Xr, ldr, Br, Cr, None)
    assert_close(Y, Yr, "f32", "Y")
    assert_close(h, hr, "f32", "h")


@pytest.mark.parametrize("shape", [(2, 37, 2, 16, 1, 8, 4), (1, 300, 24, 64, 1, 128, 4), (1, 65, 3, 32, 3, 32, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_prologue_bf16(oracle_mod, shape):
    """bf16 activations in and out: the oracle sees the bf16-rounded inputs;
    the outputs are rounded once, within the bf16 tolerance."""
    b, L, H, P, G, N, K = shape
    i = wl.m2_prologue_inputs(np.random.default_rng(sum(shape) + 7), b, L, H, P, G, N, K, hist=True)
    bf = {k: torch.from_numpy(np.ascontiguousarray(i[k])).to(torch.bfloat16) for k in ("xBC", "x_hist")}
    got = mb.mb_ssd_prologue(bf["xBC"].cuda(), _dev(i["conv_w"]), _dev(i["dt"]), _dev(i["A"]), H, P, G, N,
                             conv_b=_dev(i["conv_b"]), x_hist=bf["x_hist"].cuda(), dt_bias=_dev(i["dt_bias"]))
    torch.cuda.synchronize()
    r = {k: _ref(v) for k, v in i.items()}
    r.update({k: v.double().numpy() for k, v in bf.items()})
    ref = oracle_mod.ssd_prologue(**r, H=H, P=P, G=G, N=N)
    for name, g, rr in zip(("X", "B", "C", "logdecay"), got, ref):
        assert g.dtype == (torch.bfloat16 if name != "logdecay" else torch.float32)
        assert_close(g, rr, "bf16", name)
