"""The allocation-free Mamba-2 entry point (mb_ssd_chunked_noalloc, on the
library's static device workspace) against mb_ssd_chunked with a caller
workspace, through the C ABI: two calls in a row on one device, the second
with smaller sizes (so it runs on whatever the first left in the shared
buffer), fp32 and bf16, each compared element by element with the
workspace entry point and with the fp64 oracle at the stated tolerances."""
import ctypes

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


def _both(dev):
    Yw, hw = mb.mb_ssd_chunked(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h0"])
    Y = torch.full_like(Yw, float("nan"))
    h = torch.full_like(hw, float("nan"))
    Yn, hn = mb.mb_ssd_chunked_noalloc(dev["X"], dev["logdecay"], dev["B"], dev["C"], dev["h0"], Y=Y, h_out=h)
    assert Yn.data_ptr() == Y.data_ptr() and hn.data_ptr() == h.data_ptr()
    torch.cuda.synchronize()
    return (Yw, hw), (Yn, hn)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry_point_twice(oracle_mod, dtype):
    shapes = [(2, 1000, 6, 64, 128, 2, 0.05),   # several segments, two groups, h0
              (1, 130, 3, 32, 64, 1, 0.0)]      # smaller: a second call on the same buffer
    for k, (b, L, H, P, N, G, h0_sd) in enumerate(shapes):
        inp = wl.ssd_inputs(np.random.default_rng(300 + k), b, L, H, P, N, G=G, h0_sd=h0_sd)
        dev, ref = prepare(inp, dtype)
        (Yw, hw), (Yn, hn) = _both(dev)
        # the same kernels on the same plan: identical results
        assert torch.equal(Yn, Yw), "call %d: Y differs from the workspace entry point" % k
        assert torch.equal(hn, hw), "call %d: h_out differs from the workspace entry point" % k
        Yr, hr = oracle_mod.ssd(**ref)
        assert_close(Yn, Yr, dtype, "Y (call %d)" % k)
        assert_close(hn, hr, dtype, "h (call %d)" % k)


def test_noalloc_block_shape(oracle_mod):
    """The Mamba-2 block shape (21 MB of workspace) fits the static buffer."""
    inp = wl.ssd_block()
    dev, ref = prepare(inp, "f32")
    (Yw, hw), (Yn, hn) = _both(dev)
    assert torch.equal(Yn, Yw) and torch.equal(hn, hw)
    Yr, hr = oracle_mod.ssd(**ref)
    assert_close(Yn, Yr, "f32", "Y")
    assert_close(hn, hr, "f32", "h")


def test_noalloc_rejects_sizes_beyond_the_buffer():
    """Sizes needing more than 32 MiB of workspace are refused on the host
    (MB_ERR_WORKSPACE) before anything is enqueued: the pointers here are never
    dereferenced."""
    lib = mb.load_library()
    b, L, H, P, G, N = 16, 8192, 24, 64, 1, 128
    need = mb.mb_workspace_size(mb.MB_OP_SSD_CHUNKED, b, L, H, P, G, N, 1, 0)
    assert need > (32 << 20)
    fake = 1 << 40
    span = b * L * H * P * 4
    st = lib.mb_ssd_chunked_noalloc(ctypes.c_void_p(fake), ctypes.c_void_p(fake + 4 * span),
                                    ctypes.c_void_p(fake + 5 * span), ctypes.c_void_p(fake + 6 * span), None,
                                    ctypes.c_void_p(fake + 8 * span), ctypes.c_void_p(fake + 10 * span),
                                    b, L, H, P, G, N, 0, 0, None)
    assert st == 4   # MB_ERR_WORKSPACE
