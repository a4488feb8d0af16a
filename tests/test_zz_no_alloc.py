"""ckks_rotate_noalloc (the rotation for callers that cannot allocate: its
workspace is the library's device array) against ckks_rotate with a caller
workspace, bit for bit, on two calls in a row (the second smaller, so it runs
on what the first left in the array), plus the size limit."""
import ctypes as C

import numpy as np
import pytest

from gpu_util import gfill, gpu_ctx, host, mismatch, require_gpu, say, torch
from rns_ckks_polynomial_amd import _native as nat
from rns_ckks_polynomial_amd import synth
from rns_ckks_polynomial_amd.api import galois_rot

pytestmark = pytest.mark.gpu
LAY = (2048, 112, 28, 4)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _noalloc(g, x, ge, key, out):
    B, _, l, _ = x.shape
    k = g.key(key).descriptor()
    return nat.lib().ckks_rotate_noalloc(g.handle, x.data_ptr(), out.data_ptr(), B, l, ge, C.byref(k),
                                         C.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_rotate_noalloc_matches_rotate():
    g = gpu_ctx(*LAY)
    key = gfill(g, (4, 2, 140, 2048), 0xA110C, synth.TAG_KEY)
    for (B, l, k) in [(8, 112, 3), (2, 50, 1000)]:
        say(f"rotate_noalloc B={B} l={l} k={k}")
        assert g.workspace_size("rotate", B, l) <= (256 << 20)
        x = gfill(g, (B, 2, l, 2048), 0xA110C + l, synth.TAG_CT)
        ge = galois_rot(2048, k)
        ref = host(g.rotate(x, ge, key))
        out = torch.full_like(x, 7)
        assert _noalloc(g, x, ge, key, out) == 0
        got = host(out)
        assert np.array_equal(got, ref), mismatch(got, ref)


def test_rotate_noalloc_size_limit():
    g = gpu_ctx(*LAY)
    B, l = 16, 112  # about 340 MB of key-switching workspace
    assert g.workspace_size("rotate", B, l) > (256 << 20)
    x = torch.zeros((B, 2, l, 2048), dtype=torch.uint64, device="cuda")
    key = torch.zeros((4, 2, 140, 2048), dtype=torch.uint64, device="cuda")
    out = torch.zeros_like(x)
    assert _noalloc(g, x, galois_rot(2048, 1), key, out) == nat.EWORKSPACE
