"""The C-ABI's argument checks: every call below must be refused with the
documented error code before anything is launched (a context needs the GPU;
no kernel runs on invalid arguments).  Buffers are allocated at full size, so
that no call could read out of bounds even if a check were missing."""
import ctypes as C

import pytest

from gpu_util import dev, gpu_ctx, host, require_gpu, say, torch
from rns_ckks_polynomial_amd import _native as nat
from rns_ckks_polynomial_amd.api import SwitchKey, galois_rot

pytestmark = pytest.mark.gpu
P = (2048, 8, 2, 4)  # n, L, K, dnum (alpha = 2)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def code(fn, *args):
    with pytest.raises(nat.CkksError) as ei:
        fn(*args)
    return ei.value.code


def bufs(g, B=1, l=8):
    n, tot = g.n, g.L + g.K
    x = torch.zeros((B, 2, l, n), dtype=torch.uint64, device="cuda")
    key = torch.zeros((g.dnum, 2, tot, n), dtype=torch.uint64, device="cuda")
    return x, key


def test_workspace_too_small():
    g = gpu_ctx(*P)
    x, key = bufs(g)
    tiny = torch.zeros(16, dtype=torch.uint64, device="cuda")
    assert code(g.rotate, x, galois_rot(2048, 1), key, None, tiny) == nat.EWORKSPACE
    assert code(g.mul_tensor_relin, x, x.clone(), key, None, tiny) == nat.EWORKSPACE
    assert code(g.rescale, x, None, tiny) == nat.EWORKSPACE


def test_misaligned_pointers():
    g = gpu_ctx(*P)
    n, l = 2048, 8
    words = 2 * l * n
    big = torch.zeros(words + 8, dtype=torch.uint64, device="cuda")
    out = torch.zeros(words, dtype=torch.uint64, device="cuda")
    ws = g.workspace(g.workspace_size("rescale", 1, l))
    lib, s = nat.lib(), C.c_void_p(torch.cuda.current_stream().cuda_stream)
    odd = big.data_ptr() + 4
    assert lib.ckks_rescale(g.handle, odd, out.data_ptr(), 1, l, ws.data_ptr(), ws.numel() * 8, s) == nat.EALIGN
    assert lib.ckks_rescale(g.handle, big.data_ptr(), out.data_ptr() + 4, 1, l, ws.data_ptr(), ws.numel() * 8,
                            s) == nat.EALIGN
    need = g.workspace_size("rescale", 1, l)
    wsb = torch.zeros(need // 8 + 2, dtype=torch.uint64, device="cuda")
    assert lib.ckks_rescale(g.handle, big.data_ptr(), out.data_ptr(), 1, l, wsb.data_ptr() + 4, need + 8,
                            s) == nat.EALIGN
    x, key = bufs(g)
    kbig = torch.zeros(key.numel() + 8, dtype=torch.uint64, device="cuda")
    bad = nat.Swk(kbig.data_ptr() + 4, 2048, 8, 2, 4, 0, 0, 0)
    wr = g.workspace(g.workspace_size("rotate", 1, l))
    assert lib.ckks_rotate(g.handle, x.data_ptr(), out.data_ptr(), 1, l, galois_rot(2048, 1), C.byref(bad),
                           wr.data_ptr(), wr.numel() * 8, s) == nat.EALIGN


def test_key_for_another_parameter_set():
    g = gpu_ctx(*P)
    x, key = bufs(g)
    big = torch.zeros(4 * 2 * 10 * 65536, dtype=torch.uint64, device="cuda")  # room for every variant below
    ge = galois_rot(2048, 1)
    for kw in [dict(n=2048, L=9, K=2, dnum=4), dict(n=2048, L=8, K=3, dnum=4), dict(n=2048, L=8, K=2, dnum=5),
               dict(n=65536, L=8, K=2, dnum=4)]:
        say(f"key descriptor {kw}")
        assert code(g.rotate, x, ge, SwitchKey(big, **kw)) == nat.EKEY
        assert code(g.mul_tensor_relin, x, x.clone(), SwitchKey(big, **kw)) == nat.EKEY
    # seeded keys: accepted by rotation / relinearisation, refused where a stored key is needed
    seeded = g.key(key[:, 0].contiguous(), seeded=True, seed=5)
    pt = torch.zeros((2, 2, 8, 2048), dtype=torch.uint64, device="cuda")
    assert code(g.bsgs_linear_transform, x, pt, 2, 2, [None, seeded], [None, key]) == nat.EKEY
    assert code(g.bsgs_linear_transform, x, pt, 2, 2, [None, key], [None, seeded]) == nat.EKEY
    lib, s = nat.lib(), C.c_void_p(torch.cuda.current_stream().cuda_stream)
    stored = g.key(key).descriptor()
    out = torch.zeros_like(key)
    assert lib.ckks_key_expand(g.handle, C.byref(stored), out.data_ptr(), s) == nat.EKEY
    # a reserved field that is not zero
    d = g.key(key).descriptor()
    d.reserved = 1
    wr = g.workspace(g.workspace_size("rotate", 1, 8))
    y = torch.zeros_like(x)
    assert lib.ckks_rotate(g.handle, x.data_ptr(), y.data_ptr(), 1, 8, ge, C.byref(d), wr.data_ptr(),
                           wr.numel() * 8, s) == nat.EKEY


def test_levels_out_of_range():
    g = gpu_ctx(*P)
    lib, s = nat.lib(), C.c_void_p(torch.cuda.current_stream().cuda_stream)
    x, key = bufs(g)
    out = torch.zeros_like(x)
    k = g.key(key).descriptor()
    ws = g.workspace(g.workspace_size("rotate", 1, 8))
    for lvl in (0, 9, -1):
        assert lib.ckks_rotate(g.handle, x.data_ptr(), out.data_ptr(), 1, lvl, galois_rot(2048, 1), C.byref(k),
                               ws.data_ptr(), ws.numel() * 8, s) == nat.ELEVEL
    assert lib.ckks_rescale(g.handle, x.data_ptr(), out.data_ptr(), 1, 1, ws.data_ptr(), ws.numel() * 8,
                            s) == nat.ELEVEL
    assert lib.ckks_prepare_levels(g.handle, 0, 3) == nat.ELEVEL
    assert lib.ckks_prepare_levels(g.handle, 5, 9) == nat.ELEVEL
    assert lib.ckks_prepare_raise(g.handle, 9) == nat.ELEVEL


def test_overlapping_outputs_are_refused():
    g = gpu_ctx(*P)
    x, key = bufs(g, B=2)
    ge = galois_rot(2048, 3)
    assert code(g.rotate, x, ge, key, x) == nat.EINVAL                          # in == out
    flat = torch.zeros(4 * 2 * 8 * 2048, dtype=torch.uint64, device="cuda")
    a = flat[: 2 * 2 * 8 * 2048].view(2, 2, 8, 2048)
    shifted = flat[2048: 2048 + 2 * 2 * 8 * 2048].view(2, 2, 8, 2048)         # one limb further
    b = torch.zeros_like(a)
    assert code(g.mul_tensor_relin, a, b, key, shifted) == nat.EINVAL          # out overlaps a
    assert code(g.mul_tensor_relin, b, a, key, shifted) == nat.EINVAL          # out overlaps b
    assert code(g.rotate, a, ge, key, shifted) == nat.EINVAL
    r_out = flat[2048: 2048 + 2 * 2 * 7 * 2048].view(2, 2, 7, 2048)
    assert code(g.rescale, a, r_out) == nat.EINVAL                             # rescale in place
    pt = torch.zeros((2, 2, 8, 2048), dtype=torch.uint64, device="cuda")
    assert code(g.bsgs_linear_transform, a, pt, 2, 2, [None, key], [None, key], True,
                pt.view(-1)[: 2 * 2 * 7 * 2048].view(2, 2, 7, 2048)) == nat.EINVAL  # out overlaps the diagonals
    # pointwise: the same pointer is allowed, a partial overlap is not
    p = flat[: 4 * 2048].view(1, 4, 2048)
    g.pointwise_mul(p, p, out=p)
    assert code(g.pointwise_mul, p, p, flat[1024: 1024 + 4 * 2048].view(1, 4, 2048)) == nat.EINVAL


def test_level_not_prepared():
    """A chain above CKKS_PREPARE_ALL_MAX_L primes builds its top level only:
    other levels answer CKKS_ENOTREADY until ckks_prepare_levels."""
    g = gpu_ctx(2048, 300, 4, 75)
    x = torch.zeros((1, 2, 299, 2048), dtype=torch.uint64, device="cuda")
    key = torch.zeros((75, 2, 304, 2048), dtype=torch.uint64, device="cuda")
    ge = galois_rot(2048, 1)
    assert code(g.rotate, x, ge, key) == nat.ENOTREADY
    assert code(g.rescale, x) == nat.ENOTREADY
    assert code(g.mod_raise, x[:, :, :5].contiguous(), 299) == nat.ENOTREADY
    g.prepare_levels(299, 299)
    g.prepare_raise(5)
    torch.cuda.synchronize()
    assert not host(g.rotate(x, ge, key)).any()                  # zeros switch to zeros
    assert not host(g.mod_raise(x[:, :, :5].contiguous(), 299)).any()


def test_count_unreduced():
    """Residues are taken as reduced and never range-checked by the operations;
    ckks_count_unreduced is the caller's check.  It counts every residue at or
    above its prime (limb r against prime first_prime + r), and only those."""
    import numpy as np
    from rns_ckks_polynomial_amd import synth
    g = gpu_ctx(*P)
    n, pr = g.n, [int(q) for q in g.primes]
    nl = 4
    x = synth.uniform_mod(7, synth.TAG_POLY, np.arange(3 * nl), np.tile(np.array(pr[:nl], dtype=np.uint64), 3),
                          n).reshape(3, nl, n)
    say("count_unreduced: reduced input")
    assert g.count_unreduced(dev(x)) == 0
    y = x.copy()
    y[0, 0, 5] = pr[0]                # exactly q
    y[1, 2, 2047] = pr[2] + 7         # q + 7
    y[2, 3, 0] = (1 << 64) - 1        # the largest word
    y[2, 1, 9] = pr[1] - 1            # q - 1 is reduced
    t = dev(y)
    assert g.count_unreduced(t) == 3
    # limb r is checked against prime first_prime + r (the chain is ascending)
    z = x[:, :3].copy()
    z[0, 0, 1] = pr[1]                # limb 0: >= pr[0] and >= pr[1]
    z[0, 1, 1] = pr[1]                # limb 1: >= pr[1], below pr[2]
    tz = dev(z)
    assert g.count_unreduced(tz, first_prime=0) == 2
    assert g.count_unreduced(tz, first_prime=1) == 1
    assert g.count_unreduced(t[:0]) == 0
    with pytest.raises(nat.CkksError):
        g.count_unreduced(t, first_prime=g.L + g.K - 2)  # limbs past the last prime
