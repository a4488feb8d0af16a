"""GPU parity of the exact base conversion at the shapes where its matrix-core
kernel changes form: bases of 31 primes (the u row is the last row of the only
32-row chunk), 32 and 33 primes (two chunks: the digit table is read from
global memory), for ModUp (digits of alpha primes), ModDown (K special primes,
also summed over BSGS giant steps) and ModRaise (a prefix of l0 primes).  Every
residue against the oracle."""
import numpy as np
import pytest

from gpu_util import dev, gpu_ctx, host, mismatch, oracle_ctx, require_gpu, say
from oracle.bootstrap import mod_raise
from rns_ckks_polynomial_amd import synth
from rns_ckks_polynomial_amd.api import galois_rot

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _cts(o, seed, B, l):
    return synth.uniform_mod(seed, synth.TAG_CT, np.arange(B * 2 * l), np.tile(o.primes[:l], 2 * B),
                             o.n).reshape(B, 2, l, o.n)


def _key(o, seed, j=0):
    tot = o.L + o.K
    return synth.uniform_mod(seed, synth.TAG_KEY, np.arange(o.dnum * 2 * tot) + j * 100_000,
                             np.tile(o.primes, o.dnum * 2), o.n).reshape(o.dnum, 2, tot, o.n)


# (L, K, dnum): digit width alpha = K = 31, 32, 33; levels with a full and a partial last digit.
# L = 150, K = 30: one-chunk digits with 150 targets, i.e. 10 target tiles, which the one-chunk
# conversion covers with a full and a partial workgroup along the target axis.
@pytest.mark.parametrize("L,K,dnum,l", [(62, 31, 2, 62), (62, 31, 2, 40), (64, 32, 2, 64), (66, 33, 2, 50),
                                        (150, 30, 5, 150), (150, 30, 5, 131)])
def test_keyswitch_conversion_shapes(L, K, dnum, l):
    P = (2048, L, K, dnum)
    g, o = gpu_ctx(*P), oracle_ctx(*P)
    seed = 0x5A0 + K + l
    x, y = _cts(o, seed, 2, l), _cts(o, seed + 1, 2, l)
    key = _key(o, seed)
    say(f"conversion shapes L={L} K={K} l={l}: GPU relin / rotate")
    rel = host(g.mul_tensor_relin(dev(x), dev(y), dev(key)))
    ge = galois_rot(o.n, 3)
    rot = host(g.rotate(dev(x), ge, dev(key)))
    for b in range(2):
        ref = o.mul_tensor_relin(x[b], y[b], key, l)
        assert np.array_equal(rel[b], ref), ("relin", b, mismatch(rel[b], ref))
        ref = o.rotate(x[b], ge, key, l)
        assert np.array_equal(rot[b], ref), ("rotate", b, mismatch(rot[b], ref))


@pytest.mark.parametrize("L,K,dnum", [(62, 31, 2), (64, 32, 2)])
def test_bsgs_summed_moddown_shapes(L, K, dnum):
    """Giant steps summed in the ModDown conversion (3 steps: sets of K + 1 rows)."""
    P = (2048, L, K, dnum)
    g, o = gpu_ctx(*P), oracle_ctx(*P)
    l, bs, gs, seed = 30, 2, 4, 0x5B0 + K
    x = _cts(o, seed, 1, l)
    pt = synth.uniform_mod(seed, synth.TAG_DIAG, np.arange(gs * bs * l), np.tile(o.primes[:l], gs * bs),
                           o.n).reshape(gs, bs, l, o.n)
    baby = [None] + [_key(o, seed, 1 + b) for b in range(1, bs)]
    giant = [None] + [_key(o, seed, 100 + j) for j in range(1, gs)]
    dk = lambda ks: [None if k is None else dev(k) for k in ks]  # noqa: E731
    say(f"summed ModDown shapes K={K}: GPU")
    got = host(g.bsgs_linear_transform(dev(x), dev(pt), bs, gs, dk(baby), dk(giant), do_rescale=True))[0]
    ref = o.bsgs(x[0], pt, bs, gs, baby, giant, l, do_rescale=True)
    assert np.array_equal(got, ref), mismatch(got, ref)


@pytest.mark.parametrize("l0", [31, 32, 33])
def test_mod_raise_conversion_shapes(l0):
    P = (2048, 112, 28, 4)
    g, o = gpu_ctx(*P), oracle_ctx(*P)
    x = _cts(o, 0x5C0 + l0, 1, l0)
    say(f"mod_raise l0={l0}: GPU")
    got = host(g.mod_raise(dev(x), 70))[0]
    assert np.array_equal(got, mod_raise(o, x[0], l0, 70)), "mod_raise"
