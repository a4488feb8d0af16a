"""GPU seed-expanded switching keys (ckks_key_expand, and ckks_rotate /
ckks_mul_tensor_relin given a seeded key descriptor): the expanded a rows equal
the oracle's (oracle/seeded_keys.py) bit for bit, and a seeded key switch equals the oracle's
key switch with the expanded key on every residue, at n = 2048 (LDS inner
product) and n = 65536 (generic inner product), plus a decrypt check with a
real seeded Galois key."""
import numpy as np
import pytest

from ckks_helpers import Keys, galois_rot, rel_err
from gpu_util import dev, gpu_ctx, host, mismatch, oracle_ctx, require_gpu, say
from oracle import seeded_keys
from rns_ckks_polynomial_amd import synth

pytestmark = pytest.mark.gpu
LAY = (2048, 112, 28, 4)
C5 = (65536, 40, 8, 5)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _key_b(o, seed):
    tot = o.L + o.K
    return synth.uniform_mod(seed, synth.TAG_KEY, np.arange(o.dnum * tot), np.tile(o.primes, o.dnum),
                             o.n).reshape(o.dnum, tot, o.n)


def _full(o, kb, key_seed):
    return np.ascontiguousarray(np.stack([kb, seeded_keys.seeded_key_a(key_seed, o.dnum, o.primes, o.n)], axis=1))


def _cts(o, seed, B, l):
    return synth.uniform_mod(seed, synth.TAG_CT, np.arange(B * 2 * l), np.tile(o.primes[:l], 2 * B),
                             o.n).reshape(B, 2, l, o.n)


def test_key_expand_matches_generator():
    g, o = gpu_ctx(*LAY), oracle_ctx(*LAY)
    kb = _key_b(o, 0x5EED1)
    for key_seed in (0, 0xFFFFFFFFFFFFFFFF, 0x123456789ABCDEF):
        say(f"key_expand seed={key_seed:#x}")
        got = host(g.key_expand(dev(kb), key_seed))
        assert np.array_equal(got, _full(o, kb, key_seed)), mismatch(got, _full(o, kb, key_seed))


# full chain, a partial last digit, one limb; batches 1 and 3
@pytest.mark.parametrize("l,B", [(112, 1), (29, 3), (1, 1)])
def test_seeded_rotate_and_relin_bitexact(l, B):
    g, o = gpu_ctx(*LAY), oracle_ctx(*LAY)
    kb, key_seed = _key_b(o, 0x5EED2 + l), 0xC0FFEE + l
    full = _full(o, kb, key_seed)
    x, y = _cts(o, 0xA0 + l, B, l), _cts(o, 0xB0 + l, B, l)
    ge = galois_rot(o.n, 5)
    say(f"seeded rotate/relin l={l} B={B}: GPU")
    rot = host(g.rotate_seeded(dev(x), ge, dev(kb), key_seed))
    rel = host(g.mul_tensor_relin_seeded(dev(x), dev(y), dev(kb), key_seed))
    for b in range(B):
        say(f"seeded rotate/relin: oracle ct {b}")
        ref = o.rotate(x[b], ge, full, l)
        assert np.array_equal(rot[b], ref), ("rotate", b, mismatch(rot[b], ref))
        ref = o.mul_tensor_relin(x[b], y[b], full, l)
        assert np.array_equal(rel[b], ref), ("relin", b, mismatch(rel[b], ref))


def test_seeded_rotate_ring65536():
    g, o = gpu_ctx(*C5), oracle_ctx(*C5)
    l, key_seed = 40, 0x65536
    kb = _key_b(o, 0x5EED3)
    x = _cts(o, 0xC5, 1, l)
    ge = galois_rot(o.n, 16)
    say("seeded rotate n=65536: GPU")
    got = host(g.rotate_seeded(dev(x), ge, dev(kb), key_seed))[0]
    say("seeded rotate n=65536: oracle")
    ref = o.rotate(x[0], ge, _full(o, kb, key_seed), l)
    assert np.array_equal(got, ref), mismatch(got, ref)


def test_seeded_galois_key_decrypts():
    o, g = oracle_ctx(*LAY), gpu_ctx(*LAY)
    keys = Keys(o, 0x5EED4)
    l, delta = 112, 2.0 ** 60
    z = synth.uniform_reals(4, synth.TAG_SLOTS, 0, 1024, -1, 1) + 1j * synth.uniform_reals(4, synth.TAG_SLOTS, 1,
                                                                                             1024, -1, 1)
    ct = keys.encrypt(z, delta, l, 0)
    ge = galois_rot(o.n, 9)
    kb, _ = keys.seeded_galois_key(ge, 0xABCD)
    rot = host(g.rotate_seeded(dev(ct[None]), ge, dev(kb), 0xABCD))[0]
    assert rel_err(keys.decrypt(rot, delta, l), np.roll(z, -9)) < 2.0 ** -20


def test_seeded_rejects_bad_arguments():
    g, o = gpu_ctx(*LAY), oracle_ctx(*LAY)
    x = dev(_cts(o, 1, 1, 8))
    short = dev(np.zeros((o.dnum, o.L + o.K - 1, o.n), dtype=np.uint64))
    with pytest.raises(ValueError, match="seeded key"):
        g.rotate_seeded(x, galois_rot(o.n, 1), short, 1)
    kb = dev(_key_b(o, 2))
    with pytest.raises(Exception, match="invalid"):   # even Galois element
        g.rotate_seeded(x, 4, kb, 1)
