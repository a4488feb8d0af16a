"""Pins of the oracle's exact base conversion.

Inputs are built from known integers X (Python ints), so the expected output is
simply the centered representative of X reduced modulo each target.  The
adversarial set sits right at the +-B/2 boundary where a fixed-point
shortcut would round the wrong way.
"""
import numpy as np
import pytest

import oracle
import pyref


def _case(nb, extra_targets, values):
    ps = [int(x) for x in oracle.gen_primes(2048, nb + extra_targets)]
    b, t = ps[:nb], ps[nb:] + ps[:2]
    B = 1
    for x in b:
        B *= x
    xs = [v % B for v in values]
    x = np.array([[v % bi for v in xs] for bi in b], dtype=np.uint64)
    got = oracle.base_convert(x, b, t)
    for k, v in enumerate(xs):
        c = pyref.centered(v, B)
        assert -(B // 2) <= c <= B // 2
        assert [int(got[j, k]) for j in range(len(t))] == [c % tj for tj in t], (nb, k)


def _adversarial(B):
    h = (B - 1) // 2
    vals = [0, 1, 2, B - 1, B - 2, h, h + 1, h - 1, h + 2]
    vals += [h - t for t in range(3, 40)] + [h + 1 + t for t in range(3, 40)]
    return vals


@pytest.mark.parametrize("nb", [1, 2, 3, 8, 28])
def test_base_convert_adversarial(nb):
    ps = [int(x) for x in oracle.gen_primes(2048, nb)]
    B = 1
    for x in ps:
        B *= x
    _case(nb, 5, _adversarial(B))


@pytest.mark.parametrize("nb", [4, 28, 263])
def test_base_convert_random(nb):
    import random
    rnd = random.Random(nb)
    ps = [int(x) for x in oracle.gen_primes(2048, nb)]
    B = 1
    for x in ps:
        B *= x
    vals = [rnd.randrange(B) for _ in range(16)] + _adversarial(B)[:8]
    _case(nb, 3, vals)


def test_crt_round_trip_consistency():
    """Conversion to the basis itself is the identity (centered value reduced back)."""
    ps = [int(x) for x in oracle.gen_primes(2048, 5)]
    x = np.array([[(7919 * k + 13 * i) % p for k in range(64)] for i, p in enumerate(ps)], dtype=np.uint64)
    assert np.array_equal(oracle.base_convert(x, ps, ps), x)
