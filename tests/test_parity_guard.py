"""A parity comparison must fail hard on a single wrong bit (the article's
pitfall 3: a run that only reports the absence of errors proves nothing).
The planted mistake goes into an oracle result on the CPU; the comparisons
the GPU tests use must catch it: the element-wise equality with its report,
and the per-limb digests of the bootstrap-scale golden files."""
import os
import sys

import numpy as np

import oracle
from gpu_util import mismatch
from rns_ckks_polynomial_amd import synth

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import c4_recipe  # noqa: E402


def _ref():
    o = oracle.Ctx(2048, 6, 2, 3)
    l = 6
    x = synth.uniform_mod(3, synth.TAG_CT, np.arange(2 * l), np.tile(o.primes[:l], 2), 2048).reshape(2, l, 2048)
    return o.rescale(x, l)


def test_one_flipped_bit_fails_the_equality_check():
    ref = _ref()
    for (c, i, k, bit) in [(0, 0, 0, 0), (1, 4, 2047, 59), (0, 2, 1000, 31)]:
        bad = ref.copy()
        bad[c, i, k] ^= np.uint64(1 << bit)
        assert not np.array_equal(bad, ref)
        assert mismatch(bad, ref) == f"1 mismatches, first at {(c, i, k)}"


def test_one_flipped_bit_fails_the_limb_digests():
    ref = _ref()
    want = c4_recipe.limb_digests(ref)
    assert c4_recipe.limb_digests(ref.copy()) == want
    bad = ref.copy()
    bad[1, 3, 77] ^= np.uint64(1 << 17)
    got = c4_recipe.limb_digests(bad)
    assert got[0] == want[0]
    diff = [i for i in range(ref.shape[1]) if got[1][8 * i: 8 * i + 8] != want[1][8 * i: 8 * i + 8]]
    assert diff == [3]
