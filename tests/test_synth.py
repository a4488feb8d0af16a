"""Pins of the seeded input generator (rns_ckks_polynomial_amd/synth.py): its
SplitMix64 against the generator's published outputs, and its threaded draw
against the single-block one.  Pins of the oracle's seed-expanded key rows
(oracle/seeded_keys.py): the mapping floor(w q / 2^64) against exact integers."""
import numpy as np

from oracle import seeded_keys
from rns_ckks_polynomial_amd import synth


def test_splitmix64_published_outputs():
    """SplitMix64 seeded with 0 (Steele, Lea, Flood, OOPSLA 2014): its first three outputs."""
    got = [int(synth.splitmix(np.uint64(0), np.uint64(i))) for i in range(3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_mulhi_mod_is_the_exact_high_product():
    rng = np.random.default_rng(7)
    w = rng.integers(0, 2 ** 63, 4096, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, 4096, dtype=np.uint64)
    q = rng.integers(2 ** 59, 2 ** 60, 4096, dtype=np.uint64)
    w[:3] = [2 ** 64 - 1, 0, 2 ** 63]
    q[:3] = [2 ** 60 - 1, 2 ** 59 + 1, 2 ** 64 - 1]
    got = seeded_keys.mulhi_mod(w, q)
    ref = [(int(a) * int(b)) >> 64 for a, b in zip(w, q)]
    assert [int(v) for v in got] == ref
    assert all(int(v) < int(b) for v, b in zip(got, q))


def test_seeded_key_rows_follow_their_streams():
    """Row (j, i) is stream j (L + K) + i of the TAG_KEY_SEEDED generator, mapped
    by the high product; values are uniform over [0, q_i)."""
    moduli = np.array([(1 << 59) + 4097 + 4096 * t for t in range(5)], dtype=np.uint64)
    a = seeded_keys.seeded_key_a(0x5EED, 3, moduli, 64)
    assert a.shape == (3, 5, 64)
    for (j, i, k) in [(0, 0, 0), (2, 4, 63), (1, 3, 17)]:
        w = int(synth.words(0x5EED, seeded_keys.TAG_KEY_SEEDED, np.array([j * 5 + i], dtype=np.uint64), 64)[0, k])
        assert int(a[j, i, k]) == (w * int(moduli[i])) >> 64
    big = seeded_keys.seeded_key_a(3, 1, moduli[:1], 1 << 14)[0, 0].astype(np.float64) / float(moduli[0])
    assert abs(big.mean() - 0.5) < 0.02 and big.min() >= 0 and big.max() < 1


def test_threaded_draw_equals_one_block():
    moduli = np.array([(1 << 59) + 4097 + 4096 * t for t in range(200)], dtype=np.uint64)
    ids = np.arange(200, dtype=np.uint64) + 7
    a = synth.uniform_mod(0xC0DE, synth.TAG_KEY, ids, moduli, 2048)
    b = synth._uniform_rows(0xC0DE, synth.TAG_KEY, ids, moduli, 2048)
    assert np.array_equal(a, b) and bool((a < moduli[:, None]).all())
