"""Oracle of the seed-expanded switching-key format (TEST INFRASTRUCTURE ONLY).

Context: the EncryptedLLM GPU blog, sections 2.5 and 4.4 (switching keys of
hundreds of MB to GB; cut their size when memory or key loading is the limit).
The pages fix no format; the reading taken: a switching key's a rows carry no
secret and are uniform, so a seeded key stores its b rows and one 64-bit seed,
and residue k of a row (digit j, key prime i) is

    a_j[i][k] = floor(w q_i / 2^64),   w = word k of stream j (L + K) + i

of the input generator's SplitMix64 streams under tag 10 (the generator itself
lives in rns_ckks_polynomial_amd/synth.py and only draws 64-bit words).  The
high product maps a uniform 64-bit word to [0, q_i) without a rejection loop.

Written out plainly with numpy: the 128-bit product w q is assembled from
32-bit halves, and only its high word is kept.
"""
from __future__ import annotations

import numpy as np

from rns_ckks_polynomial_amd import synth

TAG_KEY_SEEDED = 10  # stream tag of the a rows


def mulhi_mod(w, q) -> np.ndarray:
    """floor(w q / 2^64) for 64-bit words w and moduli q < 2^64: a residue in [0, q)."""
    w = np.asarray(w, dtype=np.uint64)
    q = np.asarray(q, dtype=np.uint64)
    lo32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    wl, wh, ql, qh = w & lo32, w >> s32, q & lo32, q >> s32
    with np.errstate(over="ignore"):
        m1 = wh * ql + ((wl * ql) >> s32)
        m2 = wl * qh + (m1 & lo32)
        return wh * qh + (m1 >> s32) + (m2 >> s32)


def seeded_key_a(seed: int, dnum: int, moduli, n: int) -> np.ndarray:
    """The a rows [dnum][len(moduli)][n] of a seed-expanded switching key
    (moduli = all L + K key primes, in chain order)."""
    moduli = np.asarray(moduli, dtype=np.uint64)
    tot = len(moduli)
    w = synth.words(seed, TAG_KEY_SEEDED, np.arange(dnum * tot, dtype=np.uint64), n).reshape(dnum, tot, n)
    return mulhi_mod(w, moduli[None, :, None])
