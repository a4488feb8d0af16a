"""Seeded inputs of the bootstrap-scale linear transforms (the pages' 2100 ->
2083 prime chain: the Kestrel article, section 5.3 boot profile, with
coeff_to_slot / slot_to_coeff as BSGS 32 x 32 per its section 4.4 build
flags).  Only seeds and stream layout live here: the golden-digest script
draws the inputs with the CPU generator (synth.uniform_mod) and the GPU test
with the library's fill kernel, which produce the same residues.

Stream layout of a fill of a [.., rows, n] array with nl limbs per
polynomial: row r is stream stream0 + r and uses chain prime first + r % nl.
"""
N, L, K, DNUM = 2048, 2100, 263, 8
TOT = L + K
BS = GS = 32
BATCH = 8
L_CTS = L          # coeff_to_slot input level (output 2099, then the conjugation key switch)
L_STC = 2084       # slot_to_coeff input level (output 2083)
SEED = 0xC0DE0004

# keys [NKEYS][DNUM][2][TOT][N], one fill with SEED_KEYS from stream 0:
#   key BS - 1 + ... : index b - 1 for the baby rotation by b (b = 1..31),
#   BS - 1 + g - 1 for the giant rotation by g * BS (g = 1..31), then the conjugation key.
NKEYS = (BS - 1) + (GS - 1) + 1
SEED_KEYS = SEED + 1
CONJ_KEY = NKEYS - 1


def baby_key_index(b: int) -> int:
    return b - 1


def giant_key_index(g: int) -> int:
    return BS - 1 + g - 1


# diagonals [GS][BS][l][N] (row (g BS + b) l + i), inputs [BATCH][2][l][N] (row (t 2 + c) l + i)
SEED_CTS_DIAG, SEED_STC_DIAG = SEED + 2, SEED + 3
SEED_CTS_IN, SEED_STC_IN = SEED + 4, SEED + 5
# ciphertext 1 of each batch is the negation of ciphertext 0 (outputs: the negation of ct 0's)
NEGATED = {1: 0}

# dense 4 x 4 BSGS at 2100 primes, batch 2: all three giant steps fall in one batch of the
# GPU's giant-step sum; baby keys = keys 0..2, giant keys = keys 31..33
SMALL_BS = SMALL_GS = 4
SEED_SMALL_DIAG, SEED_SMALL_IN = SEED + 6, SEED + 7
SMALL_BATCH = 2


def small_baby_key_index(b: int) -> int:
    return b - 1


def small_giant_key_index(g: int) -> int:
    return BS - 1 + g - 1


def key_streams(k: int):
    """First stream of key k (its DNUM * 2 * TOT rows follow)."""
    return k * DNUM * 2 * TOT


def limb_digests(ct) -> list:
    """Per-limb digests of a ciphertext [2][l][N] (little-endian uint64 rows):
    for each polynomial, the first 8 hex digits of each limb's SHA-256, concatenated."""
    import hashlib

    import numpy as np
    ct = np.ascontiguousarray(ct, dtype="<u8")
    return ["".join(hashlib.sha256(ct[c, i].tobytes()).hexdigest()[:8] for i in range(ct.shape[1]))
            for c in range(ct.shape[0])]
