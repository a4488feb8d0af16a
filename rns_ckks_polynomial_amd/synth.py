"""Seeded, counter-based synthetic inputs (CPU side).

This module only draws random numbers; it holds none of the RNS-CKKS
arithmetic.  Both the oracle-backed tests and the GPU library's fill kernel
(``ckks_fill_uniform``) implement the same generator, so any element of any
input can be regenerated independently of the order it was produced in.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  With state increment
GAMMA = 0x9e3779b97f4a7c15 and the 64-bit finaliser ``mix64``, the i-th output
(i = 0, 1, ...) of a generator seeded with ``s`` is ``mix64(s + (i+1)*GAMMA)``.

Streams:
  key(seed, tag)            = splitmix(seed, tag)
  stream(seed, tag, j)      = splitmix(key(seed, tag), j)
  word(seed, tag, j, i)     = splitmix(stream(seed, tag, j), i)
Uniform residues in [0, q): element i of stream j tries
``splitmix(word(seed, tag, j, i), r) & (2^60 - 1)`` for r = 0, 1, ... and keeps
the first value below q (after 64 misses it keeps the last value mod q).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
MASK60 = np.uint64((1 << 60) - 1)
MAX_TRIES = 64

# Object tags: one per kind of synthetic input.
TAG_POLY = 1        # plain uniform polynomials (NTT inputs)
TAG_CT = 2          # ciphertext residues
TAG_KEY = 3         # switching-key residues
TAG_DIAG = 4        # plaintext diagonals
TAG_SECRET = 5
TAG_ERROR = 6
TAG_SLOTS = 7
TAG_ENC_A = 8
TAG_KEY_A = 9


def mix64(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def splitmix(state, i):
    """i-th output of SplitMix64 seeded with ``state`` (both broadcastable)."""
    state = np.asarray(state, dtype=np.uint64)
    i = np.asarray(i, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(state + (i + np.uint64(1)) * GAMMA)


def stream_key(seed: int, tag: int, j):
    return splitmix(splitmix(np.uint64(seed), np.uint64(tag)), np.asarray(j, dtype=np.uint64))


def words(seed: int, tag: int, j, count: int) -> np.ndarray:
    """Raw 64-bit words 0..count-1 of stream j (j may be an array -> [len(j), count])."""
    k = np.asarray(stream_key(seed, tag, j), dtype=np.uint64)
    idx = np.arange(count, dtype=np.uint64)
    return splitmix(k[..., None], idx)


def _uniform_rows(seed: int, tag: int, stream_ids: np.ndarray, q: np.ndarray, n: int) -> np.ndarray:
    base = words(seed, tag, stream_ids, n).ravel()  # [r * n]
    q = np.broadcast_to(q[:, None], (len(stream_ids), n)).ravel()
    out = np.empty_like(base)
    pending = np.arange(base.size)
    v = take = None
    for r in range(MAX_TRIES):
        v = splitmix(base[pending], np.uint64(r)) & MASK60
        take = v < q[pending]
        out[pending[take]] = v[take]
        pending = pending[~take]
        if pending.size == 0:
            return out.reshape(len(stream_ids), n)
    out[pending] = v[~take] % q[pending]
    return out.reshape(len(stream_ids), n)


ROWS_PER_TASK = 64  # large draws are split into row blocks drawn on a thread pool


def uniform_mod(seed: int, tag: int, stream_ids, moduli, n: int) -> np.ndarray:
    """Uniform residues: out[r, i] in [0, moduli[r]) for stream stream_ids[r].
    Every element depends only on (seed, tag, stream, i), so drawing row blocks
    on several threads (numpy releases the interpreter lock inside its loops)
    gives the same array."""
    stream_ids = np.atleast_1d(np.asarray(stream_ids, dtype=np.uint64))
    q = np.broadcast_to(np.atleast_1d(np.asarray(moduli, dtype=np.uint64)), (len(stream_ids),))
    rows = len(stream_ids)
    if rows * n <= ROWS_PER_TASK * 2048:
        return _uniform_rows(seed, tag, stream_ids, q, n)
    import concurrent.futures as cf
    import os
    out = np.empty((rows, n), dtype=np.uint64)

    def block(r0):
        r1 = min(rows, r0 + ROWS_PER_TASK)
        out[r0:r1] = _uniform_rows(seed, tag, stream_ids[r0:r1], q[r0:r1], n)

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(block, range(0, rows, ROWS_PER_TASK)))
    return out


def ternary(seed: int, tag: int, j: int, n: int) -> np.ndarray:
    """Values in {-1, 0, 1}: floor(3 * (w >> 32) / 2^32) - 1."""
    w = words(seed, tag, j, n) >> np.uint64(32)
    return ((w * np.uint64(3)) >> np.uint64(32)).astype(np.int64) - 1


def unit_reals(seed: int, tag: int, j: int, count: int) -> np.ndarray:
    """Reals in [0, 1) from the top 53 bits of each word."""
    w = words(seed, tag, j, count) >> np.uint64(11)
    return w.astype(np.float64) * (1.0 / 9007199254740992.0)


def uniform_reals(seed: int, tag: int, j: int, count: int, lo: float, hi: float) -> np.ndarray:
    return lo + (hi - lo) * unit_reals(seed, tag, j, count)


def gaussian_ints(seed: int, tag: int, j: int, n: int, sigma: float = 3.2, bound: int = 19) -> np.ndarray:
    """Rounded Box-Muller normals with standard deviation sigma, clamped to +-bound."""
    u = unit_reals(seed, tag, j, 2 * n)
    u1 = 1.0 - u[:n]  # (0, 1]
    u2 = u[n:]
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2) * sigma
    return np.clip(np.rint(z), -bound, bound).astype(np.int64)
