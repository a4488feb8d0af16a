"""BSGS linear transform of several ciphertexts with diagonals and keys
supplied per use (TEST INFRASTRUCTURE ONLY).

The same definition as the C oracle's or_bsgs (matmul2 with BB x GG in the
Kestrel article's technique table and section 4.4 build flags):

    y = sum_{g < G} rot_{g Bs}( sum_{b < Bs} pt[g][b] (.) rot_b(x) ),  then Rescale(y),

rot_0 the identity, each rotation a full key switch at level l (no hoisting).
It exists for the bootstrap-scale chain (2100 primes, 32 x 32 steps), whose
1024 diagonals (35 GB) and 62 switching keys (39 GB) do not fit a host's
memory at once: `diag(g, b)` and `baby_key(b)` / `giant_key(g)` return one
array at a time, each key is drawn once and applied to every ciphertext,
and the sums are taken with the oracle's or_mul_acc / or_add.
"""
from __future__ import annotations

import numpy as np


def galois_rot(n: int, k: int) -> int:
    return pow(5, k, 2 * n)


def bsgs_stream(o, cts, l: int, Bs: int, G: int, diag, baby_key, giant_key, do_rescale: bool = True, log=None):
    """cts: list of [2][l][n] ciphertexts; returns the list of outputs."""
    say = log or (lambda msg: None)
    rot = [[np.asarray(x, dtype=np.uint64) for x in cts]]
    for b in range(1, Bs):
        key = baby_key(b)
        rot.append([o.rotate(x, galois_rot(o.n, b), key, l) for x in cts])
        del key
        say(f"baby step {b}")
    acc = None
    for g in range(G):
        inner = [np.zeros((2, l, o.n), dtype=np.uint64) for _ in cts]
        for b in range(Bs):
            pt = diag(g, b)
            for t in range(len(cts)):
                o.mul_acc(pt, rot[b][t], inner[t], l)
        if g > 0:
            key = giant_key(g)
            inner = [o.rotate(x, galois_rot(o.n, g * Bs), key, l) for x in inner]
            del key
        acc = inner if acc is None else [o.add(a, x, l) for a, x in zip(acc, inner)]
        say(f"giant step {g}")
    return [o.rescale(a, l) if do_rescale else a for a in acc]
