"""Independent pure-Python arithmetic used to pin the oracle.

Nothing here calls the oracle: these are arbitrary-precision restatements of
the definitions (Python ints), small enough to run on tiny inputs, so a
mistake in the C oracle (a wrong index, sign, twiddle or rounding) shows up as
a mismatch.
"""
from __future__ import annotations

import math
import random


# ------------------------------------------------------------ number theory
def _mr(n: int, bases=(2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41)) -> bool:
    if n < 2:
        return False
    for p in bases:
        if n % p == 0:
            return n == p
    d, s = n - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    for a in bases:
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(s - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def _rho(n: int) -> int:
    if n % 2 == 0:
        return 2
    rnd = random.Random(n)
    while True:
        c = rnd.randrange(1, n)
        f = lambda x: (x * x + c) % n  # noqa: E731
        x = y = rnd.randrange(2, n)
        d = 1
        while d == 1:
            x = f(x)
            y = f(f(y))
            d = math.gcd(abs(x - y), n)
        if d != n:
            return d


def factor(n: int) -> dict:
    """Prime factorisation (trial division + Pollard rho)."""
    out: dict = {}
    for p in range(2, 10000):
        while n % p == 0:
            out[p] = out.get(p, 0) + 1
            n //= p
    stack = [n] if n > 1 else []
    while stack:
        m = stack.pop()
        if _mr(m):
            out[m] = out.get(m, 0) + 1
            continue
        d = _rho(m)
        stack += [d, m // d]
    return out


def lucas_prime_certificate(q: int) -> bool:
    """Lucas test: q is prime iff some a has order q-1.  Needs the factorisation of q-1."""
    fs = factor(q - 1)
    for a in range(2, 200):
        if pow(a, q - 1, q) != 1:
            return False
        if all(pow(a, (q - 1) // f, q) != 1 for f in fs):
            return True
    return False


def composite_proof(c: int) -> bool:
    """True if c is provably composite (a Fermat witness or an explicit factor)."""
    for a in (2, 3, 5, 7, 11, 13):
        if math.gcd(a, c) != 1 and c != a:
            return True
        if pow(a, c - 1, c) != 1:
            return True
    if _mr(c):
        return False
    d = _rho(c)
    return 1 < d < c


# ------------------------------------------------------------ polynomials
def ntt_def(a, q, psi):
    n = len(a)
    return [sum(int(a[i]) * pow(psi, i * (2 * j + 1), q) for i in range(n)) % q for j in range(n)]


def intt_def(A, q, psi):
    n = len(A)
    pinv = pow(psi, -1, q)
    ninv = pow(n, -1, q)
    return [ninv * sum(int(A[j]) * pow(pinv, i * (2 * j + 1), q) for j in range(n)) % q for i in range(n)]


def negacyclic_int(a, b):
    """Exact product of integer polynomials in Z[X]/(X^n + 1)."""
    n = len(a)
    out = [0] * n
    for i in range(n):
        if a[i] == 0:
            continue
        for j in range(n):
            k = i + j
            if k < n:
                out[k] += a[i] * b[j]
            else:
                out[k - n] -= a[i] * b[j]
    return out


def compose_xg(a, g):
    """a(X^g) in Z[X]/(X^n + 1), by expanding each monomial X^(i g)."""
    n = len(a)
    out = [0] * n
    for i in range(n):
        e = i * g
        sign = -1 if (e // n) % 2 else 1  # X^n = -1
        out[e % n] += sign * a[i]
    return out


def crt(residues, moduli):
    """Integer in [0, prod) with the given residues (plain Chinese remaindering)."""
    M = 1
    for m in moduli:
        M *= m
    x = 0
    for r, m in zip(residues, moduli):
        Mi = M // m
        x += int(r) * Mi * pow(Mi, -1, m)
    return x % M, M


def centered(x: int, M: int) -> int:
    x %= M
    return x - M if 2 * x > M else x
