"""Oracle of EvalMod, the modular-reduction stage of bootstrapping
(sin_fold_re / sin_fold_im in the boot profile of the Kestrel article,
section 5.3).

TEST INFRASTRUCTURE ONLY: used by the tests and the smoke check, never by the
product library.  Plain and slow: every ciphertext product and rescale goes
through the pinned C oracle (Ctx.mul_tensor_relin, Ctx.rescale); constant
multiplications and additions are exact Python-integer arithmetic.

The pages name the stage and its cost but not its polynomial.  The reading
taken (the standard cosine / double-angle construction): with slot values x
in [-K, K], u = x / K, p(u) = sum_k cheb[k] T_k(u) in the Chebyshev basis (the
caller passes the interpolant of cos(2 pi (K u - 1/4) / 2^r)), then r times
y <- 2 y^2 - 1, then out = f y; with f = 1 / (2 pi) the result approximates
sin(2 pi x) / (2 pi), i.e. x - round(x) for x near an integer.

Scale bookkeeping (a real number per ciphertext; the residues are exact):
  * constant c "at scale t" is the integer nearest c t, ties to even;
  * multiplying by c at the scale of the prime the following rescale drops
    leaves the scale unchanged;
  * a product of ciphertexts of scales sa, sb rescaled by q has scale sa sb / q;
  * sums and the Chebyshev recurrences keep the scale of their product term.
T_k are built by the doubling recurrences T_2j = 2 T_j^2 - 1 and
T_2j+1 = 2 T_j T_j+1 - T_1, so T_k sits ceil(log2 k) levels below T_1.
"""
from __future__ import annotations

import math

import numpy as np


def const_int(c: float, t: float) -> int:
    """The integer nearest c t (ties to even), as the schedule defines it."""
    return int(np.rint(float(c) * float(t)))


class _Ct:
    """Ciphertext [2][l][n] (uint64 residues, NTT domain) with its scale."""

    def __init__(self, data, l: int, s: float):
        self.data, self.l, self.s = data, l, s


class EvalModOracle:
    def __init__(self, ctx, rlk):
        self.o, self.rlk = ctx, rlk

    def _q(self, j: int) -> int:
        return int(self.o.primes[j])

    def lincomb(self, lo: int, a: _Ct, ma: int, b: _Ct = None, mb: int = 0, add: int = 0):
        """(ma a + mb b + add on c0) modulo each prime, on limbs 0..lo-1."""
        n = self.o.n
        out = np.zeros((2, lo, n), dtype=np.uint64)
        for c in range(2):
            for i in range(lo):
                q = self._q(i)
                v = a.data[c, i].astype(object) * (ma % q)
                if b is not None:
                    v = v + b.data[c, i].astype(object) * (mb % q)
                if c == 0:
                    v = v + (add % q)
                out[c, i] = np.array([int(x) % q for x in v], dtype=np.uint64)
        return out

    def truncate(self, a: _Ct, lo: int) -> _Ct:
        return _Ct(np.ascontiguousarray(a.data[:, :lo]), lo, a.s)

    def cmul_rescale(self, a: _Ct, c: float) -> _Ct:
        w = const_int(c, float(self._q(a.l - 1)))
        prod = self.lincomb(a.l, a, w)
        return _Ct(self.o.rescale(prod, a.l), a.l - 1, a.s)

    def mul_rescale(self, a: _Ct, b: _Ct) -> _Ct:
        m = min(a.l, b.l)
        ta, tb = self.truncate(a, m), self.truncate(b, m)
        prod = self.o.mul_tensor_relin(ta.data, tb.data, self.rlk, m)
        return _Ct(self.o.rescale(prod, m), m - 1, (a.s * b.s) / float(self._q(m - 1)))

    def eval_mod(self, ct, l: int, scale: float, cheb, bound_k: float, double_angles: int, out_factor: float):
        """Returns (out [2][l_out][n], l_out, scale_out)."""
        d = len(cheb) - 1
        assert d >= 1
        T = [None] * (d + 1)
        T[1] = self.cmul_rescale(_Ct(np.asarray(ct, dtype=np.uint64), l, scale), 1.0 / bound_k)
        for k in range(2, d + 1):
            j = k // 2
            if k % 2 == 0:
                p = self.mul_rescale(T[j], T[j])
                T[k] = _Ct(self.lincomb(p.l, p, 2, add=const_int(-1.0, p.s)), p.l, p.s)
            else:
                p = self.mul_rescale(T[j], T[j + 1])
                T[k] = _Ct(self.lincomb(p.l, p, 2, T[1], -1), p.l, p.s)
        m = T[d].l
        wq = float(self._q(m - 1))
        acc = _Ct(np.zeros((2, m, self.o.n), dtype=np.uint64), m, 0.0)
        for k in range(1, d + 1):
            acc = _Ct(self.lincomb(m, acc, 1, T[k], const_int(cheb[k], wq)), m, 0.0)
        p = _Ct(self.o.rescale(acc.data, m), m - 1, T[d].s)
        y = _Ct(self.lincomb(p.l, p, 1, add=const_int(cheb[0], p.s)), p.l, p.s)
        for _ in range(double_angles):
            sq = self.mul_rescale(y, y)
            y = _Ct(self.lincomb(sq.l, sq, 2, add=const_int(-1.0, sq.s)), sq.l, sq.s)
        out = self.cmul_rescale(y, out_factor)
        return out.data, out.l, out.s


def depth(degree: int, double_angles: int) -> int:
    return 3 + math.ceil(math.log2(degree)) + double_angles if degree > 1 else 3 + double_angles


def cosine_cheb(bound_k: float, double_angles: int, degree: int):
    """Chebyshev interpolant (numpy) of cos(2 pi (K u - 1/4) / 2^r) on [-1, 1]."""
    from numpy.polynomial import chebyshev as C
    return C.chebinterpolate(lambda u: np.cos(2 * np.pi * (bound_k * u - 0.25) / 2 ** double_angles), degree)
