"""Oracle of bootstrapping's stage sequence (the boot profile of the Kestrel
article, section 5.3: modraise, coeff_to_slot, conj_extract, sin_fold_re /
sin_fold_im, restore_merge, slot_to_coeff).

TEST INFRASTRUCTURE ONLY: used by the tests, never by the product library.
Plain and slow: ModRaise is the oracle's bigint centered CRT conversion
between inverse and forward NTTs; the linear transforms, rotations, products
and rescales are the pinned C oracle's; multiplying the slots by the imaginary
unit is the negacyclic shift by X^(n/2) in the coefficient domain; EvalMod is
oracle/evalmod.py.  The pages give the stage names and costs only; the
sequence below (one level for coeff_to_slot, one for conj_extract's 1/2, the
EvalMod depth, one for slot_to_coeff) is the reading that takes the pages'
2100-prime chain to their 2083 primes with a degree-31, 6-double-angle EvalMod.
"""
from __future__ import annotations

import numpy as np

from .evalmod import EvalModOracle, _Ct, const_int
from .oracle import base_convert


def mod_raise(o, ct, l0: int, lt: int):
    """[2][l0][n] -> [2][lt][n]: each coefficient lifted to its centered value modulo q_0..q_{l0-1}."""
    coef = o.ntt(np.asarray(ct, dtype=np.uint64), inverse=True)
    out = np.stack([base_convert(coef[c], o.primes[:l0], o.primes[:lt]) for c in range(2)])
    return o.ntt(out)


def times_i(o, ct, l: int):
    """Multiply the slots by the imaginary unit: both polynomials times X^(n/2) (negacyclic)."""
    n, h = o.n, o.n // 2
    coef = o.ntt(np.asarray(ct, dtype=np.uint64), inverse=True)
    out = np.empty_like(coef)
    for c in range(2):
        for i in range(l):
            q = np.uint64(o.primes[i])
            a = coef[c, i]
            neg = np.where(a == 0, a, q - a)
            out[c, i, h:] = a[:h]       # a_k X^(k + n/2)
            out[c, i, :h] = neg[h:]     # a_k X^(k + n/2) = -a_k X^(k - n/2) for k >= n/2
    return o.ntt(out)


def conj_extract(o, em, w, cj, l1: int):
    """Real and imaginary parts of the slots of w (conj = cj, both at level l1):
    re = (w + cj) / 2 and im = (w - cj) X^(n/2) (-1/2), each a constant multiply
    at the prime the following rescale drops, then that rescale (level l1 - 1)."""
    W, Cj = _Ct(w, l1, 0.0), _Ct(cj, l1, 0.0)
    re2 = em.lincomb(l1, W, 1, Cj, 1)
    im2 = times_i(o, em.lincomb(l1, W, 1, Cj, -1), l1)
    qd = float(o.primes[l1 - 1])
    re = o.rescale(em.lincomb(l1, _Ct(re2, l1, 0.0), const_int(0.5, qd)), l1)
    im = o.rescale(em.lincomb(l1, _Ct(im2, l1, 0.0), const_int(-0.5, qd)), l1)
    return re, im


def bootstrap(o, ct, l0: int, lt: int, cts_pt, stc_pt, bs: int, gs: int, baby, giant, conj_key, rlk,
              evalmod_scale: float, cheb, bound_k: float, double_angles: int, out_factor: float):
    """One ciphertext [2][l0][n] -> (out [2][l_out][n], l_out, scale entering slot_to_coeff)."""
    em = EvalModOracle(o, rlk)
    r = mod_raise(o, ct, l0, lt)
    w = o.bsgs(r, cts_pt, bs, gs, baby, giant, lt, do_rescale=True)              # level lt - 1
    l1 = lt - 1
    cj = o.rotate(w, 2 * o.n - 1, conj_key, l1)
    re, im = conj_extract(o, em, w, cj, l1)
    l2 = l1 - 1
    re_o, l3, s3 = em.eval_mod(re, l2, evalmod_scale, cheb, bound_k, double_angles, out_factor)
    im_o, _, _ = em.eval_mod(im, l2, evalmod_scale, cheb, bound_k, double_angles, out_factor)
    v = em.lincomb(l3, _Ct(re_o, l3, 0.0), 1, _Ct(times_i(o, im_o, l3), l3, 0.0), 1)
    out = o.bsgs(v, stc_pt, bs, gs, baby, giant, l3, do_rescale=True)
    return out, l3 - 1, s3
