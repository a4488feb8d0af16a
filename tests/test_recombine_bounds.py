"""Integer bounds of the matrix-core recombination (csrc/mfma_digits.h), on the CPU.

The base conversions and the baby-step giant-step multiply-accumulate form exact
int32 diagonal sums S_s (s < 15) of int8 digit products on the matrix cores and then
rebuild sum_s 256^s S_s mod t in 64-bit integer steps.  GPU parity tests run these
kernels on random residues, whose diagonal sums stay far from their worst case, so
this test walks both recombinations (mf_recombine for up to 2048 rows and
mf_recombine32 for at most 32 rows, with neighbouring diagonals merged) step by
step with 64-bit wraparound. It does that at the digit sums' extremes
(|S_s| = n_s rows 2^14, n_s digit pairs on diagonal s), asserts every intermediate
bound the kernels rely on, and compares the result with the exact big-integer
value.  The chain primes lie in (2^59, 2^59 + 2^52), the range the kernels' final
x >> 59 correction requires.
"""
import random

import pytest

M64 = (1 << 64) - 1
M30 = (1 << 30) - 1


def _s64(x):
    x &= M64
    return x - (1 << 64) if x >> 63 else x


def _i32(x):
    x &= 0xFFFFFFFF
    return x - (1 << 32) if x >> 31 else x


def _shoup_lazy(x, w, wp, q):  # x w - floor(x wp / 2^64) q mod 2^64, in [0, 2q)
    return (x * w - ((x * wp) >> 64) * q) & M64


def _table(q):
    """The per-modulus constants: 256^(8+d) mod q as 30-bit halves in one word, 2^60 mod q
    with its Shoup quotient, q, and 8q - [2^91]_q."""
    row, w = [], pow(2, 64, q)
    for _ in range(7):
        row.append((w & M30) | ((w >> 30) << 32))
        w = w * 256 % q
    r60 = pow(2, 60, q)
    return row + [r60, (r60 << 64) // q, q, 8 * q - pow(2, 91, q)]


def _finish(lo, hi, row, xmax):
    r60, r60p, tq, kfix = row[7:11]
    h0, h1 = hi & M30, hi >> 30
    assert -(1 << 31) <= h1 < (1 << 31)
    h1b = (h1 & 0xFFFFFFFF) ^ 0x80000000
    x = lo + (h0 << 30) + _shoup_lazy(h1b, r60, r60p, tq) + kfix
    assert 0 < x < xmax
    r = _s64(x - (x >> 59) * tq)
    if r < 0:
        r += tq
    assert 0 <= r < tq
    return r


def recombine(S, row):  # up to 2048 rows: |S_s| <= 2^28
    clo = [_i32(c) for c in row[:7]]
    chi = [_i32(c >> 32) for c in row[:7]]
    lo = S[0] + S[1] * 2**8 + S[2] * 2**16 + S[3] * 2**24
    hi = S[4] * 2**2 + S[5] * 2**10 + S[6] * 2**18 + S[7] * 2**26
    for d in range(7):
        lo += S[8 + d] * clo[d]
        hi += S[8 + d] * chi[d]
    assert abs(lo) < 2**61 and abs(hi) < 2**61
    return _finish(lo, hi, row, 1 << 63)


def recombine32(S, row):  # at most 32 rows: P_j = S_2j + 256 S_2j+1 in int32
    clo = [_i32(c) for c in row[:7]]
    chi = [_i32(c >> 32) for c in row[:7]]
    p = [_i32(S[2 * j] + _i32(S[2 * j + 1] * 256)) for j in range(7)]
    assert all(p[j] == S[2 * j] + 256 * S[2 * j + 1] for j in range(7)), "int32 overflow"
    lo = p[0] + p[1] * 2**16
    hi = p[2] * 2**2 + p[3] * 2**18
    for j in range(4, 7):
        lo += p[j] * clo[2 * (j - 4)]
        hi += p[j] * chi[2 * (j - 4)]
    lo += S[14] * clo[6]
    hi += S[14] * chi[6]
    assert abs(lo) < 1.52 * 2**60 and abs(hi) < 0.77 * 2**60
    return _finish(lo, hi, row, 1 << 64)


def _is_prime(n):
    if n < 2:
        return False
    bases = (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37)
    for p in bases:
        if n % p == 0:
            return n == p
    d, r = n - 1, 0
    while d % 2 == 0:
        d //= 2
        r += 1
    for a in bases:
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(r - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def _primes():
    lo = [c for c in range((1 << 59) + 1, (1 << 59) + 1 + 4096 * 3000, 4096) if _is_prime(c)][:3]
    top = (1 << 59) + (1 << 52) - 4095
    hi = [c for c in range(top, top - 4096 * 3000, -4096) if _is_prime(c)][:2]
    return lo + hi


def _npairs(s):
    return min(s, 14 - s) + 1


@pytest.mark.parametrize("rows,fn", [(32, recombine32), (32, recombine), (2048, recombine)])
def test_recombination_at_digit_sum_extremes(rows, fn):
    rng = random.Random(rows)
    for q in _primes():
        row = _table(q)
        for trial in range(600):
            S = []
            for s in range(15):
                b = _npairs(s) * rows * (1 << 14)
                S.append([rng.randint(-b, b), b, -b, rng.choice((b, -b))][trial % 4])
            assert fn(S, row) == sum(S[s] * 256**s for s in range(15)) % q


def test_paired_form_needs_the_32_row_bound():
    # with 64 rows the merged sums leave int32: the paired form is only for one chunk
    S = [_npairs(s) * 64 * (1 << 14) for s in range(15)]
    with pytest.raises(AssertionError):
        recombine32(S, _table(_primes()[0]))
