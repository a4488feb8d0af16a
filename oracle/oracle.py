"""ctypes front-end of the C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It builds the
shared object with gcc on first use if it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
U64P = C.POINTER(C.c_uint64)
I64P = C.POINTER(C.c_int64)
U32P = C.POINTER(C.c_uint32)
F64P = C.POINTER(C.c_double)


def build(force: bool = False, src: str = None, out: str = None) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, OpenMP)."""
    if os.environ.get("CKKS_ORACLE_LIB"):  # a prebuilt variant (mutation checks of the pins)
        return os.environ["CKKS_ORACLE_LIB"]
    src = src or os.path.join(HERE, "oracle.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11",
                               "-Wall", "-Wno-unused-function", src, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Params(C.Structure):
    _fields_ = [("n", C.c_uint32), ("L", C.c_uint32), ("K", C.c_uint32), ("dnum", C.c_uint32),
                ("primes", U64P), ("psi", U64P)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        L = _lib
        u64, u32 = C.c_uint64, C.c_uint32
        sig = {
            "or_mulmod": (u64, [u64, u64, u64]),
            "or_powmod": (u64, [u64, u64, u64]),
            "or_invmod": (u64, [u64, u64]),
            "or_is_prime": (C.c_int, [u64]),
            "or_gen_primes": (C.c_int, [u32, u32, U64P]),
            "or_min_psi": (u64, [u32, u64]),
            "or_ntt_definition": (None, [u32, u64, u64, U64P, U64P]),
            "or_intt_definition": (None, [u32, u64, u64, U64P, U64P]),
            "or_ntt": (None, [u32, u64, u64, U64P]),
            "or_intt": (None, [u32, u64, u64, U64P]),
            "or_negacyclic_schoolbook": (None, [u32, u64, U64P, U64P, U64P]),
            "or_automorph_coef": (None, [u32, u64, u64, U64P, U64P]),
            "or_base_convert": (None, [u32, u32, U64P, U64P, u32, U64P, U64P]),
            "or_alpha": (u32, [C.POINTER(Params)]),
            "or_beta": (u32, [C.POINTER(Params), u32]),
            "or_tensor": (None, [C.POINTER(Params), u32, U64P, U64P, U64P]),
            "or_keyswitch": (None, [C.POINTER(Params), u32, U64P, U64P, U64P]),
            "or_mul_tensor_relin": (None, [C.POINTER(Params), u32, U64P, U64P, U64P, U64P]),
            "or_rescale": (None, [C.POINTER(Params), u32, U64P, U64P]),
            "or_automorph": (None, [C.POINTER(Params), u32, u64, U64P, U64P]),
            "or_rotate": (None, [C.POINTER(Params), u32, u64, U64P, U64P, U64P]),
            "or_bsgs": (None, [C.POINTER(Params), u32, U64P, U64P, u32, u32, C.POINTER(U64P),
                               C.POINTER(U64P), C.c_int, U64P]),
            "or_mul_acc": (None, [C.POINTER(Params), u32, U64P, U64P, U64P]),
            "or_add": (None, [C.POINTER(Params), u32, u32, U64P, U64P, U64P]),
            "or_encode_coeffs": (None, [u32, F64P, F64P, C.c_double, I64P]),
            "or_coeffs_to_ntt": (None, [C.POINTER(Params), u32, U32P, I64P, U64P]),
            "or_decode": (None, [C.POINTER(Params), u32, U64P, C.c_double, F64P, F64P]),
            "or_keygen_swk": (None, [C.POINTER(Params), U64P, U64P, U64P, I64P, U64P]),
            "or_encrypt": (None, [C.POINTER(Params), u32, U64P, U64P, U64P, I64P, U64P]),
            "or_decrypt": (None, [C.POINTER(Params), u32, U64P, U64P, U64P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
    return _lib


def _p(a: np.ndarray, ptr=U64P):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data_as(ptr)


def _u64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint64)


# ---------------------------------------------------------------- scalars
def mulmod(a, b, q): return int(lib().or_mulmod(a, b, q))
def powmod(a, e, q): return int(lib().or_powmod(a, e, q))
def invmod(a, q): return int(lib().or_invmod(a, q))
def is_prime(x): return bool(lib().or_is_prime(x))
def min_psi(n, q): return int(lib().or_min_psi(n, q))


def gen_primes(n: int, count: int) -> np.ndarray:
    out = np.zeros(count, dtype=np.uint64)
    if lib().or_gen_primes(n, count, _p(out)) != 0:
        raise ValueError("not enough primes")
    return out


# ---------------------------------------------------------------- limbs
def ntt_definition(a, q, psi):
    a = _u64(a); out = np.zeros_like(a)
    lib().or_ntt_definition(len(a), q, psi, _p(a), _p(out)); return out


def intt_definition(a, q, psi):
    a = _u64(a); out = np.zeros_like(a)
    lib().or_intt_definition(len(a), q, psi, _p(a), _p(out)); return out


def ntt(a, q, psi):
    a = _u64(a).copy(); lib().or_ntt(len(a), q, psi, _p(a)); return a


def intt(a, q, psi):
    a = _u64(a).copy(); lib().or_intt(len(a), q, psi, _p(a)); return a


def negacyclic_schoolbook(a, b, q):
    a = _u64(a); b = _u64(b); out = np.zeros_like(a)
    lib().or_negacyclic_schoolbook(len(a), q, _p(a), _p(b), _p(out)); return out


def automorph_coef(a, q, g):
    a = _u64(a); out = np.zeros_like(a)
    lib().or_automorph_coef(len(a), q, g, _p(a), _p(out)); return out


def base_convert(x, bmods, tmods):
    """x: [nb][n] residues -> [nt][n] residues of the centered CRT value."""
    x = _u64(x); b = _u64(bmods); t = _u64(tmods)
    nb, n = x.shape
    out = np.zeros((len(t), n), dtype=np.uint64)
    lib().or_base_convert(n, nb, _p(b), _p(x), len(t), _p(t), _p(out)); return out


# ---------------------------------------------------------------- CKKS
class Ctx:
    """Parameter set: n, L main primes, K special primes, dnum digits."""

    def __init__(self, n: int, L: int, K: int = 0, dnum: int = 1, primes=None):
        self.n, self.L, self.K, self.dnum = n, L, K, dnum
        self.primes = _u64(primes) if primes is not None else gen_primes(n, L + K)
        assert len(self.primes) == L + K
        self.psi = np.array([min_psi(n, int(q)) for q in self.primes], dtype=np.uint64)
        self.p = Params(n, L, K, dnum, _p(self.primes), _p(self.psi))
        self.alpha = (L + dnum - 1) // dnum if dnum else 0

    @property
    def ref(self):
        return C.byref(self.p)

    def beta(self, l): return (l + self.alpha - 1) // self.alpha

    def q(self, i): return int(self.primes[i])

    # transforms on [.., l, n] arrays whose limb r uses prime first + r
    def ntt(self, x, first: int = 0, inverse: bool = False):
        x = _u64(x).copy()
        v = x.reshape(-1, x.shape[-2], x.shape[-1])
        for poly in v:
            for r in range(poly.shape[0]):
                q, psi = int(self.primes[first + r]), int(self.psi[first + r])
                (lib().or_intt if inverse else lib().or_ntt)(self.n, q, psi, _p(poly[r]))
        return x

    def tensor(self, a, b, l):
        a = _u64(a); b = _u64(b); d = np.zeros((3, l, self.n), dtype=np.uint64)
        lib().or_tensor(self.ref, l, _p(a), _p(b), _p(d)); return d

    def keyswitch(self, d, key, l):
        d = _u64(d); key = _u64(key); out = np.zeros((2, l, self.n), dtype=np.uint64)
        lib().or_keyswitch(self.ref, l, _p(d), _p(key), _p(out)); return out

    def mul_tensor_relin(self, a, b, rlk, l):
        a = _u64(a); b = _u64(b); rlk = _u64(rlk); out = np.zeros((2, l, self.n), dtype=np.uint64)
        lib().or_mul_tensor_relin(self.ref, l, _p(a), _p(b), _p(rlk), _p(out)); return out

    def rescale(self, ct, l):
        ct = _u64(ct); out = np.zeros((2, l - 1, self.n), dtype=np.uint64)
        lib().or_rescale(self.ref, l, _p(ct), _p(out)); return out

    def automorph(self, poly, g, l):
        poly = _u64(poly); out = np.zeros((l, self.n), dtype=np.uint64)
        lib().or_automorph(self.ref, l, g, _p(poly), _p(out)); return out

    def rotate(self, ct, g, key, l):
        ct = _u64(ct); key = _u64(key); out = np.zeros((2, l, self.n), dtype=np.uint64)
        lib().or_rotate(self.ref, l, g, _p(ct), _p(key), _p(out)); return out

    def bsgs(self, ct, pt, Bs, G, baby_keys, giant_keys, l, do_rescale=True):
        ct = _u64(ct); pt = _u64(pt)
        keep = []
        def arr(keys, count):
            a = (U64P * count)()
            for i in range(count):
                k = keys[i] if i < len(keys) else None
                if k is not None:
                    k = _u64(k); keep.append(k); a[i] = _p(k)
            return a
        bk, gk = arr(baby_keys, Bs), arr(giant_keys, G)
        lo = l - 1 if do_rescale else l
        out = np.zeros((2, lo, self.n), dtype=np.uint64)
        lib().or_bsgs(self.ref, l, _p(ct), _p(pt), Bs, G, bk, gk, int(do_rescale), _p(out))
        return out

    def mul_acc(self, pt, ct, acc, l):
        """acc[c] += pt (.) ct[c] for both polynomials, in place (acc: contiguous uint64 [2][l][n])."""
        pt = _u64(pt); ct = _u64(ct)
        assert acc.dtype == np.uint64 and acc.flags["C_CONTIGUOUS"]
        lib().or_mul_acc(self.ref, l, _p(pt), _p(ct), _p(acc))
        return acc

    def add(self, a, b, l):
        """a + b limb by limb over [..][l][n] arrays."""
        a = _u64(a); b = _u64(b); out = np.zeros_like(a)
        lib().or_add(self.ref, l, a.size // (l * self.n), _p(a), _p(b), _p(out)); return out

    # ---- functional helpers
    def encode_coeffs(self, z, delta):
        z = np.asarray(z, dtype=np.complex128)
        assert len(z) == self.n // 2
        re = np.ascontiguousarray(z.real); im = np.ascontiguousarray(z.imag)
        out = np.zeros(self.n, dtype=np.int64)
        lib().or_encode_coeffs(self.n, _p(re, F64P), _p(im, F64P), float(delta), _p(out, I64P)); return out

    def coeffs_to_ntt(self, coeffs, prime_idx):
        coeffs = np.ascontiguousarray(coeffs, dtype=np.int64)
        idx = np.ascontiguousarray(prime_idx, dtype=np.uint32)
        out = np.zeros((len(idx), self.n), dtype=np.uint64)
        lib().or_coeffs_to_ntt(self.ref, len(idx), _p(idx, U32P), _p(coeffs, I64P), _p(out)); return out

    def encode(self, z, delta, l):
        return self.coeffs_to_ntt(self.encode_coeffs(z, delta), np.arange(l))

    def decode(self, m_coef, delta, l):
        m_coef = _u64(m_coef)
        re = np.zeros(self.n // 2); im = np.zeros(self.n // 2)
        lib().or_decode(self.ref, l, _p(m_coef), float(delta), _p(re, F64P), _p(im, F64P))
        return re + 1j * im

    def keygen_swk(self, s_ntt, sp_ntt, a, e):
        s_ntt = _u64(s_ntt); sp_ntt = _u64(sp_ntt); a = _u64(a)
        e = np.ascontiguousarray(e, dtype=np.int64)
        key = np.zeros((self.dnum, 2, self.L + self.K, self.n), dtype=np.uint64)
        lib().or_keygen_swk(self.ref, _p(s_ntt), _p(sp_ntt), _p(a), _p(e, I64P), _p(key)); return key

    def encrypt(self, m_ntt, s_ntt, a, e, l):
        m_ntt = _u64(m_ntt); s_ntt = _u64(s_ntt); a = _u64(a)
        e = np.ascontiguousarray(e, dtype=np.int64)
        ct = np.zeros((2, l, self.n), dtype=np.uint64)
        lib().or_encrypt(self.ref, l, _p(m_ntt), _p(s_ntt), _p(a), _p(e, I64P), _p(ct)); return ct

    def decrypt(self, ct, s_ntt, l):
        ct = _u64(ct); s_ntt = _u64(s_ntt); out = np.zeros((l, self.n), dtype=np.uint64)
        lib().or_decrypt(self.ref, l, _p(ct), _p(s_ntt), _p(out)); return out
