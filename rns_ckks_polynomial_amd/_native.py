"""ctypes loader of libckksgpu.so (the HIP library).  No fallback: if the
library is missing or fails to load, importing the binding raises."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libckksgpu.so")

OPS = {"relin": 1, "rotate": 2, "rescale": 3, "bsgs": 4, "evalmod": 5, "modraise": 6}
ERRORS = {0: "ok", -1: "invalid argument", -2: "level out of range", -3: "device allocation failed",
          -4: "HIP runtime error", -5: "misaligned pointer", -6: "workspace too small",
          -7: "unsupported parameters", -8: "switching key does not match the context",
          -9: "level tables not prepared"}
EINVAL, ELEVEL, EALIGN, EWORKSPACE, EKEY, ENOTREADY = -1, -2, -5, -6, -8, -9


class CkksError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {ERRORS.get(code, 'error')} ({code})")
        self.code = code


class BootParams(C.Structure):
    """ckks_boot_params (include/ckks_gpu.h)."""
    _fields_ = [("level_raise", C.c_int), ("cts_diags", C.c_void_p), ("stc_diags", C.c_void_p),
                ("bs", C.c_int), ("gs", C.c_int), ("baby_keys", C.POINTER(C.c_void_p)),
                ("giant_keys", C.POINTER(C.c_void_p)), ("conj_key", C.c_void_p), ("rlk", C.c_void_p),
                ("evalmod_scale", C.c_double), ("cheb", C.POINTER(C.c_double)), ("degree", C.c_int),
                ("bound_k", C.c_double), ("double_angles", C.c_int), ("out_factor", C.c_double)]


class Swk(C.Structure):
    """ckks_swk (include/ckks_gpu.h): switching-key descriptor."""
    _fields_ = [("data", C.c_void_p), ("n", C.c_uint32), ("L", C.c_uint32), ("K", C.c_uint32),
                ("dnum", C.c_uint32), ("seeded", C.c_uint32), ("reserved", C.c_uint32), ("seed", C.c_uint64)]


class KernelStat(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int), ("total_ms", C.c_double),
                ("min_ms", C.c_double), ("max_ms", C.c_double)]


class Params(C.Structure):
    _fields_ = [("n", C.c_uint32), ("L", C.c_uint32), ("K", C.c_uint32), ("dnum", C.c_uint32)]


_lib = None

# name -> (restype, argtypes); these are every symbol the C headers declare
SIGNATURES = {
    "ckks_ctx_create": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(Params), C.c_int]),
    "ckks_ctx_destroy": (None, [C.c_void_p]),
    "ckks_ctx_primes": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "ckks_prepare_levels": (C.c_int, [C.c_void_p, C.c_int, C.c_int]),
    "ckks_prepare_raise": (C.c_int, [C.c_void_p, C.c_int]),
    "ckks_strerror": (C.c_char_p, [C.c_int]),
    "ckks_workspace_size": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                      C.POINTER(C.c_size_t)]),
    "ckks_ntt_fwd": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "ckks_ntt_inv": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "ckks_pointwise_mul": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                     C.c_void_p]),
    "ckks_count_unreduced": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "ckks_mul_tensor_relin": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(Swk), C.c_void_p, C.c_int,
                                        C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "ckks_rescale": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_size_t,
                               C.c_void_p]),
    "ckks_rotate": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_uint32, C.POINTER(Swk),
                              C.c_void_p, C.c_size_t, C.c_void_p]),
    "ckks_key_expand": (C.c_int, [C.c_void_p, C.POINTER(Swk), C.c_void_p, C.c_void_p]),
    "ckks_rotate_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_uint32,
                                      C.POINTER(Swk), C.c_void_p]),
    "ckks_bsgs_linear_transform": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p,
                                             C.c_int, C.c_int, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
                                             C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "ckks_eval_mod": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_double,
                                C.POINTER(C.c_double), C.c_int, C.c_double, C.c_int, C.c_double, C.POINTER(Swk),
                                C.c_void_p, C.c_size_t, C.POINTER(C.c_double), C.POINTER(C.c_int), C.c_void_p]),
    "ckks_mod_raise": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                 C.c_size_t, C.c_void_p]),
    "ckks_bootstrap_workspace_size": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p,
                                                C.POINTER(C.c_size_t)]),
    "ckks_bootstrap": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                 C.c_size_t, C.POINTER(C.c_double), C.POINTER(C.c_int), C.c_void_p]),
    "ckks_profile_begin": (C.c_int, [C.c_void_p]),
    "ckks_profile_end": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.POINTER(C.c_int)]),
    "ckks_fill_uniform": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_uint64, C.c_uint64,
                                    C.c_uint64, C.c_void_p]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rns_ckks_polynomial_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(code: int, where: str):
    if code != 0:
        raise CkksError(code, where)
