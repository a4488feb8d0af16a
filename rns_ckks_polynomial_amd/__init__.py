"""MI355X-native RNS-CKKS arithmetic core (HIP kernels behind a C ABI).

`Context` (in .api) binds the C library; `synth` generates seeded inputs.
The binding is imported lazily so CPU-only tools can use `synth` without
torch or the HIP library.
"""
__all__ = ["Context", "galois_rot", "galois_conj", "synth"]


def __getattr__(name):
    if name in ("Context", "galois_rot", "galois_conj"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
