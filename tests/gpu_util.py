"""Helpers for the GPU parity tests: host <-> device copies of residue arrays,
and one cached library context per parameter set."""
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint64)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


@functools.lru_cache(maxsize=None)
def gpu_ctx(n, L, K=0, dnum=1):
    from rns_ckks_polynomial_amd.api import Context
    return Context(n, L, K, dnum)


@functools.lru_cache(maxsize=None)
def oracle_ctx(n, L, K=0, dnum=1):
    import oracle
    return oracle.Ctx(n, L, K, dnum)


def mismatch(a, b) -> str:
    a = np.asarray(a); b = np.asarray(b)
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    bad = np.argwhere(a != b)
    return f"{len(bad)} mismatches, first at {tuple(int(v) for v in bad[0]) if len(bad) else None}"


def gfill(g, shape, seed, tag, stream0=0, first_prime=0):
    """Seeded uniform residues generated on the GPU (the library's fill kernel)."""
    t = torch.empty(shape, dtype=torch.uint64, device="cuda")
    g.fill_uniform(t, seed, tag, stream0, first_prime)
    return t


def cfill(o, seed, tag, count, nl, stream0=0, first_prime=0):
    """The same residues regenerated on the CPU: [count][nl][n]."""
    from rns_ckks_polynomial_amd import synth
    mods = np.tile(o.primes[first_prime:first_prime + nl], count)
    return synth.uniform_mod(seed, tag, np.arange(count * nl) + stream0, mods, o.n).reshape(count, nl, o.n)


def say(msg):
    print(msg, flush=True)
