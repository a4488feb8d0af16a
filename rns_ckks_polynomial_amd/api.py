"""Thin Python binding over the C ABI (include/ckks_gpu.h).

Argument marshalling only: tensors are device tensors (torch.uint64, or
int64 holding the same bits) in the layouts the C header documents; every
step of the computation runs in the HIP library.  Calls are enqueued on the
current torch stream.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _native as nat

U64 = torch.uint64


def _ptr(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if t.dtype not in (torch.uint64, torch.int64):
        raise ValueError("expected 64-bit residues")
    return t.data_ptr()


def _need(t: torch.Tensor, words: int, what: str):
    """The C ABI takes bare pointers: refuse a buffer smaller than what the call reads or writes."""
    if t.numel() < words:
        raise ValueError(f"{what} holds {t.numel()} residues; the call uses {words}")


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class SwitchKey:
    """A switching key on the device with the parameter set it was made for
    (the ckks_swk descriptor).  Stored: data [dnum][2][L+K][n]; seeded: data =
    the b rows [dnum][L+K][n] and `seed` regenerates the a rows."""

    def __init__(self, data: torch.Tensor, n: int, L: int, K: int, dnum: int, seeded: bool = False, seed: int = 0):
        self.data, self.n, self.L, self.K, self.dnum = data, n, L, K, dnum
        self.seeded, self.seed = bool(seeded), int(seed) & (2 ** 64 - 1)

    def descriptor(self) -> nat.Swk:
        rows = self.dnum * (1 if self.seeded else 2) * (self.L + self.K) * self.n
        _need(self.data, rows, "seeded key" if self.seeded else "key")
        return nat.Swk(_ptr(self.data), self.n, self.L, self.K, self.dnum, int(self.seeded), 0, self.seed)


class Context:
    """Parameter set + device tables: n, L main primes, K special primes, dnum digits."""

    def __init__(self, n: int, L: int, K: int = 0, dnum: int = 1, device: int = 0):
        self.n, self.L, self.K, self.dnum, self.device = n, L, K, dnum, device
        self.alpha = (L + dnum - 1) // dnum
        h = C.c_void_p()
        nat.check(nat.lib().ckks_ctx_create(C.byref(h), C.byref(nat.Params(n, L, K, dnum)), device),
                  "ckks_ctx_create")
        self._h = h
        import numpy as np
        self.primes = np.zeros(L + K, dtype=np.uint64)
        self.psi = np.zeros(L + K, dtype=np.uint64)
        nat.check(nat.lib().ckks_ctx_primes(h, self.primes.ctypes.data, self.psi.ctypes.data), "ckks_ctx_primes")
        self._ws = None

    def close(self):
        if getattr(self, "_h", None):
            nat.lib().ckks_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # ------------------------------------------------------------ workspace
    def workspace_size(self, op: str, batch: int, level: int, bs: int = 0, gs: int = 0) -> int:
        out = C.c_size_t()
        nat.check(nat.lib().ckks_workspace_size(self._h, nat.OPS[op], batch, level, bs, gs, C.byref(out)),
                  "ckks_workspace_size")
        return out.value

    def workspace(self, nbytes: int) -> torch.Tensor:
        """A cached device buffer of at least nbytes (grown on demand)."""
        words = (nbytes + 7) // 8
        if self._ws is None or self._ws.numel() < words:
            self._ws = torch.empty(max(words, 1), dtype=U64, device=f"cuda:{self.device}")
        return self._ws

    def _ws_for(self, op, batch, level, bs=0, gs=0, ws=None):
        need = self.workspace_size(op, batch, level, bs, gs)
        if ws is None:
            ws = self.workspace(need)
        return ws, need

    def key(self, data: torch.Tensor, seeded: bool = False, seed: int = 0) -> SwitchKey:
        """Wrap a key tensor made for this context's parameters."""
        return SwitchKey(data, self.n, self.L, self.K, self.dnum, seeded, seed)

    def _swk(self, k) -> nat.Swk:
        """A ckks_swk for a SwitchKey, or for a bare stored-key tensor of this context."""
        return (k if isinstance(k, SwitchKey) else self.key(k)).descriptor()

    def _swk_array(self, keys, count):
        """(array of descriptor addresses for the C call, the descriptors kept alive)."""
        descs = [None if k is None else self._swk(k) for k in keys]
        arr = (C.c_void_p * count)(*[None if d is None else C.addressof(d) for d in descs[:count]])
        return arr, descs

    def prepare_levels(self, lo: int, hi: int):
        nat.check(nat.lib().ckks_prepare_levels(self._h, lo, hi), "ckks_prepare_levels")

    def prepare_raise(self, level_in: int):
        nat.check(nat.lib().ckks_prepare_raise(self._h, level_in), "ckks_prepare_raise")

    def _cts(self, t, B, l, what):
        _need(t, B * 2 * l * self.n, what)
        return _ptr(t)

    # ------------------------------------------------------------ ops
    def ntt_fwd(self, x: torch.Tensor, first_prime: int = 0) -> torch.Tensor:
        count, nl = x.numel() // (x.shape[-1] * x.shape[-2]), x.shape[-2]
        nat.check(nat.lib().ckks_ntt_fwd(self._h, _ptr(x), count, first_prime, nl, _stream()), "ckks_ntt_fwd")
        return x

    def ntt_inv(self, x: torch.Tensor, first_prime: int = 0) -> torch.Tensor:
        count, nl = x.numel() // (x.shape[-1] * x.shape[-2]), x.shape[-2]
        nat.check(nat.lib().ckks_ntt_inv(self._h, _ptr(x), count, first_prime, nl, _stream()), "ckks_ntt_inv")
        return x

    def pointwise_mul(self, a, b, out=None, first_prime: int = 0):
        out = torch.empty_like(a) if out is None else out
        nl = a.shape[-2]
        count = a.numel() // (a.shape[-1] * nl)
        _need(b, a.numel(), "b")
        _need(out, a.numel(), "out")
        nat.check(nat.lib().ckks_pointwise_mul(self._h, _ptr(a), _ptr(b), _ptr(out), count, first_prime, nl,
                                               _stream()), "ckks_pointwise_mul")
        return out

    def count_unreduced(self, x, first_prime: int = 0) -> int:
        """Number of residues of x ([..][nlimbs][n]) at or above their prime (ckks_count_unreduced)."""
        nl = x.shape[-2]
        count = x.numel() // (x.shape[-1] * nl)
        cnt = torch.empty(2, dtype=torch.int32, device=x.device)  # 8-byte aligned counter
        nat.check(nat.lib().ckks_count_unreduced(self._h, _ptr(x), count, first_prime, nl, cnt.data_ptr(),
                                                 _stream()), "ckks_count_unreduced")
        return int(cnt[0].item())

    def mul_tensor_relin(self, a, b, rlk, out=None, ws=None):
        B, _, l, n = a.shape
        out = torch.empty_like(a) if out is None else out
        ws, need = self._ws_for("relin", B, l, ws=ws)
        k = self._swk(rlk)
        nat.check(nat.lib().ckks_mul_tensor_relin(self._h, _ptr(a), self._cts(b, B, l, "b"), C.byref(k),
                                                  self._cts(out, B, l, "out"), B, l,
                                                  _ptr(ws), ws.numel() * 8, _stream()), "ckks_mul_tensor_relin")
        return out

    def rescale(self, x, out=None, ws=None):
        B, _, l, n = x.shape
        out = torch.empty((B, 2, l - 1, n), dtype=x.dtype, device=x.device) if out is None else out
        ws, need = self._ws_for("rescale", B, l, ws=ws)
        nat.check(nat.lib().ckks_rescale(self._h, _ptr(x), self._cts(out, B, l - 1, "out"), B, l, _ptr(ws),
                                         ws.numel() * 8, _stream()),
                  "ckks_rescale")
        return out

    def rotate(self, x, galois_elt: int, key, out=None, ws=None):
        B, _, l, n = x.shape
        out = torch.empty_like(x) if out is None else out
        ws, need = self._ws_for("rotate", B, l, ws=ws)
        k = self._swk(key)
        nat.check(nat.lib().ckks_rotate(self._h, _ptr(x), self._cts(out, B, l, "out"), B, l, galois_elt,
                                        C.byref(k), _ptr(ws),
                                        ws.numel() * 8, _stream()), "ckks_rotate")
        return out

    def rotate_noalloc(self, x, galois_elt: int, key, out=None):
        """ckks_rotate_noalloc: ckks_rotate with the library's device array as workspace."""
        B, _, l, n = x.shape
        out = torch.empty_like(x) if out is None else out
        k = self._swk(key)
        nat.check(nat.lib().ckks_rotate_noalloc(self._h, _ptr(x), self._cts(out, B, l, "out"), B, l, galois_elt,
                                                C.byref(k), _stream()), "ckks_rotate_noalloc")
        return out

    def mul_tensor_relin_seeded(self, a, b, rlk_b, rlk_seed: int, out=None, ws=None):
        """Relinearisation with the key given as its b rows + seed (a seeded ckks_swk)."""
        return self.mul_tensor_relin(a, b, self.key(rlk_b, seeded=True, seed=rlk_seed), out=out, ws=ws)

    def rotate_seeded(self, x, galois_elt: int, key_b, key_seed: int, out=None, ws=None):
        """Rotation with the Galois key given as its b rows + seed (a seeded ckks_swk)."""
        return self.rotate(x, galois_elt, self.key(key_b, seeded=True, seed=key_seed), out=out, ws=ws)

    def key_expand(self, key_b, key_seed: int, out=None):
        """ckks_key_expand: [dnum][L+K][n] b rows + seed -> stored key [dnum][2][L+K][n]."""
        tot = self.L + self.K
        out = torch.empty((self.dnum, 2, tot, self.n), dtype=key_b.dtype, device=key_b.device) if out is None else out
        _need(out, self.dnum * 2 * tot * self.n, "out")
        k = self.key(key_b, seeded=True, seed=key_seed).descriptor()
        nat.check(nat.lib().ckks_key_expand(self._h, C.byref(k), _ptr(out), _stream()), "ckks_key_expand")
        return out

    def bsgs_linear_transform(self, x, diags, bs: int, gs: int, baby_keys, giant_keys, do_rescale=True,
                              out=None, ws=None):
        B, _, l, n = x.shape
        lo = l - 1 if do_rescale else l
        out = torch.empty((B, 2, lo, n), dtype=x.dtype, device=x.device) if out is None else out
        ws, need = self._ws_for("bsgs", B, l, bs, gs, ws=ws)
        bk, _keep_b = self._swk_array(baby_keys, bs)
        gk, _keep_g = self._swk_array(giant_keys, gs)
        _need(diags, gs * bs * l * n, "diags")
        nat.check(nat.lib().ckks_bsgs_linear_transform(self._h, _ptr(x), self._cts(out, B, lo, "out"), B, l,
                                                       _ptr(diags), bs, gs,
                                                       bk, gk, int(do_rescale), _ptr(ws), ws.numel() * 8,
                                                       _stream()), "ckks_bsgs_linear_transform")
        return out

    def mod_raise(self, x, level_out: int, out=None, ws=None):
        """ModRaise (see ckks_mod_raise): [B][2][l][n] -> [B][2][level_out][n]."""
        B, _, l, n = x.shape
        out = torch.empty((B, 2, level_out, n), dtype=x.dtype, device=x.device) if out is None else out
        ws, need = self._ws_for("modraise", B, l, ws=ws)
        nat.check(nat.lib().ckks_mod_raise(self._h, _ptr(x), self._cts(out, B, max(level_out, 0), "out"), B, l,
                                           level_out, _ptr(ws), ws.numel() * 8,
                                           _stream()), "ckks_mod_raise")
        return out

    def bootstrap(self, x, level_raise: int, cts_diags, stc_diags, bs: int, gs: int, baby_keys, giant_keys,
                  conj_key, rlk, evalmod_scale: float, cheb, bound_k: float, double_angles: int,
                  out_factor: float, out=None, ws=None):
        """Bootstrapping (see ckks_bootstrap): returns (out, scale entering slot_to_coeff)."""
        B, _, l0, n = x.shape
        cheb_c = (C.c_double * len(cheb))(*[float(v) for v in cheb])
        bk, _keep_b = self._swk_array(baby_keys, bs)
        gk, _keep_g = self._swk_array(giant_keys, gs)
        ck, rk = self._swk(conj_key), self._swk(rlk)
        lo = level_raise - 3 - (3 + max(0, (len(cheb) - 2).bit_length()) + double_angles)
        p = nat.BootParams(level_raise, _ptr(cts_diags), _ptr(stc_diags), bs, gs, bk, gk, C.addressof(ck),
                           C.addressof(rk),
                           float(evalmod_scale), cheb_c, len(cheb) - 1, float(bound_k), int(double_angles),
                           float(out_factor))
        need = C.c_size_t()
        nat.check(nat.lib().ckks_bootstrap_workspace_size(self._h, B, l0, C.byref(p), C.byref(need)),
                  "ckks_bootstrap_workspace_size")   # validates levels and parameters
        _need(cts_diags, gs * bs * level_raise * n, "cts_diags")
        _need(stc_diags, gs * bs * (lo + 1) * n, "stc_diags")
        ws = self.workspace(need.value) if ws is None else ws
        out = torch.empty((B, 2, lo, n), dtype=x.dtype, device=x.device) if out is None else out
        _need(out, B * 2 * lo * n, "out")
        s_mid, l_out = C.c_double(), C.c_int()
        nat.check(nat.lib().ckks_bootstrap(self._h, _ptr(x), _ptr(out), B, l0, C.byref(p), _ptr(ws), ws.numel() * 8,
                                           C.byref(s_mid), C.byref(l_out), _stream()), "ckks_bootstrap")
        assert l_out.value == lo
        return out, s_mid.value

    def eval_mod(self, x, scale: float, cheb, bound_k: float, double_angles: int, out_factor: float,
                 rlk, out=None, ws=None):
        """EvalMod (see ckks_eval_mod): returns (out, out_scale); out has the
        level ckks_eval_mod reports (the input level minus the depth)."""
        B, _, l, n = x.shape
        cheb = (C.c_double * len(cheb))(*[float(v) for v in cheb])
        degree = len(cheb) - 1
        ceil_log2 = max(0, (degree - 1).bit_length())
        lo = l - (3 + ceil_log2 + double_angles)
        out = torch.empty((B, 2, max(lo, 1), n), dtype=x.dtype, device=x.device) if out is None else out
        ws, need = self._ws_for("evalmod", B, l, degree, ws=ws)
        s_out, l_out = C.c_double(), C.c_int()
        rk = self._swk(rlk)
        nat.check(nat.lib().ckks_eval_mod(self._h, _ptr(x), self._cts(out, B, max(lo, 0), "out"), B, l, float(scale),
                                          cheb, degree, float(bound_k), int(double_angles), float(out_factor),
                                          C.byref(rk),
                                          _ptr(ws), ws.numel() * 8, C.byref(s_out), C.byref(l_out), _stream()),
                  "ckks_eval_mod")
        assert l_out.value == lo
        return out, s_out.value

    # ------------------------------------------------------------ profiling
    def profile_begin(self):
        nat.check(nat.lib().ckks_profile_begin(self._h), "ckks_profile_begin")

    def profile_end(self) -> dict:
        """{kernel name: (launches, total_ms, min_ms, max_ms)} since profile_begin."""
        buf = (nat.KernelStat * 64)()
        cnt = C.c_int()
        nat.check(nat.lib().ckks_profile_end(self._h, buf, 64, C.byref(cnt)), "ckks_profile_end")
        return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms, buf[i].min_ms, buf[i].max_ms)
                for i in range(min(cnt.value, 64))}

    def fill_uniform(self, dst: torch.Tensor, seed: int, tag: int, stream0: int = 0, first_prime: int = 0):
        """Seeded uniform residues (SplitMix64 streams, see include/ckks_synth.h)."""
        nl = dst.shape[-2]
        count = dst.numel() // (dst.shape[-1] * nl)
        nat.check(nat.lib().ckks_fill_uniform(self._h, _ptr(dst), count, first_prime, nl, seed, tag, stream0,
                                              _stream()), "ckks_fill_uniform")
        return dst


def galois_rot(n: int, k: int) -> int:
    """Galois element of a left rotation by k slots."""
    return pow(5, k % (n // 2), 2 * n)


def galois_conj(n: int) -> int:
    return 2 * n - 1
