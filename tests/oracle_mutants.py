"""Mutation check of the oracle's pins (CPU only; not collected by pytest).

Plants one plausible mistake at a time in a copy of oracle.c, builds it, and
runs the CPU test-suite against it (CKKS_ORACLE_LIB points the tests at the
planted copy).  Every mutant must make at least one pin fail.

    python tests/oracle_mutants.py
"""
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "floor_not_centered": ("if (big_cmp(scratch, c->B, w) > 0) {", "if (0) {"),
    "rescale_no_center": ("r[k] = (t[k] > (ql - 1) / 2) ?", "r[k] = (0) ?"),
    "psi_not_min": ("if (cur < best) best = cur;", ""),
    "ntt_twist_inverse": ("for (uint32_t i = 0; i < n; i++) { a[i] = or_mulmod(a[i], p, q); p = or_mulmod(p, psi, q); }",
                          "for (uint32_t i = 0; i < n; i++) { a[i] = or_mulmod(a[i], p, q); p = or_mulmod(p, or_invmod(psi, q), q); }"),
    "automorph_no_neg": ("else out[e - n] = in[i] ? q - in[i] : 0;", "else out[e - n] = in[i];"),
    "key_digit_offbyone": ("uint32_t lo = j * alpha, hi = (j + 1) * alpha < l ? (j + 1) * alpha : l, nb = hi - lo;",
                           "uint32_t lo = j * alpha, hi = (j + 1) * alpha < l ? (j + 1) * alpha : l, nb = hi - lo; "
                           "if (nb > 1 && j == 0) { hi--; nb--; }"),
    "moddown_no_pinv": ("out[(size_t)c * l * n + o] = or_mulmod(submod(accc[o], conv[o], q), Pinv, q);",
                        "out[(size_t)c * l * n + o] = submod(accc[o], conv[o], q);"),
    "schoolbook_cyclic": ("else out[k - n] = submod(out[k - n], p, q);", "else out[k - n] = addmod(out[k - n], p, q);"),
    "intt_no_ninv": ("uint64_t p = or_invmod(n, q);", "uint64_t p = 1;"),
    "gen_primes_skip": ("if (or_is_prime(c)) out[got++] = c;", "if (or_is_prime(c) && c % 7 != 3) out[got++] = c;"),
    "bsgs_giant_step": ("galois_rot(n, (uint64_t)g * Bs)", "galois_rot(n, (uint64_t)g * Bs + 1)"),
    "encode_sign": ("uint64_t a = (m - (e[j] * i) % m) % m;", "uint64_t a = (e[j] * i) % m;"),
}


def main():
    src = open(SRC).read()
    failures = 0
    with tempfile.TemporaryDirectory() as tmp:
        for name, (a, b) in MUTANTS.items():
            assert a in src, name
            c = os.path.join(tmp, name + ".c")
            so = os.path.join(tmp, name + ".so")
            open(c, "w").write(src.replace(a, b, 1))
            subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-I", os.path.dirname(SRC), c, "-o",
                                   so, "-lm"])
            env = dict(os.environ, CKKS_ORACLE_LIB=so)
            r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m",
                                "not gpu"], env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
            caught = r.returncode != 0
            failures += not caught
            print(f"{name:22s} {'caught' if caught else 'NOT CAUGHT'}", flush=True)
    sys.exit(1 if failures else 0)


if __name__ == "__main__":
    main()
