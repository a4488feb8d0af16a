#!/usr/bin/env python3
"""Benchmark of the RNS-CKKS hot path on one MI355X.

Workload (ring degree 2048, 112 main primes + 28 special primes, dnum = 4,
batch of 8 ciphertexts; every input seeded and resident in HBM before the
timed region):
  one step = ct x ct tensor + relinearise + rescale on 8 pairs
           + BSGS 32 x 32 plaintext-matrix x ciphertext on 8 ciphertexts
             (1024 diagonals; 31 baby + 31 giant rotations each) + rescale.
That is 8 + 8 * 62 = 504 key switches per step, and every other step of the
path (NTT/iNTT, tensor, Galois automorphisms, exact base conversion,
rescale, plaintext multiply-accumulate).

Output: one JSON line.  value = key switches per second over whole steps.
After the timed region the same step runs again with the library's
per-launch event profiler on, giving each kernel's average launch time; the
dominant kernel's achieved rate is reported against its roofline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N, L, K, DNUM, BATCH, BS, GS = 2048, 112, 28, 4, 8, 32, 32
ALPHA = (L + DNUM - 1) // DNUM
BETA = (L + ALPHA - 1) // ALPHA
HBM_PEAK_GBS = 8000.0
# VALU: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz; v_mad_u64_u32 (32x32+64) issues at full rate.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# MFMA int8 (dense): 5.0 POP/s.  The base conversions run on it: a 60 x 60-bit
# product is 8 x 8 signed 8-bit digit products, 64 multiply-adds = 128 int8 ops.
MFMA_I8_PEAK_TOPS = 5000.0
I8_OPS_PER_PRODUCT = 128
LIMB = N * 8

# HBM bytes per launch (average over the launches of the step) measured with
# rocprofv3 FETCH_SIZE / WRITE_SIZE on this workload; fetch scaled x2.0 and
# write x1.0, the factors a plain 1 GiB device copy reads from the same
# counters (profiles/bench_step_n2048_l112_b8_hbm_counters.md).  Valid only for
# the kernel sources they were taken on (hash of rns_ckks_polynomial_amd/csrc).
MEASURED_TRAFFIC = {
    "source_sha": "5ae6451959d02f82",
    "bytes_per_launch": {
        "ks_ntt_ext": 1357901990,
        "ks_modup_convert": 809505611,
        "bsgs_mac": 3758289747,
        "rotate_final": 3190481055,
        "ks_inner_product_sum": 2848543492,
        "ks_inner_product_hoisted": 1870706106,
        "giant_final": 304396161,
        "ks_intt_modup": 326825340,
        "ks_intt_moddown": 310284250,
        "ks_inner_product": 462626102,
        "ntt_fwd": 62542593,
        "ntt_inv": 62584445,
        "ks_moddown_u": 231727448,
        "relin_final": 155729082,
        "rescale_final": 118075203,
        "ks_moddown_convert": 747683036
    },
}


# VALU instructions per launch (all waves, rocprofv3 SQ_INSTS_VALU) of the step's kernels, from the
# counter run summarised in profiles/bench_step_n2048_l112_b8_sq_counters.md; like the traffic, valid
# only for the kernel sources they were taken on.  A wave's VALU instruction issues in 4 cycles on
# its SIMD (wave64 on 16 lanes; the 32-bit multiplies included, as measured on this GPU), so
# 1024 SIMDs x 2.4 GHz / 4 = 614.4 G wave-instructions/s is the issue ceiling.
MEASURED_SQ = {
    "source_sha": "5ae6451959d02f82",
    "valu_per_launch": {
        "ks_ntt_ext": 146578432,
        "ks_modup_convert": 102412288,
        "bsgs_mac": 169279488,
        "rotate_final": 293758976,
        "ks_inner_product_sum": 111356672,
        "ks_inner_product_hoisted": 179894400,
        "giant_final": 11640832,
        "ks_intt_modup": 47821312,
        "ks_intt_moddown": 45346560,
        "ks_inner_product": 24222464,
        "ntt_fwd": 6666240,
        "ntt_inv": 8515584,
        "ks_moddown_u": 9221632,
        "relin_final": 12823552,
        "rescale_final": 9583296,
        "ks_moddown_convert": 70903125
    },
}
VALU_ISSUE_PEAK_G = 1024 * 2.4e9 / 4 / 1e9
# Algorithmic bytes of one key switch of the step's shape (112 primes, K = 28, 4 digits) with the
# key amortised over the batch of 8: input polynomial + key / 8 + two output polynomials.
KS_BYTES = 7.44 * 2**20


def csrc_sha() -> str:
    import hashlib
    d = os.path.join(ROOT, "rns_ckks_polynomial_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--profile-steps", type=int, default=1)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-overlap", action="store_true",
                   help="run the step's products and transform in order on one stream")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="budget of the oracle's key-switch sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--boot-chain2100", action="store_true",
                   help="only time the bootstrap of 8 ciphertexts on the 2100 + 263 prime chain "
                        "(19 -> 2100 -> 2083 primes; about 160 GB of HBM)")
    p.add_argument("--boot-reps", type=int, default=2)
    p.add_argument("--c4-only", action="store_true",
                   help="only the 2100-prime coeff_to_slot / slot_to_coeff leg (profiler runs of it)")
    p.add_argument("--c4-reps", type=int, default=3)
    p.add_argument("--ring-only", action="store_true",
                   help="only the ring-65536 leg (profiler runs of it)")
    p.add_argument("--no-c4", action="store_true",
                   help="skip the 2100-prime coeff_to_slot / slot_to_coeff leg (about 150 GB of HBM)")
    p.add_argument("--step-only", action="store_true",
                   help="skip the EvalMod, bootstrapping, seeded-key, ring-65536, NTT-sweep and pointwise legs "
                        "(profiler runs of the step)")
    return p.parse_args()


def cpu_baseline(budget_s: float):
    """The oracle as it stands, timed on this host: relinearisation key switches
    at the same shape (ct x ct at 112 primes), repeated until the budget."""
    import numpy as np

    import oracle
    from rns_ckks_polynomial_amd import synth
    o = oracle.Ctx(N, L, K, DNUM)
    mods = np.tile(o.primes[:L], 2)
    a = synth.uniform_mod(1, synth.TAG_CT, np.arange(2 * L), mods, N).reshape(2, L, N)
    b = synth.uniform_mod(2, synth.TAG_CT, np.arange(2 * L), mods, N).reshape(2, L, N)
    key = synth.uniform_mod(3, synth.TAG_KEY, np.arange(DNUM * 2 * (L + K)), np.tile(o.primes, DNUM * 2),
                            N).reshape(DNUM, 2, L + K, N)
    o.mul_tensor_relin(a, b, key, L)  # warm (thread pool, page faults)
    done, t0 = 0, time.perf_counter()
    while True:
        o.mul_tensor_relin(a, b, key, L)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 2000:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count() or 1
    return {"value": done / el, "unit": "key-switches/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} x (tensor + relinearise) of one ciphertext pair at n=2048, 112+28 primes, dnum=4, "
                      f"{el:.1f} s, OpenMP over limbs/coefficients"}


def cpu_baseline_one_core(budget_s: float):
    """The same oracle sample on one core: a child process (OpenMP reads its
    thread count at start-up) that touches no GPU."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = (f"import json, sys; sys.path.insert(0, {ROOT!r}); import bench; "
            f"print(json.dumps(bench.cpu_baseline({budget_s!r})))")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1:] or ["child failed"]}
    d = json.loads(r.stdout.strip().splitlines()[-1])
    d["cores"] = 1
    d["sample"] = d["sample"].replace("OpenMP over limbs/coefficients", "one OpenMP thread")
    return d


def cpu_baseline_units(skip_c4: bool = False):
    """The oracle as it stands on this host, in the GPU's other units (one sample each):
    limb-NTTs/s (its textbook O(n log n) NTT, one limb per call from Python, one
    thread), BSGS 32 x 32 linear transforms/s at 112 primes (one ciphertext; its
    key switches use OpenMP, its multiply-accumulate one thread), and one key
    switch at 2100 primes (the bootstrap chain: ciphertext 0 of its coeff_to_slot)."""
    import numpy as np

    import oracle
    from rns_ckks_polynomial_amd import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count() or 1
    o = oracle.Ctx(N, L, K, DNUM)
    res = {}
    x = synth.uniform_mod(11, synth.TAG_POLY, np.arange(2 * L), np.tile(o.primes[:L], 2), N).reshape(2, L, N)
    t0 = time.perf_counter()
    o.ntt(x)
    el = time.perf_counter() - t0
    res["limb_ntt"] = {"value": 2 * L / el, "unit": "limb-NTTs/s", "cores": 1,
                       "sample": f"{2 * L} forward limb-NTTs at n={N}, {el:.2f} s"}
    tot = L + K
    ct = synth.uniform_mod(12, synth.TAG_CT, np.arange(2 * L), np.tile(o.primes[:L], 2), N).reshape(2, L, N)
    pt = synth.uniform_mod(13, synth.TAG_DIAG, np.arange(GS * BS * L), np.tile(o.primes[:L], GS * BS),
                           N).reshape(GS, BS, L, N)
    keys = synth.uniform_mod(14, synth.TAG_KEY, np.arange((BS + GS - 2) * DNUM * 2 * tot),
                             np.tile(o.primes, (BS + GS - 2) * DNUM * 2), N).reshape(BS + GS - 2, DNUM, 2, tot, N)
    t0 = time.perf_counter()
    o.bsgs(ct, pt, BS, GS, [None] + [keys[b - 1] for b in range(1, BS)],
           [None] + [keys[BS - 2 + j] for j in range(1, GS)], L, do_rescale=True)
    el = time.perf_counter() - t0
    res["linear_transform_c3"] = {"value": 1 / el, "unit": "linear-transforms/s", "cores": threads,
                                  "sample": f"one BSGS {BS}x{GS} + rescale of one ciphertext at {L} primes "
                                            f"({BS + GS - 2} key switches), {el:.1f} s"}
    del pt, keys
    if not skip_c4:
        l4, t4 = C4_L, C4_L + C4_K
        o4 = oracle.Ctx(C4_N, C4_L, C4_K, C4_DNUM)
        d = synth.uniform_mod(15, synth.TAG_CT, np.arange(l4), o4.primes[:l4], C4_N)
        k4 = synth.uniform_mod(16, synth.TAG_KEY, np.arange(C4_DNUM * 2 * t4), np.tile(o4.primes, C4_DNUM * 2),
                               C4_N).reshape(C4_DNUM, 2, t4, C4_N)
        t0 = time.perf_counter()
        o4.keyswitch(d, k4, l4)
        el = time.perf_counter() - t0
        res["key_switch_c4"] = {"value": 1 / el, "unit": "key-switches/s", "cores": threads,
                                "sample": f"one key switch at {l4} + {C4_K} primes, dnum {C4_DNUM} (ciphertext 0 of "
                                          f"a coeff_to_slot step), {el:.1f} s"}
    return res


EM_DEGREE, EM_ANGLES, EM_K = 31, 3, 8.0


def eval_mod_timing(g, x, rlk, torch, reps: int = 3):
    import numpy as np
    from numpy.polynomial import chebyshev as C
    cheb = C.chebinterpolate(lambda u: np.cos(2 * np.pi * (EM_K * u - 0.25) / 2 ** EM_ANGLES), EM_DEGREE)
    ws = g.workspace(g.workspace_size("evalmod", BATCH, L, EM_DEGREE))
    out, _ = g.eval_mod(x, 2.0 ** 59, cheb, EM_K, EM_ANGLES, 1 / (2 * np.pi), rlk, ws=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.eval_mod(x, 2.0 ** 59, cheb, EM_K, EM_ANGLES, 1 / (2 * np.pi), rlk, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms_per_batch": ms, "ciphertexts_per_s": BATCH / (ms * 1e-3),
            "config": f"batch {BATCH}, level {L} -> {out.shape[2]}, degree {EM_DEGREE} Chebyshev cosine on "
                      f"[-{EM_K:g}, {EM_K:g}], {EM_ANGLES} double angles, scale 2^59, {EM_DEGREE + EM_ANGLES - 1} "
                      f"ct x ct products per ciphertext"}


# Bootstrapping's EvalMod: degree-31 cosine interpolant on [-64, 64] (covers the
# ModRaise overflow of a dense ternary secret at n = 2048) and 6 double angles:
# depth 14, so a refresh consumes 17 levels (2100 -> 2083 on the 2100-prime chain).
BOOT_DEGREE, BOOT_ANGLES, BOOT_K = 31, 6, 64.0


def boot_stc_level(lt: int) -> int:
    """Level of slot_to_coeff's input: lt minus coeff_to_slot, conj_extract's 1/2 and EvalMod's depth."""
    return lt - 2 - (3 + (BOOT_DEGREE - 1).bit_length() + BOOT_ANGLES)


def bootstrap_timing(g, torch, lt, l0, cts, stc, baby, giant, conj, rlk, reps, seed):
    """ms per bootstrap of a batch of 8 ciphertexts at level l0 raised to lt; the
    per-scope kernel time of one more call from the library's event profiler."""
    import numpy as np
    from numpy.polynomial import chebyshev as C

    from rns_ckks_polynomial_amd import synth
    cheb = C.chebinterpolate(lambda u: np.cos(2 * np.pi * (BOOT_K * u - 0.25) / 2 ** BOOT_ANGLES), BOOT_DEGREE)
    x = torch.empty((BATCH, 2, l0, N), dtype=torch.uint64, device="cuda:0")
    g.fill_uniform(x, seed, synth.TAG_CT, 0)
    args = (x, lt, cts, stc, BS, GS, baby, giant, conj, rlk, 2.0 ** 59, cheb, BOOT_K, BOOT_ANGLES, 1 / (2 * np.pi))
    out, _ = g.bootstrap(*args)  # first call: ModRaise tables, workspace
    torch.cuda.synchronize()
    print(f"bootstrap {l0} -> {lt}: first call done", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.bootstrap(*args, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    g.profile_begin()
    g.bootstrap(*args, out=out)
    prof = g.profile_end()
    scopes = {k: round(v[1], 3) for k, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}
    return {"ms_per_batch": ms, "ciphertexts_per_s": BATCH / (ms * 1e-3), "s_per_ciphertext": ms * 1e-3 / BATCH,
            "levels": f"{l0} -> {lt} -> {out.shape[2]}",
            "config": f"batch {BATCH}, n={N}: ModRaise {l0} -> {lt} primes, coeff_to_slot BSGS {BS}x{GS} + rescale, "
                      f"conjugation key switch, EvalMod on {2 * BATCH} ciphertexts (degree {BOOT_DEGREE} cosine on "
                      f"[-{BOOT_K:g}, {BOOT_K:g}], {BOOT_ANGLES} double angles), slot_to_coeff BSGS {BS}x{GS} + "
                      f"rescale",
            "kernel_ms_by_scope": scopes}


def boot_chain2100(args):
    """The 2100 + 263 prime chain (dnum 8): 8 ciphertexts at 19 primes refreshed to 2083."""
    import torch

    from rns_ckks_polynomial_amd import synth
    from rns_ckks_polynomial_amd.api import Context
    n, l, k, dnum, l0 = 2048, 2100, 263, 8, 19
    tot = l + k
    g = Context(n, l, k, dnum, device=0)
    u64, dev = torch.uint64, "cuda:0"
    l3 = boot_stc_level(l)
    g.prepare_levels(l3, l)  # the levels the refresh passes through (long chains prepare the top one only)
    g.prepare_raise(l0)
    keys = torch.empty((BS + GS, dnum, 2, tot, n), dtype=u64, device=dev)
    cts = torch.empty((GS, BS, l, n), dtype=u64, device=dev)
    stc = torch.empty((GS, BS, l3, n), dtype=u64, device=dev)
    seed = 0xC0DE0004
    print("bootstrap 2100-prime chain: filling keys and diagonals", file=sys.stderr, flush=True)
    g.fill_uniform(keys, seed + 1, synth.TAG_KEY, 0)
    g.fill_uniform(cts, seed + 2, synth.TAG_DIAG, 0)
    g.fill_uniform(stc, seed + 3, synth.TAG_DIAG, 0)
    baby = [None] + [keys[i] for i in range(BS - 1)]
    giant = [None] + [keys[BS - 1 + i] for i in range(GS - 1)]
    r = bootstrap_timing(g, torch, l, l0, cts, stc, baby, giant, keys[BS + GS - 2], keys[BS + GS - 1],
                         args.boot_reps, seed)
    r["hbm_bytes_allocated"] = torch.cuda.max_memory_allocated()
    print(json.dumps({"metric": "bootstrap seconds per ciphertext (2100-prime chain)", "value": r["s_per_ciphertext"],
                      "unit": "s/ciphertext", "higher_is_better": False, "n_gpus": 1, "reps": args.boot_reps,
                      "dtype": "u64", "data": "synthetic (seeded SplitMix64 residues, resident in HBM)",
                      "config": {"workload": f"n={n}, {l}+{k} primes, dnum={dnum}, batch {BATCH}: " + r["config"]},
                      "vs_baseline": None, "bootstrap": r}))


def seeded_key_timing(g, torch, a, key, reps: int = 40):
    """Rotation at 112 primes with a stored key vs the same key seed-expanded
    (b rows + seed), batch 1 and batch 8; each call's inner-product kernel time
    from the library's event profiler."""
    from rns_ckks_polynomial_amd.api import galois_rot
    kb = key[:, 0].contiguous()
    ge, seed = galois_rot(N, 3), 0x5EED
    res = {"level": L, "key_bytes_stored": key.numel() * 8, "key_bytes_seeded": kb.numel() * 8}
    for B in (1, BATCH):
        x = a[:B]
        out = torch.empty_like(x)
        ws = g.workspace(g.workspace_size("rotate", B, L))
        calls = {"stored": lambda: g.rotate(x, ge, key, out=out, ws=ws),
                 "seeded": lambda: g.rotate_seeded(x, ge, kb, seed, out=out, ws=ws)}
        row = {}
        for name, f in calls.items():
            f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            g.profile_begin()
            f()
            prof = g.profile_end()
            ip = prof.get("ks_inner_product", (1, 0.0, 0, 0))
            row[name] = {"us_per_call": e0.elapsed_time(e1) / reps * 1e3, "inner_product_us": ip[1] / ip[0] * 1e3}
        row["key_switches_per_s"] = {k: B / (v["us_per_call"] * 1e-6) for k, v in row.items()}
        res[f"batch{B}"] = row
    return res


C4_N, C4_L, C4_K, C4_DNUM, C4_L_STC = 2048, 2100, 263, 8, 2084


def c4_work(l: int, B: int, conj: bool):
    """Algorithmic work of one 32 x 32 BSGS + rescale at level l on B ciphertexts
    (hoisted baby steps: one ModUp; 31 giant rotations; every key switch
    converts exactly), plus one conjugation key switch at l - 1 if `conj`."""
    K, alpha = C4_K, (C4_L + C4_DNUM - 1) // C4_DNUM

    def digits(lv):
        return [min(alpha, lv - j * alpha) for j in range((lv + alpha - 1) // alpha)]

    def up(lv):  # ModUp products per coefficient of one ciphertext
        return sum(m * (lv + K - m) for m in digits(lv))

    def ext_limbs(lv):
        return sum(lv + K - m for m in digits(lv))

    sb, sg = BS - 1, GS - 1
    lc = l - 1
    n_up = [(l, B), (l, sg * B)] + ([(lc, B)] if conj else [])
    n_dn = [(l, (sb + sg) * B)] + ([(lc, B)] if conj else [])
    return {
        "ks_modup_convert": {"products": sum(up(lv) * c * N for lv, c in n_up)},
        "ks_moddown_convert": {"products": sum(2 * K * lv * c * N for lv, c in n_dn)},
        "ks_ntt_ext": {"bytes": sum(2 * ext_limbs(lv) * c * LIMB for lv, c in n_up)},
        "bsgs_mac": {"mads": 4 * GS * BS * 2 * B * l * N,
                     "bytes": (GS * BS * l + BS * 2 * B * l + GS * 2 * B * l) * LIMB},
    }


def c4_timing(torch, reps: int = 3):
    """The bootstrap-scale linear transforms at their real shape (2100 + 263
    primes, dnum 8, batch 8, BSGS 32 x 32, seeded dense diagonals and keys):
    coeff_to_slot = BSGS + rescale at 2100 primes, then the conjugation key
    switch at 2099; slot_to_coeff = BSGS + rescale at 2084 primes.  Each timed
    over `reps` runs after one untimed run; per-kernel times from one more
    profiled run of each."""
    from rns_ckks_polynomial_amd import synth
    from rns_ckks_polynomial_amd.api import Context
    n, l, k, dnum, lst = C4_N, C4_L, C4_K, C4_DNUM, C4_L_STC
    tot = l + k
    g = Context(n, l, k, dnum, device=0)
    g.prepare_levels(lst, l)
    u64, dev = torch.uint64, "cuda:0"
    seed = 0xC0DE0004
    print("c4: drawing keys and diagonals (110 GB)", file=sys.stderr, flush=True)
    keys = torch.empty((BS + GS - 1, dnum, 2, tot, n), dtype=u64, device=dev)
    g.fill_uniform(keys, seed + 1, synth.TAG_KEY, 0)
    cts_d = torch.empty((GS, BS, l, n), dtype=u64, device=dev)
    stc_d = torch.empty((GS, BS, lst, n), dtype=u64, device=dev)
    g.fill_uniform(cts_d, seed + 2, synth.TAG_DIAG, 0)
    g.fill_uniform(stc_d, seed + 3, synth.TAG_DIAG, 0)
    x = torch.empty((BATCH, 2, l, n), dtype=u64, device=dev)
    xs = torch.empty((BATCH, 2, lst, n), dtype=u64, device=dev)
    g.fill_uniform(x, seed + 4, synth.TAG_CT, 0)
    g.fill_uniform(xs, seed + 5, synth.TAG_CT, 0)
    baby = [None] + [keys[b - 1] for b in range(1, BS)]
    giant = [None] + [keys[BS - 2 + j] for j in range(1, GS)]
    conj = keys[BS + GS - 2]
    w = torch.empty((BATCH, 2, l - 1, n), dtype=u64, device=dev)
    cj, y = torch.empty_like(w), torch.empty((BATCH, 2, lst - 1, n), dtype=u64, device=dev)
    ws = g.workspace(max(g.workspace_size("bsgs", BATCH, l, BS, GS), g.workspace_size("rotate", BATCH, l - 1)))

    def cts():
        g.bsgs_linear_transform(x, cts_d, BS, GS, baby, giant, do_rescale=True, out=w, ws=ws)
        g.rotate(w, 2 * n - 1, conj, out=cj, ws=ws)

    def stc():
        g.bsgs_linear_transform(xs, stc_d, BS, GS, baby, giant, do_rescale=True, out=y, ws=ws)

    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fn, lv, conj_ks in (("coeff_to_slot", cts, l, True), ("slot_to_coeff", stc, lst, False)):
        fn()
        torch.cuda.synchronize()
        print(f"c4 {name}: first run done", file=sys.stderr, flush=True)
        times = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        ms = times[len(times) // 2]
        g.profile_begin()
        fn()
        prof = g.profile_end()
        ks = BATCH * (BS + GS - 2 + (1 if conj_ks else 0))
        work = c4_work(lv, BATCH, conj_ks)
        kern = {}
        for kn, (cnt, tot_ms, mn, mx) in prof.items():
            row = {"launches": cnt, "avg_us": tot_ms / cnt * 1e3, "total_ms": tot_ms}
            wk = work.get(kn, {})
            if "products" in wk:
                row["algo_int8_TOPs"] = wk["products"] * I8_OPS_PER_PRODUCT / (tot_ms * 1e-3) / 1e12
            if "bytes" in wk:
                row["algo_GBps"] = wk["bytes"] / (tot_ms * 1e-3) / 1e9
            if "mads" in wk:
                row["algo_Tmads"] = wk["mads"] / (tot_ms * 1e-3) / 1e12
            kern[kn] = row
        dom = max(kern, key=lambda kk: kern[kk]["total_ms"])
        d = kern[dom]
        if "algo_int8_TOPs" in d:
            roof = {"bound": "mfma", "achieved": d["algo_int8_TOPs"], "peak": MFMA_I8_PEAK_TOPS, "unit": "int8 TOP/s"}
        elif "algo_Tmads" in d:
            roof = {"bound": "alu", "achieved": d["algo_Tmads"], "peak": VALU_PEAK_TOPS, "unit": "T int32-MAD/s"}
        else:
            roof = {"bound": "hbm", "achieved": d.get("algo_GBps"), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof.update({"kernel": dom, "frac": roof["achieved"] / roof["peak"] if roof["achieved"] else None,
                     "avg_launch_us": d["avg_us"], "kernel_ms": d["total_ms"]})
        res[name] = {"ms_per_batch": ms, "ms_all": times, "linear_transforms_per_s": BATCH / (ms * 1e-3),
                     "key_switches_per_s": ks / (ms * 1e-3), "key_switches": ks, "level": lv,
                     "roofline": roof, "kernels": kern}
        print(f"c4 {name}: {ms:.1f} ms per batch", file=sys.stderr, flush=True)
    res["config"] = (f"n={n}, {l}+{k} primes, dnum={dnum}, batch {BATCH}, BSGS {BS}x{GS}, dense seeded diagonals: "
                     f"coeff_to_slot at {l} (+ conjugation key switch at {l - 1}), slot_to_coeff at {lst}")
    res["hbm_bytes_allocated"] = torch.cuda.max_memory_allocated()
    del keys, cts_d, stc_d, x, xs, w, cj, y, ws, g
    torch.cuda.empty_cache()
    return res


def ring65536_timing(torch, reps: int = 5):
    """The ring-65536 workload: n = 65536, 40 + 8 primes, dnum 5, 4 ciphertext pairs.  Batched NTT /
    iNTT over the [4][2][40] limbs, tensor + relinearise of the 4 pairs (4 key switches) and rotations
    of the 4 products (4 key switches each, one rotation key reused)."""
    from rns_ckks_polynomial_amd import synth
    from rns_ckks_polynomial_amd.api import Context, galois_rot
    n, l, k, dnum, b = 65536, 40, 8, 5, 4
    g = Context(n, l, k, dnum, device=0)
    u64 = torch.uint64
    x = torch.empty((b, 2, l, n), dtype=u64, device="cuda")
    y = torch.empty_like(x)
    rlk = torch.empty((dnum, 2, l + k, n), dtype=u64, device="cuda")
    rk = torch.empty_like(rlk)
    g.fill_uniform(x, 0xC0DE0005, synth.TAG_CT, 0)
    g.fill_uniform(y, 0xC0DE0006, synth.TAG_CT, 0)
    g.fill_uniform(rlk, 0xC0DE0005, synth.TAG_KEY, 0)
    g.fill_uniform(rk, 0xC0DE0007, synth.TAG_KEY, 0)
    ws = g.workspace(max(g.workspace_size("relin", b, l), g.workspace_size("rotate", b, l)))
    prod, rot = torch.empty_like(x), torch.empty_like(x)
    limbs = x.clone().view(b * 2, l, n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn(0)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ntt_ms = timed(lambda i: (g.ntt_fwd(limbs), g.ntt_inv(limbs))) / 2
    relin_ms = timed(lambda i: g.mul_tensor_relin(x, y, rlk, out=prod, ws=ws))
    rot_ms = timed(lambda i: g.rotate(prod, galois_rot(n, 1 << (i % 16)), rk, out=rot, ws=ws))
    nl = b * 2 * l
    out = {"limb_ntts_per_s": nl / (ntt_ms * 1e-3),
           "ntt_algo_GBps": nl * 2 * n * 8 / (ntt_ms * 1e-3) / 1e9,
           "ntt_ms_per_direction": ntt_ms,
           "key_switches_per_s_relin": b / (relin_ms * 1e-3), "relin_ms": relin_ms,
           "key_switches_per_s_rotate": b / (rot_ms * 1e-3), "rotate_ms": rot_ms,
           "config": "n=65536, 40+8 primes, dnum=5, 4 ciphertext pairs: NTT/iNTT of [4][2][40] limbs, "
                     "tensor+relin (4 key switches), rotation by 2^i (4 key switches)"}
    del x, y, rlk, rk, ws, prod, rot, limbs, g
    torch.cuda.empty_cache()
    return out


def kernel_work():
    """Algorithmic work of each kernel per benchmark step (all launches of that
    kernel in one step; launches differ in size since BSGS batches its steps).
    bytes: residues that must be read + written once (twiddles/tables excluded);
    mads: 32x32-bit multiply-adds, 4 per 60x60-bit product (the minimum on a
    32-bit multiplier); products: 60x60-bit products of the base conversions,
    which run on the matrix cores (I8_OPS_PER_PRODUCT int8 ops each)."""
    B, l, el, a, beta = BATCH, L, L + K, ALPHA, BETA
    sb, sg = BS - 1, GS - 1           # baby / giant key switches per ciphertext
    n_up = (1 + 1 + sg) * B           # ciphertexts through ModUp: relin, hoisted baby, giant
    n_dn = (1 + sb + sg) * B          # ciphertexts through ModDown
    limb = LIMB
    return {
        "ks_intt_modup": {"bytes": 2 * n_up * l * limb},
        "ks_modup_u": {"bytes": n_up * l * limb},
        "ks_modup_convert": {"products": n_up * beta * a * (l + K - a) * N,
                             "bytes": (n_up * l + n_up * beta * (el - a)) * limb},
        "ks_ntt_ext": {"bytes": 2 * n_up * beta * (el - a) * limb},
        # relinearisation (all limbs) + the giant steps' P-limbs
        "ks_inner_product": {"bytes": (B * (beta + 2) * el + 2 * beta * el
                                       + sg * B * (beta + 2) * K + sg * 2 * beta * K) * limb},
        # giant steps' Q-limbs summed over the steps: digits + c0 in, 4 partial sums out
        "ks_inner_product_sum": {"bytes": (sg * B * (beta + 1) * l + sg * 2 * beta * l + 4 * B * 2 * l) * limb},
        "ks_inner_product_hoisted": {"bytes": (sb * B * (beta + 2) * el + sb * 2 * beta * el) * limb},
        "ks_intt_moddown": {"bytes": 2 * n_dn * 2 * K * limb},
        "ks_moddown_u": {"bytes": n_dn * 2 * K * limb},
        # giant-step conversions are summed in the kernel: one output per ciphertext
        "ks_moddown_convert": {"products": n_dn * 2 * K * l * N,
                               "bytes": (n_dn * 2 * K + (1 + sb + 1) * B * 2 * l) * limb},
        "rotate_final": {"bytes": sb * B * 7 * l * limb},
        # accumulators, converted P-part, both input ciphertexts in, the product out
        "relin_final": {"bytes": B * 2 * l * 5 * limb},
        # two rescales per step (the product and the transform's output): 2l limbs in, 2(l - 1) out
        "rescale_final": {"bytes": 2 * B * 2 * (2 * l - 1) * limb},
        # conv in, 4 partial sums in, output read + written
        "giant_final": {"bytes": B * 2 * l * (1 + 4 + 2) * limb},
        "bsgs_mac": {"mads": 4 * GS * BS * 2 * B * l * N,
                     "bytes": (GS * BS * l + BS * 2 * B * l + GS * 2 * B * l) * limb},
        "ntt_fwd": {"bytes": 2 * B * 2 * l * limb, "standalone": True},
        "ntt_inv": {"bytes": 2 * B * 2 * l * limb, "standalone": True},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the hot path is measured on one "
                                   "GPU's share; pass --gpus 1"}))
        sys.exit(2)
    if args.boot_chain2100:
        boot_chain2100(args)
        return
    if args.ring_only:
        import torch
        r = ring65536_timing(torch)
        print(json.dumps({"metric": "limb-NTTs/s at n=65536", "unit": "limb-NTTs/s", "value": r["limb_ntts_per_s"],
                          "n_gpus": 1, "dtype": "u64", "data": "synthetic", "config": {"workload": r["config"]},
                          "ring65536": r}))
        return
    if args.c4_only:
        import torch
        r = c4_timing(torch, args.c4_reps)
        print(json.dumps({"metric": "BSGS 32x32 linear transforms/s at 2100 primes", "unit": "linear-transforms/s",
                          "value": r["coeff_to_slot"]["linear_transforms_per_s"], "n_gpus": 1, "dtype": "u64",
                          "data": "synthetic", "config": {"workload": r["config"]}, "c4": r}))
        return
    import torch

    from rns_ckks_polynomial_amd import synth
    from rns_ckks_polynomial_amd.api import Context
    dev = "cuda:0"
    g = Context(N, L, K, DNUM, device=0)
    u64 = torch.uint64
    a = torch.empty((BATCH, 2, L, N), dtype=u64, device=dev)
    b = torch.empty_like(a)
    rlk = torch.empty((DNUM, 2, L + K, N), dtype=u64, device=dev)
    keys = torch.empty((BS + GS - 2, DNUM, 2, L + K, N), dtype=u64, device=dev)
    diags = torch.empty((GS, BS, L, N), dtype=u64, device=dev)
    seed = 0xC0DE0002
    g.fill_uniform(a, seed, synth.TAG_CT, 0)
    g.fill_uniform(b, seed + 1, synth.TAG_CT, 0)
    g.fill_uniform(rlk, seed, synth.TAG_KEY, 0)
    g.fill_uniform(keys, seed + 2, synth.TAG_KEY, 0)
    g.fill_uniform(diags, 0xC0DE0003, synth.TAG_DIAG, 0)
    baby = [None] + [keys[i] for i in range(BS - 1)]
    giant = [None] + [keys[BS - 1 + i] for i in range(GS - 1)]
    prod = torch.empty_like(a)
    res = torch.empty((BATCH, 2, L - 1, N), dtype=u64, device=dev)
    lt = torch.empty_like(res)
    ws = g.workspace(max(g.workspace_size("bsgs", BATCH, L, BS, GS), g.workspace_size("relin", BATCH, L)))
    # the products (tensor + relinearisation + rescale) do not depend on the transform: the timed
    # steps run them on a second stream (default priority) with a workspace of their own, so they
    # fill the chip while the transform's launches drain; split timing and profiling run in order
    ws2 = g.workspace(max(g.workspace_size("relin", BATCH, L), g.workspace_size("rescale", BATCH, L)))
    side = torch.cuda.Stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    parts = {"mul_relin_rescale_ms": 0.0, "bsgs_ms": 0.0}

    def step(timed=False, overlap=False):
        if overlap:
            main = torch.cuda.current_stream()
            side.wait_stream(main)
            with torch.cuda.stream(side):
                g.mul_tensor_relin(a, b, rlk, out=prod, ws=ws2)
                g.rescale(prod, out=res, ws=ws2)
            g.bsgs_linear_transform(a, diags, BS, GS, baby, giant, do_rescale=True, out=lt, ws=ws)
            main.wait_stream(side)
            return
        if timed:
            ev[0].record()
        g.mul_tensor_relin(a, b, rlk, out=prod, ws=ws)
        g.rescale(prod, out=res, ws=ws)
        if timed:
            ev[1].record()
        g.bsgs_linear_transform(a, diags, BS, GS, baby, giant, do_rescale=True, out=lt, ws=ws)
        if timed:
            ev[2].record()
            ev[2].synchronize()
            parts["mul_relin_rescale_ms"] += ev[0].elapsed_time(ev[1])
            parts["bsgs_ms"] += ev[1].elapsed_time(ev[2])

    overlap = not args.no_overlap
    for _ in range(args.warmup):
        step(overlap=overlap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(overlap=overlap)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el / args.steps * 1e3
    ks_per_step = BATCH + BATCH * (BS + GS - 2)

    # split of the step (separate pass, event-bracketed); also each step's own time
    nsplit, step_times = 5, []
    for _ in range(nsplit):
        before = parts["mul_relin_rescale_ms"] + parts["bsgs_ms"]
        step(timed=True)
        step_times.append(parts["mul_relin_rescale_ms"] + parts["bsgs_ms"] - before)
    mr_ms, bsgs_ms = parts["mul_relin_rescale_ms"] / nsplit, parts["bsgs_ms"] / nsplit
    step_times.sort()
    # the products alone, 10 back to back between two events: a 0.3 ms segment right after a host
    # synchronisation (as in the split above) also holds the host's launch latency.  Left out of
    # --step-only runs, whose per-launch counter averages must keep the step's own launch mix.
    prod_ms = mr_ms
    if not args.step_only:
        nprod = 10
        ev[0].record()
        for _ in range(nprod):
            g.mul_tensor_relin(a, b, rlk, out=prod, ws=ws)
            g.rescale(prod, out=res, ws=ws)
        ev[1].record()
        ev[1].synchronize()
        prod_ms = ev[0].elapsed_time(ev[1]) / nprod

    # standalone batched NTT throughput on the same [8][2][112] limbs
    x = a.clone().view(BATCH * 2, L, N)
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.ntt_fwd(x)
    g.ntt_inv(x)
    e0.record()
    for _ in range(reps):
        g.ntt_fwd(x)
        g.ntt_inv(x)
    e1.record()
    torch.cuda.synchronize()
    ntt_ms = e0.elapsed_time(e1) / (2 * reps)
    limbs = BATCH * 2 * L
    ntt_rate = limbs / (ntt_ms * 1e-3)

    # per-kernel launch times (library event profiler) over profiled steps + the NTT pair, taken
    # right after the timed steps, before the other legs load the GPU for seconds
    g.profile_begin()
    for _ in range(args.profile_steps):
        step()
    g.ntt_fwd(x)
    g.ntt_inv(x)
    prof = g.profile_end()

    # forward-NTT batch sweep at the 4-prime shape of the standalone NTT workload (the chain's
    # first 4 primes): polynomials x 4 limbs, to show where the launch saturates the chip
    sweep = []
    for polys in (() if args.step_only else (1, 4, 16, 64, 256, 1024, 4096)):
        y = torch.empty((polys, 4, N), dtype=u64, device=dev)
        g.fill_uniform(y.view(polys, 4, N), 0xC0DE0001, synth.TAG_CT, 0)
        g.ntt_fwd(y)
        r = max(5, min(200, 20000 // polys))
        e0.record()
        for _ in range(r):
            g.ntt_fwd(y)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / r * 1e3
        sweep.append({"polys": polys, "limbs": 4 * polys, "us_per_launch": us,
                      "limb_ntts_per_s": 4 * polys / (us * 1e-6),
                      "algo_GBps": 4 * polys * 2 * LIMB / (us * 1e-6) / 1e9})
        del y

    # pointwise product (an HBM-bound step on its own): [8][2][112] limbs, 2 read + 1 written
    pointwise = None
    pw = torch.empty_like(x) if not args.step_only else None
    if pw is not None:
        g.pointwise_mul(x, x, out=pw)
        e0.record()
        for _ in range(reps):
            g.pointwise_mul(x, x, out=pw)
        e1.record()
        torch.cuda.synchronize()
        pw_us = e0.elapsed_time(e1) / reps * 1e3
        pw_gbs = 3 * limbs * LIMB / (pw_us * 1e-6) / 1e9
        pointwise = {"limbs": limbs, "us_per_launch": pw_us, "algo_GBps": pw_gbs,
                     "frac_of_8TBps": pw_gbs / HBM_PEAK_GBS,
                     "work": "a * b mod q elementwise: 2 limbs read + 1 written per limb"}
        del pw

    # EvalMod (bootstrapping's modular reduction, outside the step): batch 8 at
    # the 112-prime level, degree-31 cosine interpolant on [-8, 8], 3 double angles
    em = boot = seeded = ring = c4 = None
    if not args.step_only:
        em = eval_mod_timing(g, a, rlk, torch)
        # seed-expanded switching keys: rotation with the key's a rows regenerated in the kernel
        seeded = seeded_key_timing(g, torch, a, keys[0])
        # bootstrapping of 8 ciphertexts on this 112-prime chain (1 -> 112 -> 95 primes; slot_to_coeff's
        # diagonals at 96 primes) with the step's rotation keys and a second diagonal set
        stc = torch.empty((GS, BS, boot_stc_level(L), N), dtype=u64, device=dev)
        g.fill_uniform(stc, 0xC0DE0005, synth.TAG_DIAG, 0)
        boot = bootstrap_timing(g, torch, L, 1, diags, stc, baby, giant, keys[0], rlk, 2, 0xC0DE0006)
        del stc
        ring = ring65536_timing(torch)
    if not args.step_only and not args.no_c4:
        del x
        torch.cuda.empty_cache()
        c4 = c4_timing(torch)

    work = kernel_work()
    kernels = {}
    sq_valid = csrc_sha() == MEASURED_SQ["source_sha"]
    for name, (cnt, tot, mn, mx) in prof.items():
        avg = tot / cnt
        w = work.get(name, {})
        per_step = tot / (1 if w.get("standalone") else args.profile_steps)  # ms of this kernel per step
        row = {"launches": cnt, "avg_us": avg * 1e3, "total_ms_per_step": per_step}
        if "bytes" in w:
            row["algo_GBps"] = w["bytes"] / (per_step * 1e-3) / 1e9
        if "mads" in w:
            row["algo_Tmads"] = w["mads"] / (per_step * 1e-3) / 1e12
        if "products" in w:
            row["algo_Tproducts"] = w["products"] / (per_step * 1e-3) / 1e12
            row["algo_int8_TOPs"] = row["algo_Tproducts"] * I8_OPS_PER_PRODUCT
        if sq_valid and name in MEASURED_SQ["valu_per_launch"]:
            # counted VALU instructions per launch over this run's mean launch time
            row["valu_issue"] = MEASURED_SQ["valu_per_launch"][name] / (avg * 1e-3) / 1e9 / VALU_ISSUE_PEAK_G
        kernels[name] = row
    for name in ("ntt_fwd", "ntt_inv"):
        if name in kernels:
            kernels[name]["total_ms_per_step"] = 0.0  # standalone call, not part of the step
    step_kernels = {k: v for k, v in kernels.items() if k not in ("ntt_fwd", "ntt_inv")}
    dom = max(step_kernels, key=lambda k: step_kernels[k]["total_ms_per_step"])
    dw, drow = work.get(dom, {}), kernels[dom]
    if "products" in dw:
        roofline = {"bound": "mfma", "kernel": dom, "achieved": drow["algo_int8_TOPs"], "peak": MFMA_I8_PEAK_TOPS,
                    "unit": "int8 TOP/s", "traffic": None,
                    "work_per_step": f"{dw['products']} 60x60-bit products x {I8_OPS_PER_PRODUCT} int8 ops "
                                     f"in {drow['launches'] // args.profile_steps} launch(es)"}
    elif "mads" in dw:
        roofline = {"bound": "alu", "kernel": dom, "achieved": drow["algo_Tmads"], "peak": VALU_PEAK_TOPS,
                    "unit": "T int32-MAD/s", "traffic": None,
                    "work_per_step": f"{dw['mads']} 32x32-bit multiply-adds (4 per 60x60-bit product) "
                                     f"in {drow['launches'] // args.profile_steps} launch(es)"}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": drow.get("algo_GBps"), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "traffic": None,
                    "work_per_step": f"{dw.get('bytes')} bytes in {drow['launches'] // args.profile_steps} launch(es)"}
    roofline["frac"] = roofline["achieved"] / roofline["peak"] if roofline["achieved"] else None
    roofline["avg_launch_us"] = drow["avg_us"]
    roofline["kernel_ms_per_step"] = drow["total_ms_per_step"]
    sha = csrc_sha()
    traffic_valid = sha == MEASURED_TRAFFIC["source_sha"]
    launches = drow["launches"] // args.profile_steps
    # VALU issue: the counted instructions of the dominant kernel over its live launch time.  When it
    # exceeds the fraction above, the kernel is bound by the vector ALU: reported as such, with the
    # HBM fraction kept beside it.
    if sha == MEASURED_SQ["source_sha"] and dom in MEASURED_SQ["valu_per_launch"]:
        vi = MEASURED_SQ["valu_per_launch"][dom]
        rate = vi / (drow["avg_us"] * 1e-6) / 1e9
        roofline["valu_issue"] = rate / VALU_ISSUE_PEAK_G
        if roofline["frac"] is None or roofline["valu_issue"] > roofline["frac"]:
            roofline["frac_" + roofline["bound"]] = roofline["frac"]
            roofline.update({"bound": "alu", "achieved": rate, "peak": VALU_ISSUE_PEAK_G,
                             "unit": "G VALU wave-instructions/s", "frac": roofline["valu_issue"],
                             "work_per_launch": f"{vi} VALU wave-instructions (rocprofv3 SQ_INSTS_VALU)"})
    if traffic_valid and dom in MEASURED_TRAFFIC["bytes_per_launch"]:
        roofline["traffic"] = MEASURED_TRAFFIC["bytes_per_launch"][dom]
        roofline["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        if "bytes" in dw:
            roofline["traffic_over_algorithmic"] = roofline["traffic"] / (dw["bytes"] / launches)
    ntt_row = kernels.get("ntt_fwd", {})
    ntt_roof = {"bound": "hbm", "kernel": "ntt_fwd [16][112] limbs", "achieved": ntt_row.get("algo_GBps"),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "avg_launch_us": ntt_row.get("avg_us"),
                "work_per_launch": f"{work['ntt_fwd']['bytes']} bytes (each limb read and written once)"}
    if ntt_roof["achieved"]:
        ntt_roof["frac"] = ntt_roof["achieved"] / HBM_PEAK_GBS
    ntt_roof["traffic"] = MEASURED_TRAFFIC["bytes_per_launch"].get("ntt_fwd") if traffic_valid else None
    if sha == MEASURED_SQ["source_sha"] and ntt_row.get("avg_us") and "ntt_fwd" in MEASURED_SQ["valu_per_launch"]:
        ntt_roof["valu_issue"] = (MEASURED_SQ["valu_per_launch"]["ntt_fwd"] / (ntt_row["avg_us"] * 1e-6) / 1e9
                                  / VALU_ISSUE_PEAK_G)

    out = {
        "metric": "limb-NTTs/s + key-switches/s @n=2048,112 primes; % HBM roofline",
        "value": ks_per_step / (ms * 1e-3),
        "unit": "key-switches/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u64",
        "data": "synthetic (seeded SplitMix64 residues, resident in HBM)",
        "config": {"workload": "n=2048, 112+28 primes, dnum=4, batch 8: ct x ct tensor+relin+rescale "
                               "and BSGS 32x32 linear transform + rescale at 112 primes",
                   "global_batch": BATCH, "parallelism": "single GPU",
                   "streams": 1 if args.no_overlap else 2},
        "key_switches_per_step": ks_per_step,
        "key_switch_hbm": {"algorithmic_bytes": KS_BYTES,
                           "GBps": ks_per_step / (ms * 1e-3) * KS_BYTES / 1e9,
                           "frac": ks_per_step / (ms * 1e-3) * KS_BYTES / (HBM_PEAK_GBS * 1e9)},
        "eval_mod": em,
        "bootstrap": boot,
        "seeded_keys": seeded,
        "ring65536": ring,
        "c4": c4,
        "limb_ntts_per_s": ntt_rate,
        "linear_transforms_per_s": BATCH / (bsgs_ms * 1e-3),
        "ct_mults_per_s": BATCH / (prod_ms * 1e-3),
        "ct_mult_ms": prod_ms,
        "step_split_ms": {"mul_relin_rescale": mr_ms, "bsgs": bsgs_ms},
        # the same step with its two parts in order on one stream
        "step_ms_events": {"median": step_times[nsplit // 2], "min": step_times[0], "steps": nsplit,
                           "streams": 1},
        "ntt_sweep": sweep,
        "pointwise": pointwise,
        "roofline": roofline,
        "ntt_roofline": ntt_roof,
        "kernels": kernels,
    }
    if args.calibrate_copy:
        src = torch.empty(1 << 27, dtype=u64, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 2 * src.numel() * 8
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        out["cpu_baseline"]["one_core"] = cpu_baseline_one_core(min(5.0, args.cpu_seconds))
        out["cpu_baseline"]["units"] = cpu_baseline_units(skip_c4=args.no_c4 or args.step_only)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
