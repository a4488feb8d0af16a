#!/usr/bin/env python3
"""Benchmark of the RNS-CKKS hot path on one MI355X.

Workload (n = 2048, 112 main primes + 28 special primes, dnum = 4, batch of
8 ciphertexts, all inputs seeded and resident in HBM before timing):
  one step = ct x ct tensor + relinearise + rescale on 8 pairs
           + BSGS 32 x 32 plaintext-matrix x ciphertext (1024 diagonals,
             31 baby + 31 giant rotations per ciphertext) + rescale on 8 cts.
That is 8 + 8 * 62 = 504 key switches per step, plus every other step of the
path (NTT/iNTT, tensor, Galois automorphisms, base conversion, rescale, MAC).

Prints one JSON line.  `value` = key switches per second over the whole step.
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
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    return p.parse_args()


def cpu_baseline(budget_s: float):
    """The oracle as it stands, timed on this host: key switches at the same
    shape (relinearisation of ct x ct at 112 primes), repeated until the budget."""
    import numpy as np

    import oracle
    from rns_ckks_polynomial_amd import synth
    o = oracle.Ctx(N, L, K, DNUM)
    mods = np.tile(o.primes[:L], 2)
    a = synth.uniform_mod(1, synth.TAG_CT, np.arange(2 * L), mods, N).reshape(2, L, N)
    b = synth.uniform_mod(2, synth.TAG_CT, np.arange(2 * L), mods, N).reshape(2, L, N)
    key = synth.uniform_mod(3, synth.TAG_KEY, np.arange(DNUM * 2 * (L + K)), np.tile(o.primes, DNUM * 2),
                            N).reshape(DNUM, 2, L + K, N)
    done, t0 = 0, time.perf_counter()
    while True:
        o.mul_tensor_relin(a, b, key, L)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 64:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": done / el, "unit": "key-switches/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} x (tensor + relinearise) of one ciphertext pair at n=2048, 112+28 primes, "
                      f"dnum=4 ({el:.1f} s, OpenMP over coefficients/limbs)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
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

    def step():
        g.mul_tensor_relin(a, b, rlk, out=prod, ws=ws)
        g.rescale(prod, out=res, ws=ws)
        g.bsgs_linear_transform(a, diags, BS, GS, baby, giant, do_rescale=True, out=lt, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el / args.steps * 1e3
    ks_per_step = BATCH + BATCH * (BS + GS - 2)

    # standalone limb-NTT throughput on the same batch (forward + inverse of [8][2][112] limbs)
    x = a.clone().view(BATCH * 2, L, N)
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.ntt_fwd(x); g.ntt_inv(x)
    e0.record()
    for _ in range(reps):
        g.ntt_fwd(x)
        g.ntt_inv(x)
    e1.record()
    torch.cuda.synchronize()
    ntt_ms = e0.elapsed_time(e1) / (2 * reps)
    limbs = BATCH * 2 * L
    ntt_rate = limbs / (ntt_ms * 1e-3)
    ntt_bytes = limbs * N * 8 * 2  # read + write each limb once
    roofline = {"bound": "hbm", "kernel": "k_ntt2048 (fwd, [16][112] limbs)", "achieved": ntt_bytes / (ntt_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None}
    roofline["frac"] = roofline["achieved"] / roofline["peak"]

    out = {
        "metric": "limb-NTTs/s + key-switches/s @n=2048,112 primes; % HBM roofline",
        "value": ks_per_step / (ms * 1e-3),
        "unit": "key-switches/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u64 (exact 60-bit RNS)",
        "data": "synthetic (seeded SplitMix64 residues, resident in HBM)",
        "config": {"workload": "config 2 + config 3 shapes: n=2048, 112+28 primes, dnum=4, batch 8; "
                               "ct x ct tensor+relin+rescale and BSGS 32x32 linear transform + rescale",
                   "global_batch": BATCH, "parallelism": "single GPU"},
        "key_switches_per_step": ks_per_step,
        "limb_ntts_per_s": ntt_rate,
        "linear_transforms_per_s": None,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
