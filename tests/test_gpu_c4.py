"""Parity of the bootstrap-scale linear transforms at their real shape: the
2100 -> 2083 prime chain (n = 2048, 263 special primes, dnum 8) of the
Kestrel article's section 5.3 boot profile, BSGS 32 x 32 (its section 4.4
build flags), batch 8, dense seeded diagonals and keys:

  * coeff_to_slot: BSGS + rescale at 2100 primes, then the conjugation key
    switch of the result at 2099 (the input of conj_extract);
  * slot_to_coeff: BSGS + rescale at 2084 primes (-> 2083);
  * a dense 4 x 4 BSGS at 2100 primes, whose three giant steps fall in one
    batch of the GPU's summed giant-step key switch.

Expected values: per-limb digests written by tests/golden/make_c4_digests.py
from the oracle (inputs per tests/golden/c4_recipe.py, drawn here by the
library's fill kernel, which equals the CPU generator).  Ciphertext 0 is
compared on every limb; ciphertext 1 is the negation of ciphertext 0, and
centered rounding makes every step odd (pinned on the CPU), so its output
must be the negation of ciphertext 0's; ciphertexts 2..7 are compared on
every limb where the golden file holds them.
"""
import json
import os
import sys

import numpy as np
import pytest

from gpu_util import gfill, gpu_ctx, host, require_gpu, say, torch
from rns_ckks_polynomial_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import c4_recipe as R  # noqa: E402

pytestmark = pytest.mark.gpu


def golden(case):
    path = os.path.join(HERE, "golden", f"c4_{case}.json")
    if not os.path.exists(path):
        pytest.skip(f"tests/golden/c4_{case}.json not written yet (make_c4_digests.py --case {case})")
    return json.load(open(path))


@pytest.fixture(scope="module")
def ctx():
    require_gpu()
    g = gpu_ctx(R.N, R.L, R.K, R.DNUM)
    g.prepare_levels(R.L_STC, R.L)
    yield g
    g._ws = None  # the 40 GB BSGS workspace the context cached
    torch.cuda.empty_cache()


def key_tensor(g, idx):
    """Keys idx (recipe indices) as one [len][DNUM][2][TOT][N] tensor, drawn by the fill kernel."""
    t = torch.empty((len(idx), R.DNUM, 2, R.TOT, R.N), dtype=torch.uint64, device="cuda")
    for j, k in enumerate(idx):
        g.fill_uniform(t[j], R.SEED_KEYS, synth.TAG_KEY, R.key_streams(k))
    return t


def inputs(g, seed, B, l):
    """[B][2][l][N] seeded ciphertexts with ciphertext 1 replaced by the negation of ciphertext 0."""
    x = gfill(g, (B, 2, l, R.N), seed, synth.TAG_CT)
    q = torch.tensor(g.primes[:l].astype(np.int64), device="cuda").view(1, l, 1)
    x0 = x[0].view(torch.int64)
    x[1].view(torch.int64).copy_(torch.where(x0 == 0, x0, q - x0))
    return x


def negate(ct, primes):
    q = primes[: ct.shape[1]].astype(np.uint64)[None, :, None]
    return np.where(ct == 0, ct, q - ct)


def check(name, got, want, primes):
    """got: host [B][2][l][N]; want: {ct index: [poly digests]}; returns the indices compared."""
    done = []
    for t in range(got.shape[0]):
        if str(t) in want:
            exp = want[str(t)]
        elif t in R.NEGATED and str(R.NEGATED[t]) in want:
            # the expected output is the negation of the source ciphertext's output, itself checked
            src = R.NEGATED[t]
            assert R.limb_digests(got[src]) == want[str(src)], name
            exp = R.limb_digests(negate(got[src], primes))
        else:
            continue
        d = R.limb_digests(got[t])
        for c in range(2):
            bad = [i for i in range(got.shape[2]) if d[c][8 * i: 8 * i + 8] != exp[c][8 * i: 8 * i + 8]]
            assert not bad, f"{name}: ciphertext {t} polynomial {c}: {len(bad)} limbs differ, first {bad[:5]}"
        done.append(t)
    return done


def test_c4_dense_4x4_batch2(ctx):
    g = ctx
    want = golden("small")["ciphertexts"]
    l, bs, gs = R.L, R.SMALL_BS, R.SMALL_GS
    say("c4 dense 4x4: keys, diagonals, inputs")
    keys = key_tensor(g, [R.small_baby_key_index(b) for b in range(1, bs)] +
                      [R.small_giant_key_index(j) for j in range(1, gs)])
    baby = [None] + [keys[b - 1] for b in range(1, bs)]
    giant = [None] + [keys[bs - 2 + j] for j in range(1, gs)]
    pt = gfill(g, (gs, bs, l, R.N), R.SEED_SMALL_DIAG, synth.TAG_DIAG)
    x = inputs(g, R.SEED_SMALL_IN, R.SMALL_BATCH, l)
    say("c4 dense 4x4: GPU")
    out = host(g.bsgs_linear_transform(x, pt, bs, gs, baby, giant, do_rescale=True))
    del keys, pt, x
    assert check("4x4", out, {k: v["bsgs"] for k, v in want.items()}, g.primes) == [0, 1]


@pytest.fixture(scope="module")
def all_keys(ctx):
    say("c4: drawing the 63 switching keys (39 GB)")
    k = key_tensor(ctx, list(range(R.NKEYS)))
    yield k
    del k
    torch.cuda.empty_cache()


def _bsgs32(g, keys, l, seed_diag, seed_in):
    baby = [None] + [keys[R.baby_key_index(b)] for b in range(1, R.BS)]
    giant = [None] + [keys[R.giant_key_index(j)] for j in range(1, R.GS)]
    pt = gfill(g, (R.GS, R.BS, l, R.N), seed_diag, synth.TAG_DIAG)
    x = inputs(g, seed_in, R.BATCH, l)
    say(f"c4 BSGS 32x32 at {l} primes, batch {R.BATCH}: GPU")
    y = g.bsgs_linear_transform(x, pt, R.BS, R.GS, baby, giant, do_rescale=True)
    del pt, x
    torch.cuda.empty_cache()
    return y


def test_c4_coeff_to_slot_batch8(ctx, all_keys):
    g, keys = ctx, all_keys
    want = golden("cts")["ciphertexts"]
    w = _bsgs32(g, keys, R.L_CTS, R.SEED_CTS_DIAG, R.SEED_CTS_IN)
    say("c4 coeff_to_slot: conjugation key switch")
    cj = g.rotate(w, 2 * R.N - 1, keys[R.CONJ_KEY])
    done = check("coeff_to_slot", host(w), {k: v["bsgs"] for k, v in want.items()}, g.primes)
    done_c = check("conj", host(cj), {k: v["conj"] for k, v in want.items()}, g.primes)
    say(f"c4 coeff_to_slot: ciphertexts compared {done}, conjugates {done_c}")
    assert 0 in done and 1 in done and done == done_c


def test_c4_slot_to_coeff_batch8(ctx, all_keys):
    g, keys = ctx, all_keys
    want = golden("stc")["ciphertexts"]
    y = _bsgs32(g, keys, R.L_STC, R.SEED_STC_DIAG, R.SEED_STC_IN)
    done = check("slot_to_coeff", host(y), {k: v["bsgs"] for k, v in want.items()}, g.primes)
    say(f"c4 slot_to_coeff: ciphertexts compared {done}")
    assert 0 in done and 1 in done
