/* Host sanitizer run of the C oracle (oracle/oracle.c): every entry point on
 * a small parameter set, with a few result checks (round trips, a known base
 * conversion).  Built with -fsanitize=address,undefined by
 * tests/test_host_sanitize.py; exits non-zero on a failed check. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

#define N 64
#define L 6
#define K 2
#define DNUM 3
#define TOT (L + K)

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint64_t rnd(uint64_t q) {
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return st % q;
}
static int fails = 0;
#define CHECK(c, msg) do { if (!(c)) { fprintf(stderr, "FAIL: %s\n", msg); fails++; } } while (0)

int main(void) {
    uint64_t primes[TOT], psi[TOT];
    CHECK(or_gen_primes(N, TOT, primes) == 0, "gen_primes");
    for (int i = 0; i < TOT; i++) psi[i] = or_min_psi(N, primes[i]);
    or_params pp = {N, L, K, DNUM, primes, psi};
    uint64_t a[N], b[N], c[N], d[N];
    for (int k = 0; k < N; k++) { a[k] = rnd(primes[0]); b[k] = rnd(primes[0]); }
    memcpy(c, a, sizeof a);
    or_ntt(N, primes[0], psi[0], c);
    or_ntt_definition(N, primes[0], psi[0], a, d);
    CHECK(memcmp(c, d, sizeof c) == 0, "ntt vs definition");
    or_intt(N, primes[0], psi[0], c);
    CHECK(memcmp(c, a, sizeof c) == 0, "ntt round trip");
    or_intt_definition(N, primes[0], psi[0], d, c);
    CHECK(memcmp(c, a, sizeof c) == 0, "definition round trip");
    or_negacyclic_schoolbook(N, primes[0], a, b, c);
    or_automorph_coef(N, primes[0], 5, a, c);
    /* base conversion of the known value -3 from 3 primes to 2 others */
    uint64_t x[3 * N], out[2 * N];
    for (int i = 0; i < 3; i++)
        for (int k = 0; k < N; k++) x[i * N + k] = primes[i] - 3;
    or_base_convert(N, 3, primes, x, 2, primes + 3, out);
    CHECK(out[0] == primes[3] - 3 && out[2 * N - 1] == primes[4] - 3, "base conversion of -3");
    /* ciphertext operations at full level */
    size_t ctw = 2 * (size_t)L * N;
    uint64_t *ct = malloc(ctw * 8), *ct2 = malloc(ctw * 8), *res = malloc(ctw * 8), *res2 = malloc(ctw * 8);
    uint64_t *key = malloc((size_t)DNUM * 2 * TOT * N * 8), *pt = malloc((size_t)4 * L * N * 8);
    uint64_t *dd = malloc(3 * (size_t)L * N * 8);
    for (int c2 = 0; c2 < 2; c2++)
        for (int i = 0; i < L; i++)
            for (int k = 0; k < N; k++) {
                ct[(c2 * L + i) * N + k] = rnd(primes[i]);
                ct2[(c2 * L + i) * N + k] = rnd(primes[i]);
            }
    for (int j = 0; j < DNUM * 2; j++)
        for (int i = 0; i < TOT; i++)
            for (int k = 0; k < N; k++) key[((size_t)j * TOT + i) * N + k] = rnd(primes[i]);
    for (int g = 0; g < 4; g++)
        for (int i = 0; i < L; i++)
            for (int k = 0; k < N; k++) pt[((size_t)g * L + i) * N + k] = rnd(primes[i]);
    or_tensor(&pp, L, ct, ct2, dd);
    or_keyswitch(&pp, L, dd + 2 * L * N, key, res);
    or_mul_tensor_relin(&pp, L, ct, ct2, key, res);
    or_rescale(&pp, L, res, res2);
    or_rotate(&pp, L, 5, ct, key, res);
    or_rotate(&pp, L - 1, 2 * N - 1, ct, key, res);  /* a partial last digit */
    const uint64_t *keys[2] = {NULL, key};
    or_bsgs(&pp, L, ct, pt, 2, 2, keys, keys, 1, res);
    memset(res2, 0, ctw * 8);
    or_mul_acc(&pp, L, pt, ct, res2);
    or_add(&pp, L, 2, res2, res2, res);
    /* encode / encrypt / decrypt */
    double zr[N / 2], zi[N / 2], orr[N / 2], oi[N / 2];
    for (int j = 0; j < N / 2; j++) { zr[j] = (double)j / N; zi[j] = -(double)j / N; }
    int64_t coeffs[N], e[N * DNUM];
    or_encode_coeffs(N, zr, zi, 1099511627776.0, coeffs);
    uint32_t idx[TOT];
    for (int i = 0; i < TOT; i++) idx[i] = i;
    uint64_t *m = malloc((size_t)L * N * 8), *s = malloc((size_t)TOT * N * 8), *ea = malloc((size_t)L * N * 8);
    int64_t sc[N];
    for (int k = 0; k < N; k++) { sc[k] = (int64_t)rnd(3) - 1; e[k] = (int64_t)rnd(7) - 3; }
    for (int k = N; k < N * DNUM; k++) e[k] = (int64_t)rnd(7) - 3;
    or_coeffs_to_ntt(&pp, L, idx, coeffs, m);
    or_coeffs_to_ntt(&pp, TOT, idx, sc, s);
    for (int i = 0; i < L; i++)
        for (int k = 0; k < N; k++) ea[(size_t)i * N + k] = rnd(primes[i]);
    or_keygen_swk(&pp, s, s, key + (size_t)TOT * N, e, key);
    or_encrypt(&pp, L, m, s, ea, e, ct);
    or_decrypt(&pp, L, ct, s, res);
    or_decode(&pp, L, res, 1099511627776.0, orr, oi);
    double err = 0;
    for (int j = 0; j < N / 2; j++) {
        double d1 = orr[j] - zr[j], d2 = oi[j] - zi[j];
        if (d1 < 0) d1 = -d1;
        if (d2 < 0) d2 = -d2;
        if (d1 > err) err = d1;
        if (d2 > err) err = d2;
    }
    CHECK(err < 1e-6, "encrypt / decrypt");
    free(ct); free(ct2); free(res); free(res2); free(key); free(pt); free(dd); free(m); free(s); free(ea);
    printf("oracle under sanitizers: %s\n", fails ? "FAILED" : "ok");
    return fails ? 1 : 0;
}
