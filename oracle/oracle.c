/*
 * oracle.c -- plain CPU reference of the RNS-CKKS hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Written for obviousness, not
 * speed: every modular product is an exact 128-bit product reduced with `%`,
 * base conversion reconstructs the CRT integer as a multi-word bigint, the
 * automorphism goes through the coefficient domain with the direct index
 * map.  OpenMP only splits independent coefficients / limbs; results do not
 * depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

/* ======================================================================
 * Scalar arithmetic
 * ====================================================================== */
uint64_t or_mulmod(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)(((u128)a * b) % q); }

static uint64_t addmod(uint64_t a, uint64_t b, uint64_t q) {
    uint64_t s = a + b; /* a, b < q < 2^63: no overflow */
    return s >= q ? s - q : s;
}
static uint64_t submod(uint64_t a, uint64_t b, uint64_t q) { return a >= b ? a - b : a + q - b; }

uint64_t or_powmod(uint64_t a, uint64_t e, uint64_t q) {
    uint64_t r = 1 % q;
    a %= q;
    while (e) {
        if (e & 1) r = or_mulmod(r, a, q);
        a = or_mulmod(a, a, q);
        e >>= 1;
    }
    return r;
}

/* inverse modulo a prime, by Fermat's little theorem */
uint64_t or_invmod(uint64_t a, uint64_t q) { return or_powmod(a, q - 2, q); }

/* reduce a signed integer into [0, q) */
static uint64_t from_signed(int64_t v, uint64_t q) {
    if (v >= 0) return (uint64_t)v % q;
    uint64_t m = (uint64_t)(-(v + 1)) + 1; /* |v| without overflow */
    m %= q;
    return m ? q - m : 0;
}

/* Deterministic Miller-Rabin: bases 2..37 decide every 64-bit integer. */
int or_is_prime(uint64_t x) {
    static const uint64_t bases[12] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
    if (x < 2) return 0;
    for (int i = 0; i < 12; i++) {
        if (x == bases[i]) return 1;
        if (x % bases[i] == 0) return 0;
    }
    uint64_t d = x - 1;
    int s = 0;
    while ((d & 1) == 0) { d >>= 1; s++; }
    for (int i = 0; i < 12; i++) {
        uint64_t y = or_powmod(bases[i], d, x);
        if (y == 1 || y == x - 1) continue;
        int comp = 1;
        for (int r = 1; r < s; r++) {
            y = or_mulmod(y, y, x);
            if (y == x - 1) { comp = 0; break; }
        }
        if (comp) return 0;
    }
    return 1;
}

/* The chain rule: 60-bit primes q = 1 (mod 2n), taken in ascending order from
 * 2^59 upward (one prime per rescale: Kestrel article, "wall 2"; 60-bit
 * primes, 112 / 2100 of them: relay README section 1, article section 4.1). */
int or_gen_primes(uint32_t n, uint32_t count, uint64_t *out) {
    const uint64_t lo = 1ULL << 59, hi = 1ULL << 60, step = 2ULL * n;
    uint32_t got = 0;
    for (uint64_t c = lo + 1; c < hi && got < count; c += step)
        if (or_is_prime(c)) out[got++] = c;
    return got == count ? 0 : -1;
}

/* Smallest primitive 2n-th root of unity: find any element of order exactly
 * 2n (n a power of two, so w^n = -1 suffices), then take the least of its odd
 * powers, which are exactly all primitive 2n-th roots. */
uint64_t or_min_psi(uint32_t n, uint64_t q) {
    uint64_t m = 2ULL * n, w = 0;
    for (uint64_t x = 2; x < q; x++) {
        w = or_powmod(x, (q - 1) / m, q);
        if (or_powmod(w, n, q) == q - 1) break;
    }
    uint64_t w2 = or_mulmod(w, w, q), cur = w, best = w;
    for (uint64_t k = 1; k < m; k += 2) {
        if (cur < best) best = cur;
        cur = or_mulmod(cur, w2, q);
    }
    return best;
}

/* ======================================================================
 * Single-limb transforms
 * ====================================================================== */
/* A_j = sum_i a_i psi^(i(2j+1)) */
void or_ntt_definition(uint32_t n, uint64_t q, uint64_t psi, const uint64_t *a, uint64_t *out) {
    for (uint32_t j = 0; j < n; j++) {
        uint64_t x = or_powmod(psi, 2ULL * j + 1, q), p = 1, acc = 0;
        for (uint32_t i = 0; i < n; i++) {
            acc = addmod(acc, or_mulmod(a[i], p, q), q);
            p = or_mulmod(p, x, q);
        }
        out[j] = acc;
    }
}

/* a_i = n^-1 sum_j A_j psi^(-i(2j+1)) */
void or_intt_definition(uint32_t n, uint64_t q, uint64_t psi, const uint64_t *A, uint64_t *out) {
    uint64_t psi_inv = or_invmod(psi, q), n_inv = or_invmod(n, q);
    for (uint32_t i = 0; i < n; i++) {
        uint64_t x = or_powmod(psi_inv, i, q), x2 = or_mulmod(x, x, q), p = x, acc = 0;
        for (uint32_t j = 0; j < n; j++) { /* p = psi^(-i(2j+1)) */
            acc = addmod(acc, or_mulmod(A[j], p, q), q);
            p = or_mulmod(p, x2, q);
        }
        out[i] = or_mulmod(acc, n_inv, q);
    }
}

static uint32_t bitrev(uint32_t x, int bits) {
    uint32_t r = 0;
    for (int i = 0; i < bits; i++) { r = (r << 1) | (x & 1); x >>= 1; }
    return r;
}

/* Textbook iterative radix-2 cyclic transform A_j = sum_i b_i w^(ij), natural order. */
static void cyclic_ntt(uint32_t n, uint64_t q, uint64_t w, uint64_t *b) {
    int bits = 0;
    while ((1u << bits) < n) bits++;
    for (uint32_t i = 0; i < n; i++) {
        uint32_t r = bitrev(i, bits);
        if (r > i) { uint64_t t = b[i]; b[i] = b[r]; b[r] = t; }
    }
    for (uint32_t len = 2; len <= n; len <<= 1) {
        uint64_t wlen = or_powmod(w, n / len, q);
        for (uint32_t i = 0; i < n; i += len) {
            uint64_t wk = 1;
            for (uint32_t j = 0; j < len / 2; j++) {
                uint64_t u = b[i + j], v = or_mulmod(b[i + j + len / 2], wk, q);
                b[i + j] = addmod(u, v, q);
                b[i + j + len / 2] = submod(u, v, q);
                wk = or_mulmod(wk, wlen, q);
            }
        }
    }
}

/* Negacyclic NTT = twist by psi^i, then cyclic NTT with w = psi^2. */
void or_ntt(uint32_t n, uint64_t q, uint64_t psi, uint64_t *a) {
    uint64_t p = 1;
    for (uint32_t i = 0; i < n; i++) { a[i] = or_mulmod(a[i], p, q); p = or_mulmod(p, psi, q); }
    cyclic_ntt(n, q, or_mulmod(psi, psi, q), a);
}

void or_intt(uint32_t n, uint64_t q, uint64_t psi, uint64_t *a) {
    uint64_t psi_inv = or_invmod(psi, q);
    cyclic_ntt(n, q, or_mulmod(psi_inv, psi_inv, q), a);
    uint64_t p = or_invmod(n, q);
    for (uint32_t i = 0; i < n; i++) { a[i] = or_mulmod(a[i], p, q); p = or_mulmod(p, psi_inv, q); }
}

void or_negacyclic_schoolbook(uint32_t n, uint64_t q, const uint64_t *a, const uint64_t *b, uint64_t *out) {
    memset(out, 0, sizeof(uint64_t) * n);
    for (uint32_t i = 0; i < n; i++)
        for (uint32_t j = 0; j < n; j++) {
            uint64_t p = or_mulmod(a[i], b[j], q);
            uint32_t k = i + j;
            if (k < n) out[k] = addmod(out[k], p, q);
            else out[k - n] = submod(out[k - n], p, q); /* X^n = -1 */
        }
}

/* a(X) -> a(X^g): coefficient i moves to i*g mod 2n; X^(n+r) = -X^r. */
void or_automorph_coef(uint32_t n, uint64_t q, uint64_t g, const uint64_t *in, uint64_t *out) {
    uint64_t m = 2ULL * n;
    for (uint32_t i = 0; i < n; i++) {
        uint64_t e = ((uint64_t)i * (g % m)) % m;
        if (e < n) out[e] = in[i];
        else out[e - n] = in[i] ? q - in[i] : 0;
    }
}

/* ======================================================================
 * Bigints (little-endian 64-bit words, fixed width w) for exact CRT
 * ====================================================================== */
/* r[0..w) = a[0..w) * m  (no overflow beyond w words assumed by caller) */
static void big_mul_word(uint64_t *r, const uint64_t *a, uint64_t m, int w) {
    u128 carry = 0;
    for (int i = 0; i < w; i++) {
        u128 t = (u128)a[i] * m + carry;
        r[i] = (uint64_t)t;
        carry = t >> 64;
    }
}
/* r += a * m */
static void big_addmul_word(uint64_t *r, const uint64_t *a, uint64_t m, int w) {
    u128 carry = 0;
    for (int i = 0; i < w; i++) {
        u128 t = (u128)a[i] * m + r[i] + carry;
        r[i] = (uint64_t)t;
        carry = t >> 64;
    }
}
static int big_cmp(const uint64_t *a, const uint64_t *b, int w) {
    for (int i = w - 1; i >= 0; i--)
        if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
    return 0;
}
static void big_sub(uint64_t *a, const uint64_t *b, int w) { /* a -= b, a >= b */
    uint64_t borrow = 0;
    for (int i = 0; i < w; i++) {
        uint64_t bi = b[i] + borrow;
        uint64_t nb = (bi < borrow) || (a[i] < bi);
        a[i] -= bi;
        borrow = nb;
    }
}
/* a mod t by Horner over the words */
static uint64_t big_mod_word(const uint64_t *a, uint64_t t, int w) {
    u128 r = 0;
    for (int i = w - 1; i >= 0; i--) r = ((r << 64) | a[i]) % t;
    return (uint64_t)r;
}

/* Precomputed CRT data for a basis b[0..nb): B, Bhat_i = B / b_i, [Bhat_i^-1]_{b_i}. */
typedef struct {
    int w;           /* words per bigint */
    uint64_t *B;     /* [w]      */
    uint64_t *Bhat;  /* [nb][w]  */
    uint64_t *inv;   /* [nb]     */
} crt_basis;

static void crt_init(crt_basis *c, uint32_t nb, const uint64_t *b) {
    c->w = (int)nb + 2; /* nb 60-bit factors need < nb words; 2 spare for sums */
    c->B = calloc(c->w, sizeof(uint64_t));
    c->Bhat = calloc((size_t)nb * c->w, sizeof(uint64_t));
    c->inv = malloc(sizeof(uint64_t) * nb);
    uint64_t *tmp = calloc(c->w, sizeof(uint64_t));
    c->B[0] = 1;
    for (uint32_t i = 0; i < nb; i++) { big_mul_word(tmp, c->B, b[i], c->w); memcpy(c->B, tmp, sizeof(uint64_t) * c->w); }
    for (uint32_t i = 0; i < nb; i++) {
        uint64_t *h = c->Bhat + (size_t)i * c->w;
        h[0] = 1;
        for (uint32_t k = 0; k < nb; k++) {
            if (k == i) continue;
            big_mul_word(tmp, h, b[k], c->w);
            memcpy(h, tmp, sizeof(uint64_t) * c->w);
        }
        c->inv[i] = or_invmod(big_mod_word(h, b[i], c->w), b[i]);
    }
    free(tmp);
}
static void crt_free(crt_basis *c) { free(c->B); free(c->Bhat); free(c->inv); }

/* Centered CRT reconstruction of residues x_i (mod b_i): returns the
 * magnitude in mag[0..w) and the sign (1 if negative). */
static int crt_centered(const crt_basis *c, uint32_t nb, const uint64_t *b, const uint64_t *xi,
                        uint64_t *mag, uint64_t *scratch) {
    int w = c->w;
    memset(mag, 0, sizeof(uint64_t) * w);
    /* X = sum_i [x_i Bhat_i^-1]_{b_i} Bhat_i  (< nb * B) */
    for (uint32_t i = 0; i < nb; i++)
        big_addmul_word(mag, c->Bhat + (size_t)i * w, or_mulmod(xi[i], c->inv[i], b[i]), w);
    while (big_cmp(mag, c->B, w) >= 0) big_sub(mag, c->B, w); /* X mod B */
    /* negative representative iff X > (B-1)/2, i.e. 2X > B (B is odd) */
    memcpy(scratch, mag, sizeof(uint64_t) * w);
    big_mul_word(scratch, mag, 2, w);
    if (big_cmp(scratch, c->B, w) > 0) {
        memcpy(scratch, c->B, sizeof(uint64_t) * w);
        big_sub(scratch, mag, w); /* |X - B| = B - X */
        memcpy(mag, scratch, sizeof(uint64_t) * w);
        return 1;
    }
    return 0;
}

void or_base_convert(uint32_t n, uint32_t nb, const uint64_t *b, const uint64_t *x,
                     uint32_t nt, const uint64_t *t, uint64_t *out) {
    crt_basis c;
    crt_init(&c, nb, b);
#pragma omp parallel
    {
        uint64_t *mag = malloc(sizeof(uint64_t) * c.w), *scr = malloc(sizeof(uint64_t) * c.w);
        uint64_t *xi = malloc(sizeof(uint64_t) * nb);
#pragma omp for schedule(static)
        for (uint32_t k = 0; k < n; k++) {
            for (uint32_t i = 0; i < nb; i++) xi[i] = x[(size_t)i * n + k];
            int neg = crt_centered(&c, nb, b, xi, mag, scr);
            for (uint32_t j = 0; j < nt; j++) {
                uint64_t r = big_mod_word(mag, t[j], c.w);
                out[(size_t)j * n + k] = (neg && r) ? t[j] - r : r;
            }
        }
        free(mag); free(scr); free(xi);
    }
    crt_free(&c);
}

/* ======================================================================
 * CKKS operations
 * ====================================================================== */
uint32_t or_alpha(const or_params *pp) { return (pp->L + pp->dnum - 1) / pp->dnum; }
uint32_t or_beta(const or_params *pp, uint32_t l) { uint32_t a = or_alpha(pp); return (l + a - 1) / a; }

static uint64_t *alloc_limbs(size_t limbs, uint32_t n) { return calloc(limbs * n, sizeof(uint64_t)); }

/* forward / inverse NTT of limbs whose primes are given by index list */
static void ntt_limbs(const or_params *pp, uint32_t nl, const uint32_t *idx, uint64_t *x, int inverse) {
#pragma omp parallel for schedule(dynamic)
    for (uint32_t r = 0; r < nl; r++) {
        uint64_t *a = x + (size_t)r * pp->n;
        if (inverse) or_intt(pp->n, pp->primes[idx[r]], pp->psi[idx[r]], a);
        else or_ntt(pp->n, pp->primes[idx[r]], pp->psi[idx[r]], a);
    }
}

void or_tensor(const or_params *pp, uint32_t l, const uint64_t *a, const uint64_t *b, uint64_t *d) {
    size_t ln = (size_t)l * pp->n;
    const uint64_t *a0 = a, *a1 = a + ln, *b0 = b, *b1 = b + ln;
    for (uint32_t i = 0; i < l; i++) {
        uint64_t q = pp->primes[i];
        for (uint32_t k = 0; k < pp->n; k++) {
            size_t o = (size_t)i * pp->n + k;
            d[o] = or_mulmod(a0[o], b0[o], q);
            d[ln + o] = addmod(or_mulmod(a0[o], b1[o], q), or_mulmod(a1[o], b0[o], q), q);
            d[2 * ln + o] = or_mulmod(a1[o], b1[o], q);
        }
    }
}

/* Hybrid key switching (the Galois-key / relinearisation machinery behind
 * ckks_gk_gen and matmul2 in the Kestrel article's technique table):
 *   1. bring d to the coefficient domain;
 *   2. per digit j (primes [j*alpha, min((j+1)*alpha, l))), lift the digit
 *      exactly (centered CRT) to every prime of Q_l u P and return to NTT form;
 *   3. inner product with the key rows (b_j, a_j);
 *   4. ModDown: subtract the centered CRT lift of acc mod P and divide by P. */
void or_keyswitch(const or_params *pp, uint32_t l, const uint64_t *d, const uint64_t *key, uint64_t *out) {
    const uint32_t n = pp->n, L = pp->L, K = pp->K, alpha = or_alpha(pp), beta = or_beta(pp, l);
    const uint32_t ext = l + K; /* extended basis Q_l u P */
    /* prime index of extended limb r */
    uint32_t *eidx = malloc(sizeof(uint32_t) * ext);
    uint64_t *emod = malloc(sizeof(uint64_t) * ext);
    for (uint32_t r = 0; r < ext; r++) { eidx[r] = r < l ? r : L + (r - l); emod[r] = pp->primes[eidx[r]]; }

    uint64_t *dcoef = alloc_limbs(l, n);
    memcpy(dcoef, d, sizeof(uint64_t) * l * n);
    ntt_limbs(pp, l, eidx, dcoef, 1);

    uint64_t *acc = alloc_limbs(2 * (size_t)ext, n); /* [2][ext][n], zero */
    uint64_t *dt = alloc_limbs(ext, n);
    uint64_t *tgt = malloc(sizeof(uint64_t) * ext);
    uint32_t *tidx = malloc(sizeof(uint32_t) * ext);
    for (uint32_t j = 0; j < beta; j++) {
        uint32_t lo = j * alpha, hi = (j + 1) * alpha < l ? (j + 1) * alpha : l, nb = hi - lo;
        /* targets: every extended prime outside the digit */
        uint32_t nt = 0;
        for (uint32_t r = 0; r < ext; r++)
            if (r < lo || r >= hi) { tidx[nt] = r; tgt[nt] = emod[r]; nt++; }
        uint64_t *conv = alloc_limbs(nt, n);
        or_base_convert(n, nb, emod + lo, dcoef + (size_t)lo * n, nt, tgt, conv);
        for (uint32_t r = lo; r < hi; r++) memcpy(dt + (size_t)r * n, dcoef + (size_t)r * n, sizeof(uint64_t) * n);
        for (uint32_t s = 0; s < nt; s++) memcpy(dt + (size_t)tidx[s] * n, conv + (size_t)s * n, sizeof(uint64_t) * n);
        free(conv);
        ntt_limbs(pp, ext, eidx, dt, 0);
        /* key rows of digit j: [2][L+K][n] */
        const uint64_t *kb = key + (size_t)j * 2 * (L + K) * n, *ka = kb + (size_t)(L + K) * n;
        for (uint32_t r = 0; r < ext; r++) {
            uint64_t q = emod[r];
            const uint64_t *x = dt + (size_t)r * n, *brow = kb + (size_t)eidx[r] * n, *arow = ka + (size_t)eidx[r] * n;
            uint64_t *o0 = acc + (size_t)r * n, *o1 = acc + (size_t)(ext + r) * n;
            for (uint32_t k = 0; k < n; k++) {
                o0[k] = addmod(o0[k], or_mulmod(x[k], brow[k], q), q);
                o1[k] = addmod(o1[k], or_mulmod(x[k], arow[k], q), q);
            }
        }
    }
    free(dt); free(tgt); free(tidx);

    /* ModDown of both accumulators */
    uint64_t *pmod = emod + l;
    uint32_t *pidx = eidx + l;
    for (uint32_t c = 0; c < 2; c++) {
        uint64_t *accc = acc + (size_t)c * ext * n;
        uint64_t *pc = alloc_limbs(K, n), *conv = alloc_limbs(l, n);
        memcpy(pc, accc + (size_t)l * n, sizeof(uint64_t) * K * n);
        ntt_limbs(pp, K, pidx, pc, 1);
        or_base_convert(n, K, pmod, pc, l, emod, conv);
        ntt_limbs(pp, l, eidx, conv, 0);
        for (uint32_t i = 0; i < l; i++) {
            uint64_t q = emod[i], Pq = 1;
            for (uint32_t k = 0; k < K; k++) Pq = or_mulmod(Pq, pmod[k] % q, q);
            uint64_t Pinv = or_invmod(Pq, q);
            for (uint32_t k = 0; k < n; k++) {
                size_t o = (size_t)i * n + k;
                out[(size_t)c * l * n + o] = or_mulmod(submod(accc[o], conv[o], q), Pinv, q);
            }
        }
        free(pc); free(conv);
    }
    free(acc); free(dcoef); free(eidx); free(emod);
}

void or_mul_tensor_relin(const or_params *pp, uint32_t l, const uint64_t *a, const uint64_t *b,
                         const uint64_t *rlk, uint64_t *out) {
    size_t ln = (size_t)l * pp->n;
    uint64_t *d = alloc_limbs(3 * (size_t)l, pp->n), *ks = alloc_limbs(2 * (size_t)l, pp->n);
    or_tensor(pp, l, a, b, d);
    or_keyswitch(pp, l, d + 2 * ln, rlk, ks);
    for (uint32_t c = 0; c < 2; c++)
        for (uint32_t i = 0; i < l; i++)
            for (uint32_t k = 0; k < pp->n; k++) {
                size_t o = (size_t)i * pp->n + k;
                out[c * ln + o] = addmod(d[c * ln + o], ks[c * ln + o], pp->primes[i]);
            }
    free(d); free(ks);
}

/* Rescale (Kestrel article, wall 2: every rescale uses up one prime of the chain):
 * out = round(c / q_{l-1}) = (c - [c]_{q_{l-1}, centered}) * q_{l-1}^-1. */
void or_rescale(const or_params *pp, uint32_t l, const uint64_t *in, uint64_t *out) {
    const uint32_t n = pp->n;
    const uint64_t ql = pp->primes[l - 1];
    uint64_t *t = malloc(sizeof(uint64_t) * n), *r = malloc(sizeof(uint64_t) * n);
    for (uint32_t c = 0; c < 2; c++) {
        const uint64_t *ci = in + (size_t)c * l * n;
        memcpy(t, ci + (size_t)(l - 1) * n, sizeof(uint64_t) * n);
        or_intt(n, ql, pp->psi[l - 1], t);
        for (uint32_t i = 0; i + 1 < l; i++) {
            uint64_t q = pp->primes[i], inv = or_invmod(ql % q, q);
            for (uint32_t k = 0; k < n; k++) /* centered value of t mod q */
                r[k] = (t[k] > (ql - 1) / 2) ? submod(t[k] % q, ql % q, q) : t[k] % q;
            or_ntt(n, q, pp->psi[i], r);
            for (uint32_t k = 0; k < n; k++) {
                size_t o = (size_t)i * n + k;
                out[(size_t)c * (l - 1) * n + o] = or_mulmod(submod(ci[o], r[k], q), inv, q);
            }
        }
    }
    free(t); free(r);
}

void or_automorph(const or_params *pp, uint32_t l, uint64_t g, const uint64_t *in, uint64_t *out) {
    const uint32_t n = pp->n;
    uint64_t *t = malloc(sizeof(uint64_t) * n);
    for (uint32_t i = 0; i < l; i++) {
        memcpy(t, in + (size_t)i * n, sizeof(uint64_t) * n);
        or_intt(n, pp->primes[i], pp->psi[i], t);
        or_automorph_coef(n, pp->primes[i], g, t, out + (size_t)i * n);
        or_ntt(n, pp->primes[i], pp->psi[i], out + (size_t)i * n);
    }
    free(t);
}

void or_rotate(const or_params *pp, uint32_t l, uint64_t g, const uint64_t *in, const uint64_t *key,
               uint64_t *out) {
    size_t ln = (size_t)l * pp->n;
    uint64_t *d = alloc_limbs(l, pp->n), *ks = alloc_limbs(2 * (size_t)l, pp->n);
    or_automorph(pp, l, g, in, out);        /* sigma_g(c0) */
    or_automorph(pp, l, g, in + ln, d);     /* sigma_g(c1) */
    or_keyswitch(pp, l, d, key, ks);
    for (uint32_t i = 0; i < l; i++)
        for (uint32_t k = 0; k < pp->n; k++) {
            size_t o = (size_t)i * pp->n + k;
            out[o] = addmod(out[o], ks[o], pp->primes[i]);
            out[ln + o] = ks[ln + o];
        }
    free(d); free(ks);
}

static uint64_t galois_rot(uint32_t n, uint64_t k) { return or_powmod(5, k, 2ULL * n); }

/* Baby-step giant-step diagonal method (matmul2 with BB x GG in the Kestrel
 * article, section 3 and section 4.4 build flags): Bs - 1 baby rotations and
 * G - 1 giant rotations replace Bs * G rotations. */
void or_bsgs(const or_params *pp, uint32_t l, const uint64_t *in, const uint64_t *pt,
             uint32_t Bs, uint32_t G, const uint64_t *const *baby_keys,
             const uint64_t *const *giant_keys, int do_rescale, uint64_t *out) {
    const uint32_t n = pp->n;
    const size_t ln = (size_t)l * n, ctw = 2 * ln;
    uint64_t *rot = alloc_limbs((size_t)Bs * 2 * l, n);
    for (uint32_t b = 0; b < Bs; b++) {
        if (b == 0) memcpy(rot, in, sizeof(uint64_t) * ctw);
        else or_rotate(pp, l, galois_rot(n, b), in, baby_keys[b], rot + b * ctw);
    }
    uint64_t *acc = alloc_limbs(2 * (size_t)l, n), *inner = alloc_limbs(2 * (size_t)l, n),
             *tmp = alloc_limbs(2 * (size_t)l, n);
    for (uint32_t g = 0; g < G; g++) {
        memset(inner, 0, sizeof(uint64_t) * ctw);
        for (uint32_t b = 0; b < Bs; b++) {
            const uint64_t *p = pt + ((size_t)g * Bs + b) * ln;
            for (uint32_t c = 0; c < 2; c++)
                for (uint32_t i = 0; i < l; i++)
                    for (uint32_t k = 0; k < n; k++) {
                        size_t o = (size_t)i * n + k;
                        inner[c * ln + o] = addmod(inner[c * ln + o],
                                                   or_mulmod(p[o], rot[b * ctw + c * ln + o], pp->primes[i]),
                                                   pp->primes[i]);
                    }
        }
        const uint64_t *add = inner;
        if (g > 0) { or_rotate(pp, l, galois_rot(n, (uint64_t)g * Bs), inner, giant_keys[g], tmp); add = tmp; }
        for (uint32_t c = 0; c < 2; c++)
            for (uint32_t i = 0; i < l; i++)
                for (uint32_t k = 0; k < n; k++) {
                    size_t o = c * ln + (size_t)i * n + k;
                    acc[o] = addmod(acc[o], add[o], pp->primes[i]);
                }
    }
    if (do_rescale) or_rescale(pp, l, acc, out);
    else memcpy(out, acc, sizeof(uint64_t) * ctw);
    free(rot); free(acc); free(inner); free(tmp);
}

/* The two element-wise steps of the BSGS sum above, as separate calls (a
 * caller that streams diagonals and keys composes the same sum from them):
 * acc[c][i][k] += pt[i][k] ct[c][i][k] mod q_i for both polynomials c, and
 * out = a + b mod q_i over [count][l][n] arrays. */
void or_mul_acc(const or_params *pp, uint32_t l, const uint64_t *pt, const uint64_t *ct, uint64_t *acc) {
    const uint32_t n = pp->n;
    const size_t ln = (size_t)l * n;
#pragma omp parallel for schedule(static)
    for (uint32_t i = 0; i < l; i++)
        for (uint32_t c = 0; c < 2; c++)
            for (uint32_t k = 0; k < n; k++) {
                size_t o = (size_t)i * n + k;
                acc[c * ln + o] = addmod(acc[c * ln + o], or_mulmod(pt[o], ct[c * ln + o], pp->primes[i]),
                                         pp->primes[i]);
            }
}

void or_add(const or_params *pp, uint32_t l, uint32_t count, const uint64_t *a, const uint64_t *b, uint64_t *out) {
    const uint32_t n = pp->n;
#pragma omp parallel for schedule(static)
    for (uint32_t r = 0; r < count * l; r++)
        for (uint32_t k = 0; k < n; k++) {
            size_t o = (size_t)r * n + k;
            out[o] = addmod(a[o], b[o], pp->primes[r % l]);
        }
}

/* ======================================================================
 * Encoding, keys, encryption (used by the functional checks only)
 * ====================================================================== */
/* Slot j is the value at zeta^(5^j mod 2n), zeta = exp(i pi / n); the real
 * coefficients are m_i = (2/n) Re sum_j z_j zeta^(-(5^j) i). */
void or_encode_coeffs(uint32_t n, const double *z_re, const double *z_im, double delta, int64_t *coeffs) {
    const uint32_t m = 2 * n, slots = n / 2;
    long double *cs = malloc(sizeof(long double) * m), *sn = malloc(sizeof(long double) * m);
    const long double pi = 3.141592653589793238462643383279502884L;
    for (uint32_t k = 0; k < m; k++) { cs[k] = cosl(pi * k / n); sn[k] = sinl(pi * k / n); }
    uint64_t *e = malloc(sizeof(uint64_t) * slots);
    for (uint32_t j = 0; j < slots; j++) e[j] = or_powmod(5, j, m);
    for (uint32_t i = 0; i < n; i++) {
        long double re = 0;
        for (uint32_t j = 0; j < slots; j++) {
            uint64_t a = (m - (e[j] * i) % m) % m; /* angle index of zeta^(-e_j i) */
            re += (long double)z_re[j] * cs[a] - (long double)z_im[j] * sn[a];
        }
        long double v = re * 2.0L / n * (long double)delta;
        coeffs[i] = (int64_t)(v >= 0 ? floorl(v + 0.5L) : -floorl(-v + 0.5L));
    }
    free(cs); free(sn); free(e);
}

void or_coeffs_to_ntt(const or_params *pp, uint32_t nlimbs, const uint32_t *prime_idx,
                      const int64_t *coeffs, uint64_t *out) {
    for (uint32_t r = 0; r < nlimbs; r++) {
        uint64_t q = pp->primes[prime_idx[r]];
        for (uint32_t k = 0; k < pp->n; k++) out[(size_t)r * pp->n + k] = from_signed(coeffs[k], q);
    }
    ntt_limbs(pp, nlimbs, prime_idx, out, 0);
}

void or_decode(const or_params *pp, uint32_t l, const uint64_t *m_coef, double delta, double *z_re, double *z_im) {
    const uint32_t n = pp->n, m = 2 * n, slots = n / 2;
    crt_basis c;
    crt_init(&c, l, pp->primes);
    long double *v = malloc(sizeof(long double) * n);
    uint64_t *mag = malloc(sizeof(uint64_t) * c.w), *scr = malloc(sizeof(uint64_t) * c.w), *xi = malloc(sizeof(uint64_t) * l);
    for (uint32_t k = 0; k < n; k++) {
        for (uint32_t i = 0; i < l; i++) xi[i] = m_coef[(size_t)i * n + k];
        int neg = crt_centered(&c, l, pp->primes, xi, mag, scr);
        long double x = 0;
        for (int w = c.w - 1; w >= 0; w--) x = x * 18446744073709551616.0L + (long double)mag[w];
        v[k] = neg ? -x : x;
    }
    long double *cs = malloc(sizeof(long double) * m), *sn = malloc(sizeof(long double) * m);
    const long double pi = 3.141592653589793238462643383279502884L;
    for (uint32_t k = 0; k < m; k++) { cs[k] = cosl(pi * k / n); sn[k] = sinl(pi * k / n); }
    for (uint32_t j = 0; j < slots; j++) {
        uint64_t e = or_powmod(5, j, m);
        long double re = 0, im = 0;
        for (uint32_t i = 0; i < n; i++) {
            uint64_t a = (e * i) % m;
            re += v[i] * cs[a];
            im += v[i] * sn[a];
        }
        z_re[j] = (double)(re / delta);
        z_im[j] = (double)(im / delta);
    }
    free(v); free(mag); free(scr); free(xi); free(cs); free(sn);
    crt_free(&c);
}

/* Switching key: row j encodes P * s' on the primes of digit j (full chain),
 * i.e. b_j = -a_j s + e_j + [P]_q s' there, and -a_j s + e_j elsewhere. */
void or_keygen_swk(const or_params *pp, const uint64_t *s_ntt, const uint64_t *sp_ntt,
                   const uint64_t *a, const int64_t *e, uint64_t *key) {
    const uint32_t n = pp->n, L = pp->L, K = pp->K, alpha = or_alpha(pp), dn = pp->dnum;
    const uint32_t tot = L + K;
    uint32_t *idx = malloc(sizeof(uint32_t) * tot);
    for (uint32_t r = 0; r < tot; r++) idx[r] = r;
    uint64_t *en = alloc_limbs(tot, n);
    for (uint32_t j = 0; j < dn; j++) {
        uint32_t lo = j * alpha, hi = (j + 1) * alpha < L ? (j + 1) * alpha : L;
        or_coeffs_to_ntt(pp, tot, idx, e + (size_t)j * n, en);
        uint64_t *kb = key + (size_t)j * 2 * tot * n, *ka = kb + (size_t)tot * n;
        const uint64_t *aj = a + (size_t)j * tot * n;
        for (uint32_t r = 0; r < tot; r++) {
            uint64_t q = pp->primes[r], Pq = 1;
            for (uint32_t k = 0; k < K; k++) Pq = or_mulmod(Pq, pp->primes[L + k] % q, q);
            for (uint32_t k = 0; k < n; k++) {
                size_t o = (size_t)r * n + k;
                uint64_t v = submod(en[o], or_mulmod(aj[o], s_ntt[o], q), q);
                if (r >= lo && r < hi) v = addmod(v, or_mulmod(Pq, sp_ntt[o], q), q);
                kb[o] = v;
                ka[o] = aj[o];
            }
        }
    }
    free(idx); free(en);
}

void or_encrypt(const or_params *pp, uint32_t l, const uint64_t *m_ntt, const uint64_t *s_ntt,
                const uint64_t *a, const int64_t *e, uint64_t *ct) {
    const uint32_t n = pp->n;
    uint32_t *idx = calloc(l ? l : 1, sizeof(uint32_t));
    for (uint32_t r = 0; r < l; r++) idx[r] = r;
    uint64_t *en = alloc_limbs(l, n);
    or_coeffs_to_ntt(pp, l, idx, e, en);
    for (uint32_t i = 0; i < l; i++) {
        uint64_t q = pp->primes[i];
        for (uint32_t k = 0; k < n; k++) {
            size_t o = (size_t)i * n + k;
            ct[o] = addmod(submod(en[o], or_mulmod(a[o], s_ntt[o], q), q), m_ntt[o], q);
            ct[(size_t)l * n + o] = a[o];
        }
    }
    free(idx); free(en);
}

void or_decrypt(const or_params *pp, uint32_t l, const uint64_t *ct, const uint64_t *s_ntt, uint64_t *m_coef) {
    const uint32_t n = pp->n;
    uint32_t *idx = calloc(l ? l : 1, sizeof(uint32_t));
    for (uint32_t r = 0; r < l; r++) idx[r] = r;
    for (uint32_t i = 0; i < l; i++) {
        uint64_t q = pp->primes[i];
        for (uint32_t k = 0; k < n; k++) {
            size_t o = (size_t)i * n + k;
            m_coef[o] = addmod(ct[o], or_mulmod(ct[(size_t)l * n + o], s_ntt[o], q), q);
        }
    }
    ntt_limbs(pp, l, idx, m_coef, 1);
    free(idx);
}
