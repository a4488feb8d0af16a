/*
 * oracle.h -- plain, slow, CPU reference for the RNS-CKKS hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the GPU library.
 *
 * What it computes (sources are the pages this project is built from):
 *  - Kestrel FHE relay README, section 1 ("what we are doing"): ring degree
 *    n = 2048, 1024 slots, scale 2^60, 112 RNS primes for the layer chain and
 *    2100 for bootstrapping.
 *  - The Kestrel article on encrypted 2B-model inference, section 3 (technique
 *    table: NTT/INTT, RNS decomposition, modulus chain + rescale, RNS base
 *    conversion, Galois rotation/conjugation, baby-step giant-step matmul),
 *    section 4.1 (key parameters), wall 2 (every rescale uses up one prime)
 *    and "wall 3" (boot profile: coeff_to_slot / slot_to_coeff).
 *  - The EncryptedLLM GPU blog, section 3.4 (NTT kernel, base conversion
 *    between prime sets).
 *
 * The pages print no formulas.  Every arithmetic convention below is the
 * plain textbook reading of those words (the readings are listed with the
 * design notes of the repository):
 *  - primes: the smallest primes in (2^59, 2^60) with q = 1 mod 2n, ascending;
 *    main primes first, special primes are the continuation of that list;
 *  - psi: the smallest primitive 2n-th root of unity mod q;
 *  - NTT: A_j = sum_i a_i psi^(i(2j+1)) mod q, natural order j;
 *  - base conversion: exact CRT, centered representative in (-B/2, B/2);
 *  - hybrid key switching (ModUp per digit, inner product, ModDown = round(./P));
 *  - rescale: divide by the last prime with rounding;
 *  - Galois automorphism X -> X^g, rotation g = 5^k mod 2n, conjugation 2n-1.
 *
 * Layouts: a polynomial at level l is l limbs of n uint64 residues, limb-major
 * ([l][n]); a ciphertext is two such polynomials ([2][l][n]).  Ciphertexts,
 * keys and plaintexts live in the NTT (evaluation) domain.  All residues are
 * fully reduced to [0, q).
 */
#ifndef CKKS_ORACLE_H
#define CKKS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------- scalar modular arithmetic and parameter generation ---------- */
uint64_t or_mulmod(uint64_t a, uint64_t b, uint64_t q);
uint64_t or_powmod(uint64_t a, uint64_t e, uint64_t q);
uint64_t or_invmod(uint64_t a, uint64_t q);
int      or_is_prime(uint64_t x);
/* The `count` smallest primes q in (2^59, 2^60) with q = 1 (mod 2n), ascending. */
int      or_gen_primes(uint32_t n, uint32_t count, uint64_t *out);
/* Smallest primitive 2n-th root of unity modulo prime q (q = 1 mod 2n). */
uint64_t or_min_psi(uint32_t n, uint64_t q);

/* ---------- single-limb transforms ---------- */
/* O(n^2) definition of the negacyclic NTT and its inverse. */
void or_ntt_definition(uint32_t n, uint64_t q, uint64_t psi, const uint64_t *a, uint64_t *out);
void or_intt_definition(uint32_t n, uint64_t q, uint64_t psi, const uint64_t *a, uint64_t *out);
/* Textbook O(n log n) version: twist by psi^i, radix-2 cyclic NTT with psi^2. In place. */
void or_ntt(uint32_t n, uint64_t q, uint64_t psi, uint64_t *a);
void or_intt(uint32_t n, uint64_t q, uint64_t psi, uint64_t *a);
/* Schoolbook product in Z_q[X]/(X^n + 1). */
void or_negacyclic_schoolbook(uint32_t n, uint64_t q, const uint64_t *a, const uint64_t *b, uint64_t *out);
/* Coefficient-domain automorphism a(X) -> a(X^g), g odd. */
void or_automorph_coef(uint32_t n, uint64_t q, uint64_t g, const uint64_t *in, uint64_t *out);

/* ---------- exact base conversion (bigint CRT) ---------- */
/* x: [nb][n] residues modulo b[0..nb); out: [nt][n] residues modulo t[0..nt)
 * of the centered CRT representative of x modulo B = prod b. */
void or_base_convert(uint32_t n, uint32_t nb, const uint64_t *b, const uint64_t *x,
                     uint32_t nt, const uint64_t *t, uint64_t *out);

/* ---------- CKKS parameter set ---------- */
typedef struct {
    uint32_t n, L, K, dnum;
    const uint64_t *primes; /* [L + K]: q_0..q_{L-1}, then p_0..p_{K-1} */
    const uint64_t *psi;    /* [L + K]: minimal primitive 2n-th roots    */
} or_params;

/* digit width alpha = ceil(L / dnum); number of digits at level l = ceil(l / alpha) */
uint32_t or_alpha(const or_params *pp);
uint32_t or_beta(const or_params *pp, uint32_t l);

/* ---------- ciphertext operations (NTT domain) ---------- */
/* d = (c0 c0', c0 c1' + c1 c0', c1 c1'); a,b: [2][l][n]; d: [3][l][n] */
void or_tensor(const or_params *pp, uint32_t l, const uint64_t *a, const uint64_t *b, uint64_t *d);
/* Hybrid key switch of d ([l][n], NTT domain) with key [dnum][2][L+K][n];
 * out: [2][l][n] = ModDown(sum_j ModUp_j(d) * (b_j, a_j)). */
void or_keyswitch(const or_params *pp, uint32_t l, const uint64_t *d, const uint64_t *key, uint64_t *out);
/* Tensor then relinearise: out [2][l][n]. */
void or_mul_tensor_relin(const or_params *pp, uint32_t l, const uint64_t *a, const uint64_t *b,
                         const uint64_t *rlk, uint64_t *out);
/* Drop the last prime with rounding: in [2][l][n] -> out [2][l-1][n]. */
void or_rescale(const or_params *pp, uint32_t l, const uint64_t *in, uint64_t *out);
/* NTT-domain automorphism of one polynomial at level l (via iNTT, index map, NTT). */
void or_automorph(const or_params *pp, uint32_t l, uint64_t g, const uint64_t *in, uint64_t *out);
/* Rotation / conjugation: out = (sigma_g(c0), 0) + KS(sigma_g(c1)). */
void or_rotate(const or_params *pp, uint32_t l, uint64_t g, const uint64_t *in, const uint64_t *key,
               uint64_t *out);
/* Baby-step giant-step linear transform:
 *   y = sum_{g<G} rot_{g*Bs}( sum_{b<Bs} pt[g][b] (.) rot_b(x) ), then rescale if asked.
 * pt: [G][Bs][l][n]; baby_keys[b] for b = 1..Bs-1; giant_keys[g] for g = 1..G-1.
 * out: [2][l][n] or [2][l-1][n]. */
void or_bsgs(const or_params *pp, uint32_t l, const uint64_t *in, const uint64_t *pt,
             uint32_t Bs, uint32_t G, const uint64_t *const *baby_keys,
             const uint64_t *const *giant_keys, int do_rescale, uint64_t *out);

/* The element-wise steps of or_bsgs: acc[c] += pt (.) ct[c] (c = 0, 1; pt
 * [l][n], ct and acc [2][l][n]), and out = a + b over [count][l][n]. */
void or_mul_acc(const or_params *pp, uint32_t l, const uint64_t *pt, const uint64_t *ct, uint64_t *acc);
void or_add(const or_params *pp, uint32_t l, uint32_t count, const uint64_t *a, const uint64_t *b, uint64_t *out);

/* ---------- encoding / keys / encryption (functional checks only) ---------- */
/* Integer coefficients of the encoding of z (slots = n/2) at scale delta,
 * rounded half away from zero.  z_re/z_im: [n/2]. */
void or_encode_coeffs(uint32_t n, const double *z_re, const double *z_im, double delta, int64_t *coeffs);
/* Residues of integer coefficients, then NTT: out [l][n] over primes idx[0..l). */
void or_coeffs_to_ntt(const or_params *pp, uint32_t nlimbs, const uint32_t *prime_idx,
                      const int64_t *coeffs, uint64_t *out);
/* Decode coefficient-domain residues m [l][n] (centered CRT) at scale delta. */
void or_decode(const or_params *pp, uint32_t l, const uint64_t *m_coef, double delta,
               double *z_re, double *z_im);
/* Switching key for target s' (NTT domain over Q_L u P, [L+K][n]) under secret s
 * (NTT domain, [L+K][n]).  a: uniform [dnum][L+K][n] (NTT domain); e: small
 * integer errors [dnum][n].  key out: [dnum][2][L+K][n] with row 0 = b, row 1 = a. */
void or_keygen_swk(const or_params *pp, const uint64_t *s_ntt, const uint64_t *sp_ntt,
                   const uint64_t *a, const int64_t *e, uint64_t *key);
/* Symmetric encryption at level l: (-a s + e + m, a); m, a: [l][n] NTT; e: [n]. */
void or_encrypt(const or_params *pp, uint32_t l, const uint64_t *m_ntt, const uint64_t *s_ntt,
                const uint64_t *a, const int64_t *e, uint64_t *ct);
/* m = c0 + c1 s, returned in the coefficient domain [l][n]. */
void or_decrypt(const or_params *pp, uint32_t l, const uint64_t *ct, const uint64_t *s_ntt, uint64_t *m_coef);

#ifdef __cplusplus
}
#endif
#endif
