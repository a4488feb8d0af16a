/*
 * ckks_gpu.h -- C ABI of the MI355X (gfx950) RNS-CKKS arithmetic core.
 *
 * Scope: the data-parallel hot path of RNS-CKKS as described by the Kestrel
 * FHE relay pages: batched negacyclic NTT/iNTT over many 60-bit primes,
 * ciphertext-ciphertext multiply with relinearisation, rescale, Galois
 * rotation/conjugation with hybrid key switching, and the baby-step
 * giant-step (BSGS) plaintext-matrix times ciphertext transform that
 * coeff_to_slot / slot_to_coeff are made of.
 *
 * Conventions shared by every call
 *  - Ring Z_q[X]/(X^n + 1), n a power of two (2048 or 65536 here).
 *  - Chain: the L + K smallest primes q in (2^59, 2^60) with q = 1 (mod 2n),
 *    ascending; the first L are the main primes q_0..q_{L-1}, the next K the
 *    special primes p_0..p_{K-1} used by key switching.  Prime index g in
 *    [0, L+K) names one of them.
 *  - psi_g = the smallest primitive 2n-th root of unity modulo prime g.
 *  - NTT (evaluation) domain: A_j = sum_i a_i psi^(i(2j+1)) mod q, j in
 *    natural order.  Ciphertexts, keys and plaintexts are passed in this domain.
 *  - A polynomial at level l is l limbs of n uint64 residues, limb-major
 *    ([l][n], limb i modulo q_i); a ciphertext is [2][l][n]; a batch of B
 *    ciphertexts is [B][2][l][n].  Every residue is fully reduced to [0, q)
 *    on input and is returned fully reduced.
 *  - Switching key: [dnum][2][L+K][n]; row (j, 0) = b_j, row (j, 1) = a_j,
 *    limb g modulo prime g (main primes, then special primes).  Digit j
 *    covers main primes [j*alpha, min((j+1)*alpha, l)), alpha = ceil(L/dnum).
 *  - Rotation left by k slots uses Galois element 5^k mod 2n; conjugation
 *    uses 2n - 1.
 *
 * Memory and streams
 *  - Data pointers are DEVICE pointers on the context's device, allocated and
 *    owned by the caller (8-byte aligned).  Pointer-array arguments
 *    (BSGS keys) are HOST arrays of key descriptors.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; nothing synchronises with the host and no call
 *    allocates device memory after context creation and level preparation.
 *  - Levels: an operation at level l uses constant tables of that level (the
 *    partial last key-switching digit, rescale inverses).  ckks_ctx_create
 *    builds them for every level when L <= CKKS_PREPARE_ALL_MAX_L; for longer
 *    chains the caller builds the levels it will use with ckks_prepare_levels
 *    (and ckks_prepare_raise for ModRaise) before the first call there.  A
 *    call at a level that is not prepared returns CKKS_ENOTREADY.  The
 *    context is read-only after that: concurrent calls on different streams
 *    are safe given distinct workspaces (preparation must not run concurrently
 *    with other calls on the same context).
 *  - Workspace: ops that need scratch take (ws, ws_bytes); query the size with
 *    ckks_workspace_size.  The caller owns it.  At n = 65536 the workspace also
 *    holds the four-step NTT's transpose buffer; the bare NTT calls, which take
 *    no workspace, share one context buffer and are ordered across streams by
 *    a context event (at n = 2048 every transform stays in LDS).
 *  - Aliasing: the NTT calls work in place; ckks_pointwise_mul accepts
 *    out == a or out == b exactly; every other call rejects (CKKS_EINVAL) an
 *    output whose byte range overlaps an input's.
 *
 * Errors: every call returns CKKS_OK (0) or a negative CKKS_E* code; arguments
 * are validated before any launch; nothing is printed.
 */
#ifndef CKKS_GPU_H
#define CKKS_GPU_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKKS_OK 0
#define CKKS_EINVAL (-1)     /* bad argument (null pointer, size out of range) */
#define CKKS_ELEVEL (-2)     /* level out of range for this context / op      */
#define CKKS_ENOMEM (-3)     /* device allocation failed (context creation)   */
#define CKKS_EHIP (-4)       /* a HIP runtime call or kernel launch failed     */
#define CKKS_EALIGN (-5)     /* pointer not 8-byte aligned                     */
#define CKKS_EWORKSPACE (-6) /* workspace missing or smaller than required     */
#define CKKS_EUNSUPPORTED (-7) /* ring degree / parameter not supported        */
#define CKKS_EKEY (-8)       /* switching key made for another parameter set,  */
                             /* or a seeded key where a stored one is needed    */
#define CKKS_ENOTREADY (-9)  /* level tables not prepared (ckks_prepare_levels) */

/* Chains up to this many main primes get every level's tables at creation. */
#define CKKS_PREPARE_ALL_MAX_L 256

typedef struct ckks_ctx ckks_ctx;

typedef struct {
    uint32_t n;    /* ring degree: 2048 or 65536                          */
    uint32_t L;    /* number of main primes (top level)                    */
    uint32_t K;    /* number of special primes (0: no key switching)      */
    uint32_t dnum; /* number of key-switching digits (>= 1 when K > 0)    */
} ckks_params;

/* Create a context on HIP device `device`: generates the chain primes and
 * roots (Kestrel relay README section 1 / article section 4.1 parameters:
 * n = 2048, 60-bit primes, 112 or 2100 of them), and uploads twiddle and
 * base-conversion tables; with L <= CKKS_PREPARE_ALL_MAX_L also every level's
 * tables and every ModRaise source level's.  Returns CKKS_EUNSUPPORTED for
 * unsupported n, for a chain prime at or above 2^59 + 2^52, or for a digit
 * width ceil(L/dnum) or K above 1000 (the bounds of the exact 128-bit
 * base-conversion sums).  Blocking; allocates. */
int ckks_ctx_create(ckks_ctx **out, const ckks_params *params, int device);
void ckks_ctx_destroy(ckks_ctx *ctx);
/* Build the tables of levels level_lo..level_hi (inclusive; levels already
 * built are kept).  Blocking; allocates; not concurrent with other calls on
 * the context.  CKKS_ELEVEL for a range outside [1, L]. */
int ckks_prepare_levels(ckks_ctx *ctx, int level_lo, int level_hi);
/* Build the ModRaise tables of source level level_in (ckks_mod_raise,
 * ckks_bootstrap).  Same rules as ckks_prepare_levels; level_in <= min(L, 1000). */
int ckks_prepare_raise(ckks_ctx *ctx, int level_in);
/* Copy the chain primes and their psi to host arrays of L+K entries (either may be NULL). */
int ckks_ctx_primes(const ckks_ctx *ctx, uint64_t *host_primes, uint64_t *host_psi);
const char *ckks_strerror(int code);

/* Switching key descriptor (hybrid key switching, Kestrel article technique
 * table: relinearisation and Galois keys; EncryptedLLM GPU blog section 2.5:
 * keys of hundreds of MB to GB, preloaded on the device).
 *  - Stored key (seeded = 0): data = [dnum][2][L+K][n], NTT domain; row
 *    (j, 0) = b_j, row (j, 1) = a_j, limb g modulo chain prime g.
 *  - Seeded key (seeded = 1, EncryptedLLM blog section 4.4: cut key size when
 *    memory or key loading is the limit): data = the b rows [dnum][L+K][n];
 *    the a rows are regenerated from `seed` where they are used:
 *      a_j[i][k] = floor(w q_i / 2^64),  w = S(S(S(seed, 10), j (L+K) + i), k),
 *      S(s, t) = mix64(s + (t + 1) 0x9e3779b97f4a7c15),
 *    mix64 the SplitMix64 finaliser (Steele, Lea, Flood, OOPSLA 2014):
 *      z ^= z >> 30; z *= 0xbf58476d1ce4e5b9; z ^= z >> 27; z *= 0x94d049bb133111eb;
 *      z ^= z >> 31.
 *    Relinearisation and rotation take seeded keys; BSGS, EvalMod and
 *    bootstrapping need stored ones (ckks_key_expand converts).
 * (n, L, K, dnum) name the parameter set the key was generated for: every
 * call checks them against its context and returns CKKS_EKEY on a mismatch.
 * The descriptor is read during the call only; `data` must stay valid until
 * the stream work completes. */
typedef struct {
    const uint64_t *data;
    uint32_t n, L, K, dnum;
    uint32_t seeded;
    uint32_t reserved; /* 0 */
    uint64_t seed;
} ckks_swk;

/* Workspace sizes.  op: one of the CKKS_OP_* values; batch = ciphertexts per
 * call; level = l; for CKKS_OP_BSGS, bs and gs are the baby/giant step counts
 * (ignored otherwise). */
#define CKKS_OP_RELIN 1
#define CKKS_OP_ROTATE 2
#define CKKS_OP_RESCALE 3
#define CKKS_OP_BSGS 4
#define CKKS_OP_EVALMOD 5 /* bs = Chebyshev degree */
#define CKKS_OP_MODRAISE 6 /* level = the source level */
int ckks_workspace_size(const ckks_ctx *ctx, int op, int batch, int level, int bs, int gs, size_t *bytes);

/* Forward / inverse negacyclic NTT, in place, of `count` polynomials of
 * `nlimbs` limbs each ([count][nlimbs][n]); limb r uses prime index
 * first_prime + r.  The "NTT/INTT" multiply accelerator of the Kestrel
 * article's technique table; natural order in and out. */
int ckks_ntt_fwd(const ckks_ctx *ctx, uint64_t *x, int count, int first_prime, int nlimbs, void *stream);
int ckks_ntt_inv(const ckks_ctx *ctx, uint64_t *x, int count, int first_prime, int nlimbs, void *stream);

/* Pointwise product in the NTT domain (the middle step of an NTT-based
 * negacyclic polynomial multiply): out = a (.) b limb by limb, layouts as
 * ckks_ntt_fwd ([count][nlimbs][n], limb r modulo prime first_prime + r).
 * out may equal a or b (the same pointer); partial overlap is rejected. */
int ckks_pointwise_mul(const ckks_ctx *ctx, const uint64_t *a, const uint64_t *b, uint64_t *out, int count,
                       int first_prime, int nlimbs, void *stream);

/* Range check of residues: writes to *out_count (device memory, 8-byte
 * aligned) the number of residues of x ([count][nlimbs][n], limb r modulo
 * prime first_prime + r) that are not below their prime.  The operations
 * take residues as reduced and do not check them (that would cost one more
 * read of every input); a caller whose residues come from outside (files,
 * other processes) runs this first and rejects a non-zero count.  count = 0
 * or nlimbs = 0 writes 0.  Stream-ordered: the count is ready when the work
 * queued before it on `stream` is.  Errors: CKKS_EINVAL (null context or
 * counter, negative sizes, limbs past the last prime), CKKS_EALIGN (x or the
 * counter not 8-byte aligned). */
int ckks_count_unreduced(const ckks_ctx *ctx, const uint64_t *x, int count, int first_prime, int nlimbs,
                         uint32_t *out_count, void *stream);

/* Ciphertext-ciphertext multiply with relinearisation (the Kestrel
 * article's wall 2: a product's noise grows, and relinearisation brings the
 * degree-2 ciphertext back to two polynomials): for each of `batch` pairs,
 * (d0, d1, d2) = (a0 b0, a0 b1 + a1 b0, a1 b1) and
 * out = (d0, d1) + KeySwitch(d2, rlk).  a, b, out: [batch][2][level][n];
 * rlk: switching key for s^2 (stored or seeded); out must not overlap a or b. */
int ckks_mul_tensor_relin(const ckks_ctx *ctx, const uint64_t *a, const uint64_t *b, const ckks_swk *rlk,
                          uint64_t *out, int batch, int level, void *ws, size_t ws_bytes, void *stream);

/* Rescale: drop the last prime q_{l-1} with rounding, out = round(c / q_{l-1})
 * (Kestrel article wall 2: every rescale uses up one prime of the chain).
 * in: [batch][2][level][n]; out: [batch][2][level-1][n], not overlapping in. */
int ckks_rescale(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level, void *ws,
                 size_t ws_bytes, void *stream);

/* Galois automorphism X -> X^g followed by hybrid key switching back to s
 * (Galois rotation / conjugation of the Kestrel article's technique table):
 * out = (sigma_g(c0), 0) + KeySwitch(sigma_g(c1), key).  g odd, in [1, 2n).
 * in, out: [batch][2][level][n] (no overlap); key stored or seeded. */
int ckks_rotate(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level, uint32_t galois_elt,
                const ckks_swk *key, void *ws, size_t ws_bytes, void *stream);

/* Expand a seeded key to the stored format: key_out [dnum][2][L + K][n] with
 * key_out[j][0] = the b rows and key_out[j][1] the regenerated a rows (for
 * the calls that take stored keys: BSGS, EvalMod, bootstrapping).  key_out
 * must not overlap the key's data. */
int ckks_key_expand(const ckks_ctx *ctx, const ckks_swk *seeded_key, uint64_t *key_out, void *stream);

/* Rotation for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and errors as ckks_rotate, with no workspace argument.
 * Its workspace is a device array of CKKS_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; a call needing more
 * (ckks_workspace_size with CKKS_OP_ROTATE) returns CKKS_EWORKSPACE.  All
 * calls on one GPU share that array: calls that overlap on a GPU (other
 * streams, other threads, other contexts) race, so the caller serialises
 * them. */
#define CKKS_NOALLOC_SCRATCH_BYTES (256ull << 20)
int ckks_rotate_noalloc(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level,
                        uint32_t galois_elt, const ckks_swk *key, void *stream);

/* Baby-step giant-step plaintext-matrix x ciphertext (matmul2 with BB x GG,
 * Kestrel article technique table and section 4.4; coeff_to_slot /
 * slot_to_coeff are this transform):
 *   y = sum_{g<gs} rot_{g*bs}( sum_{b<bs} diags[g][b] (.) rot_b(x) ),
 * then, if do_rescale, out = Rescale(y).  diags: [gs][bs][level][n]
 * (encoded pre-rotated diagonals, NTT domain); baby_keys[b] is the key of
 * rotation by b (b = 1..bs-1, entry 0 ignored); giant_keys[g] the key of
 * rotation by g*bs (g = 1..gs-1, entry 0 ignored); stored keys.  in:
 * [batch][2][level][n]; out: [batch][2][level - do_rescale][n], no overlap. */
int ckks_bsgs_linear_transform(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level,
                               const uint64_t *diags, int bs, int gs, const ckks_swk *const *baby_keys,
                               const ckks_swk *const *giant_keys, int do_rescale, void *ws, size_t ws_bytes,
                               void *stream);

/* ModRaise, the first step of bootstrapping (modraise in the Kestrel
 * article's section 5.3 boot profile: a ciphertext down to 19 primes is
 * raised to 2100): every coefficient of both polynomials is lifted exactly to
 * its centered representative modulo q_0 ... q_{level_in - 1} and reduced
 * modulo q_0 ... q_{level_out - 1}.  The plaintext becomes m + (q_0...) I
 * for a small integer polynomial I, which EvalMod later removes.  in:
 * [batch][2][level_in][n] (NTT domain); out: [batch][2][level_out][n]; no
 * aliasing; level_in <= min(level_out, 1000); ModRaise tables of level_in
 * prepared (ckks_prepare_raise). */
int ckks_mod_raise(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level_in, int level_out,
                   void *ws, size_t ws_bytes, void *stream);

/* EvalMod: the modular-reduction stage of bootstrapping (sin_fold_re /
 * sin_fold_im of the Kestrel article's section 5.3 boot profile, the second
 * largest bootstrap cost there), on real slot values x in [-K, K]:
 *   u = x / K,   p = sum_{k<=degree} cheb[k] T_k(u)   (Chebyshev basis),
 *   y = p, then y <- 2 y^2 - 1 (double_angles times),   out = out_factor y.
 * With cheb the interpolant of cos(2 pi (K u - 1/4) / 2^double_angles) on
 * [-1, 1] and out_factor = 1 / (2 pi), out ~ sin(2 pi x) / (2 pi).
 * Exact schedule (every step a ciphertext operation; s(.) = tracked scale,
 * q_j = chain prime j, const(c, t) = the integer nearest c t, ties to even):
 *   CMul(a, c): multiply by const(c, q_{l_a - 1}), rescale; scale kept;
 *   Mul(a, b): both truncated to the lower level m, tensor + relinearise,
 *     rescale; scale s(a) s(b) / q_{m-1};
 *   T_1 = CMul(in, 1/K); T_2j = 2 Mul(T_j, T_j) + const(-1, s);
 *   T_2j+1 = 2 Mul(T_j, T_j+1) - T_1 (truncated); scale that of the Mul;
 *   p: with m = level of T_degree, sum_k const(cheb[k], q_{m-1}) T_k (each
 *     truncated to m), rescale, scale s(T_degree), then + const(cheb[0], s);
 *   y <- 2 Mul(y, y) + const(-1, s(Mul));  out = CMul(y, out_factor).
 * Constants enter c0 of the NTT-domain ciphertext in every coefficient.
 * Levels consumed: 3 + ceil(log2 degree) + double_angles; out is written at
 * level *level_out = level minus that, scale *scale_out.  The scales stay
 * near scale_in only if scale_in is close to the chain primes (e.g. 2^59 for
 * primes just above 2^59).  in: [batch][2][level][n]; out:
 * [batch][2][*level_out][n] (may alias in exactly); cheb: host array of degree + 1
 * doubles, |cheb[k]| < 2; 0.5 <= K; |out_factor| < 2; 1 <= degree <= 1024;
 * 0 <= double_angles <= 64; scale_in in (0, 2^61); rlk as
 * ckks_mul_tensor_relin (stored key); every level from level down to
 * *level_out + 1 prepared.  Returns CKKS_EINVAL (after queuing the work) if a
 * constant times its scale reaches 2^62, the output then being invalid. */
int ckks_eval_mod(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level, double scale_in,
                  const double *cheb, int degree, double bound_k, int double_angles, double out_factor,
                  const ckks_swk *rlk, void *ws, size_t ws_bytes, double *scale_out, int *level_out,
                  void *stream);

/* Bootstrapping (the boot of the Kestrel article's section 5.3, with its
 * stages modraise, coeff_to_slot, conj_extract, sin_fold_re / sin_fold_im,
 * restore_merge, slot_to_coeff):
 *   r  = ModRaise(in, level_in -> level_raise);
 *   w  = BSGS(r, cts_diags) with rescale                (coeff_to_slot);
 *   re = CMul(w + conj(w), 1/2),  im = CMul((w - conj(w)) X^(n/2), -1/2)
 *        (conj = rotation by g = 2n - 1 with conj_key; CMul as ckks_eval_mod;
 *        X^(n/2) multiplies the slots by the imaginary unit)  (conj_extract);
 *   re', im' = EvalMod of both (one call on 2 batch ciphertexts, input scale
 *        evalmod_scale, parameters as ckks_eval_mod)    (sin_fold);
 *   v  = re' + im' X^(n/2)                               (restore_merge);
 *   out = BSGS(v, stc_diags) with rescale                (slot_to_coeff).
 * Both transforms use bs x gs steps and the same rotation keys (as
 * ckks_bsgs_linear_transform).  The caller builds the diagonals (the slot
 * <-> coefficient matrices with their scale factors) and the EvalMod
 * constants.  Output level *level_out = level_raise - 3 - (3 + ceil(log2
 * degree) + double_angles); *scale_mid = the EvalMod output scale (the scale
 * entering slot_to_coeff).  in: [batch][2][level_in][n]; cts_diags:
 * [gs][bs][level_raise][n]; stc_diags: [gs][bs][*level_out + 1][n]; out:
 * [batch][2][*level_out][n]; no aliasing; stored keys; the ModRaise tables
 * of level_in and every level from level_raise down to *level_out + 1
 * prepared. */
typedef struct {
    int level_raise;
    const uint64_t *cts_diags;
    const uint64_t *stc_diags;
    int bs, gs;
    const ckks_swk *const *baby_keys;
    const ckks_swk *const *giant_keys;
    const ckks_swk *conj_key;
    const ckks_swk *rlk;
    double evalmod_scale;
    const double *cheb;
    int degree;
    double bound_k;
    int double_angles;
    double out_factor;
} ckks_boot_params;
int ckks_bootstrap_workspace_size(const ckks_ctx *ctx, int batch, int level_in, const ckks_boot_params *params,
                                  size_t *bytes);
int ckks_bootstrap(const ckks_ctx *ctx, const uint64_t *in, uint64_t *out, int batch, int level_in,
                   const ckks_boot_params *params, void *ws, size_t ws_bytes, double *scale_mid, int *level_out,
                   void *stream);

#ifdef __cplusplus
}
#endif
#endif
