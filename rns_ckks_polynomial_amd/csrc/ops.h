// ops.h -- internal launchers (host side) for the hot-path operations.
#pragma once
#include "../../include/ckks_gpu.h"
#include "ctx_internal.h"

namespace ckks {

// NTT of plain strided limbs: [count][nlimbs][n], limb r uses prime first + r.
int op_ntt(const ckks_ctx *c, uint64_t *x, int count, int first, int nlimbs, bool inverse, hipStream_t s);

int op_pointwise_mul(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, uint64_t *out, int count, int first,
                     int nlimbs, hipStream_t s);
// Residues >= their prime in [count][nlimbs][n] (limb r modulo prime first + r), written to *out.
int op_count_unreduced(const ckks_ctx *c, const uint64_t *x, int count, int first, int nlimbs, uint32_t *out,
                       hipStream_t s);

size_t ws_bytes_relin(const ckks_ctx *c, int B, int l);
size_t ws_bytes_rotate(const ckks_ctx *c, int B, int l);
size_t ws_bytes_rescale(const ckks_ctx *c, int B, int l);
size_t ws_bytes_bsgs(const ckks_ctx *c, int B, int l, int bs, int gs);

// Keys are validated descriptors (stored, or seeded where the caller allows it).
// Every op returns CKKS_ENOTREADY when a level it needs was not prepared.
int op_mul_tensor_relin(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, const ckks_swk *rlk, uint64_t *out,
                        int B, int l, void *ws, hipStream_t s);
int op_rescale(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, void *ws, hipStream_t s);
int op_rotate(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, uint32_t g, const ckks_swk *key,
              void *ws, bool accumulate, hipStream_t s);
int op_key_expand(const ckks_ctx *c, const ckks_swk *key, uint64_t *key_out, hipStream_t s);
int op_bsgs(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, const uint64_t *diags, int bs, int gs,
            const ckks_swk *const *baby, const ckks_swk *const *giant, bool rescale, void *ws, hipStream_t s);
// ModRaise: centered lift of [B][2][l0][n] (primes [0, l0)) to [B][2][lt][n].
size_t ws_bytes_mod_raise(const ckks_ctx *c, int B, int l0);
int op_mod_raise(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l0, int lt, void *ws, hipStream_t s);
// out = ma a + mb b' (+ add on c0) on limbs [0, lo) of B ciphertexts; b' = b X^(n/2) if mono_b.
int op_lincomb(const ckks_ctx *c, uint64_t *out, int lo, const uint64_t *a, int la, const uint64_t *b, int lb,
               int64_t ma, int64_t mb, int64_t add, bool mono_b, int B, hipStream_t s);
// The integer nearest c t (ties to even); clears *ok if |c t| >= 2^62.
int64_t enc_const(double c, double t, bool *ok);
// EvalMod (Chebyshev cosine + double angles); levels consumed = eval_mod_depth(degree, double_angles).
int eval_mod_depth(int degree, int double_angles);
size_t ws_bytes_eval_mod(const ckks_ctx *c, int B, int l, int degree);
int op_eval_mod(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, double scale_in, const double *cheb,
                int degree, double bound_k, int double_angles, double out_factor, const ckks_swk *rlk, void *ws,
                double *scale_out, int *level_out, hipStream_t s);
// Bootstrapping: ModRaise -> CtS -> conj_extract -> EvalMod (re, im) -> merge -> StC.
int boot_levels(const ckks_boot_params *p, int *l_out);
size_t ws_bytes_bootstrap(const ckks_ctx *c, int B, int l0, const ckks_boot_params *p);
int op_bootstrap(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l0, const ckks_boot_params *p,
                 void *ws, double *scale_mid, hipStream_t s);
// Look up (once per device, with that device current) the device address of the
// no-allocation workspace array.
int noalloc_init(int device);
int op_fill_uniform(const ckks_ctx *c, uint64_t *dst, int count, int first, int nlimbs, uint64_t seed, uint64_t tag,
                    uint64_t stream0, hipStream_t s);

}  // namespace ckks
