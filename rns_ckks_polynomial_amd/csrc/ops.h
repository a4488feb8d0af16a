// ops.h -- internal launchers (host side) for the hot-path operations.
#pragma once
#include "ctx_internal.h"

namespace ckks {

// NTT of plain strided limbs: [count][nlimbs][n], limb r uses prime first + r.
int op_ntt(const ckks_ctx *c, uint64_t *x, int count, int first, int nlimbs, bool inverse, hipStream_t s);

int op_pointwise_mul(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, uint64_t *out, int count, int first,
                     int nlimbs, hipStream_t s);

size_t ws_bytes_relin(const ckks_ctx *c, int B, int l);
size_t ws_bytes_rotate(const ckks_ctx *c, int B, int l);
size_t ws_bytes_rescale(const ckks_ctx *c, int B, int l);
size_t ws_bytes_bsgs(const ckks_ctx *c, int B, int l, int bs, int gs);

int op_mul_tensor_relin(ckks_ctx *c, const uint64_t *a, const uint64_t *b, const uint64_t *rlk, uint64_t *out, int B,
                        int l, void *ws, hipStream_t s);
int op_rescale(ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, void *ws, hipStream_t s);
int op_rotate(ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, uint32_t g, const uint64_t *key, void *ws,
              bool accumulate, hipStream_t s);
int op_bsgs(ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, const uint64_t *diags, int bs, int gs,
            const uint64_t *const *baby, const uint64_t *const *giant, bool rescale, void *ws, hipStream_t s);
// EvalMod (Chebyshev cosine + double angles); levels consumed = eval_mod_depth(degree, double_angles).
int eval_mod_depth(int degree, int double_angles);
size_t ws_bytes_eval_mod(const ckks_ctx *c, int B, int l, int degree);
int op_eval_mod(ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, double scale_in, const double *cheb,
                int degree, double bound_k, int double_angles, double out_factor, const uint64_t *rlk, void *ws,
                double *scale_out, int *level_out, hipStream_t s);
int op_fill_uniform(const ckks_ctx *c, uint64_t *dst, int count, int first, int nlimbs, uint64_t seed, uint64_t tag,
                    uint64_t stream0, hipStream_t s);

}  // namespace ckks
