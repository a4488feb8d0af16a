// bootstrap.hip -- ciphertext refresh, the stage sequence of the boot profile
// in the Kestrel article (section 5.3): modraise -> coeff_to_slot ->
// conj_extract -> sin_fold (real and imaginary parts) -> restore_merge ->
// slot_to_coeff.  Every stage runs on the GPU through the library's own
// operations; this file only sequences them and lays out the workspace.
#include <algorithm>

#include "../../include/ckks_gpu.h"
#include "ops.h"

namespace ckks {

namespace {
inline size_t ct_bytes(const ckks_ctx *c, int B, int l) {
    return (((size_t)B * 2 * l * c->n * 8) + 255) & ~(size_t)255;
}
struct BootLayout {
    int lt, l_ri, l_em, l_out, depth;
    size_t r, w, cj, x, ri, em, v, stage;  // byte sizes
    size_t total() const { return r + w + cj + x + ri + em + v + stage; }
};
BootLayout boot_layout(const ckks_ctx *c, int B, int l0, const ckks_boot_params *p) {
    BootLayout L{};
    L.lt = p->level_raise;
    L.depth = eval_mod_depth(p->degree, p->double_angles);
    L.l_ri = L.lt - 2;             // after CtS (1 level) and the conj_extract constant (1 level)
    L.l_em = L.l_ri - L.depth;     // after EvalMod
    L.l_out = L.l_em - 1;          // after StC
    L.r = ct_bytes(c, B, L.lt);
    L.w = L.cj = ct_bytes(c, B, L.lt - 1);
    L.x = ct_bytes(c, 2 * B, L.lt - 1);
    L.ri = ct_bytes(c, 2 * B, L.l_ri);
    L.em = ct_bytes(c, 2 * B, L.l_em);
    L.v = ct_bytes(c, B, L.l_em);
    L.stage = std::max({ws_bytes_mod_raise(c, B, l0), ws_bytes_bsgs(c, B, L.lt, p->bs, p->gs),
                        ws_bytes_rotate(c, B, L.lt - 1), ws_bytes_rescale(c, 2 * B, L.lt - 1),
                        ws_bytes_eval_mod(c, 2 * B, L.l_ri, p->degree),
                        ws_bytes_bsgs(c, B, L.l_em, p->bs, p->gs)});
    return L;
}
}  // namespace

int boot_levels(const ckks_boot_params *p, int *l_out) {
    *l_out = p->level_raise - 3 - eval_mod_depth(p->degree, p->double_angles);
    return CKKS_OK;
}

size_t ws_bytes_bootstrap(const ckks_ctx *c, int B, int l0, const ckks_boot_params *p) {
    return boot_layout(c, B, l0, p).total();
}

int op_bootstrap(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l0, const ckks_boot_params *p,
                 void *ws, double *scale_mid, hipStream_t s) {
    const BootLayout L = boot_layout(c, B, l0, p);
    uint8_t *base = (uint8_t *)ws;
    auto take = [&](size_t bytes) {
        uint64_t *q = (uint64_t *)base;
        base += bytes;
        return q;
    };
    uint64_t *R = take(L.r), *W = take(L.w), *Cj = take(L.cj), *X = take(L.x), *RI = take(L.ri), *EM = take(L.em),
             *V = take(L.v), *stage = take(L.stage);
    const size_t half_x = (size_t)B * 2 * (L.lt - 1) * c->n;
    int e;
    // modraise: l0 -> lt primes
    if ((e = op_mod_raise(c, in, R, B, l0, L.lt, stage, s))) return e;
    // coeff_to_slot: BSGS with rescale (lt -> lt - 1); slots w = t_lo + i t_hi
    if ((e = op_bsgs(c, R, W, B, L.lt, p->cts_diags, p->bs, p->gs, p->baby_keys, p->giant_keys, true, stage, s)))
        return e;
    // conj_extract: re = (w + conj w) / 2, im = (w - conj w) X^(n/2) (-1/2)
    if ((e = op_rotate(c, W, Cj, B, L.lt - 1, 2 * c->n - 1, p->conj_key, stage, false, s))) return e;
    if ((e = op_lincomb(c, X, L.lt - 1, W, L.lt - 1, Cj, L.lt - 1, 1, 1, 0, false, B, s))) return e;
    if ((e = op_lincomb(c, X + half_x, L.lt - 1, W, L.lt - 1, Cj, L.lt - 1, 1, -1, 0, false, B, s))) return e;
    if ((e = op_lincomb(c, X + half_x, L.lt - 1, X + half_x, L.lt - 1, X + half_x, L.lt - 1, 0, 1, 0, true, B, s)))
        return e;
    bool ok = true;
    const double qd = (double)c->primes[L.lt - 2];
    if ((e = op_lincomb(c, X, L.lt - 1, X, L.lt - 1, nullptr, 0, enc_const(0.5, qd, &ok), 0, 0, false, B, s)))
        return e;
    if ((e = op_lincomb(c, X + half_x, L.lt - 1, X + half_x, L.lt - 1, nullptr, 0, enc_const(-0.5, qd, &ok), 0, 0,
                        false, B, s)))
        return e;
    if ((e = op_rescale(c, X, RI, 2 * B, L.lt - 1, stage, s))) return e;
    // sin_fold of both parts in one EvalMod call (2B ciphertexts)
    double s_em = 0;
    int l_em = 0;
    if ((e = op_eval_mod(c, RI, EM, 2 * B, L.l_ri, p->evalmod_scale, p->cheb, p->degree, p->bound_k,
                         p->double_angles, p->out_factor, p->rlk, stage, &s_em, &l_em, s)))
        return e;
    // restore_merge: v = re' + im' X^(n/2)
    const size_t half_em = (size_t)B * 2 * l_em * c->n;
    if ((e = op_lincomb(c, V, l_em, EM, l_em, EM + half_em, l_em, 1, 1, 0, true, B, s))) return e;
    // slot_to_coeff: BSGS with rescale (l_em -> l_em - 1)
    if ((e = op_bsgs(c, V, out, B, l_em, p->stc_diags, p->bs, p->gs, p->baby_keys, p->giant_keys, true, stage, s)))
        return e;
    if (!ok) return CKKS_EINVAL;
    if (scale_mid) *scale_mid = s_em;
    return CKKS_OK;
}

}  // namespace ckks
