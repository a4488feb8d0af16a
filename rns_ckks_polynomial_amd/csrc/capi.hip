// capi.hip -- the extern "C" entry points: argument validation, then launch.
#include <cmath>

#include "../../include/ckks_gpu.h"
#include "../../include/ckks_synth.h"
#include "ctx_internal.h"
#include "ops.h"

using namespace ckks;

namespace {
inline bool aligned(const void *p) { return ((uintptr_t)p & 7) == 0; }
struct DeviceGuard {
    int saved = 0;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        hipGetDevice(&saved);
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() { hipSetDevice(saved); }
};
int check_ptr(const void *p) {
    if (!p) return CKKS_EINVAL;
    if (!aligned(p)) return CKKS_EALIGN;
    return CKKS_OK;
}
int check_level(const ckks_ctx *c, int batch, int level, int min_level) {
    if (batch < 1) return CKKS_EINVAL;
    if (level < min_level || (uint32_t)level > c->L) return CKKS_ELEVEL;
    return CKKS_OK;
}
// every level in [lo, hi] prepared
int check_ready(const ckks_ctx *c, int lo, int hi) {
    for (int l = lo; l <= hi; l++)
        if (!find_level(c, (uint32_t)l)) return CKKS_ENOTREADY;
    return CKKS_OK;
}
// a switching-key descriptor made for this context's parameter set
int check_key(const ckks_ctx *c, const ckks_swk *k, bool allow_seeded) {
    if (!k) return CKKS_EINVAL;
    int e = check_ptr(k->data);
    if (e) return e;
    if (k->n != c->n || k->L != c->L || k->K != c->K || k->dnum != c->dnum || k->seeded > 1 || k->reserved)
        return CKKS_EKEY;
    if (k->seeded && !allow_seeded) return CKKS_EKEY;
    return CKKS_OK;
}
size_t key_bytes(const ckks_ctx *c, const ckks_swk *k) {
    return (size_t)c->dnum * (k->seeded ? 1 : 2) * (c->L + c->K) * c->n * 8;
}
// the byte ranges [a, a + na) and [b, b + nb) intersect
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}
size_t ct_bytes(const ckks_ctx *c, int batch, int level) { return (size_t)batch * 2 * level * c->n * 8; }
}  // namespace

extern "C" int ckks_workspace_size(const ckks_ctx *c, int op, int batch, int level, int bs, int gs, size_t *bytes) {
    if (!c || !bytes || batch < 1) return CKKS_EINVAL;
    if (level < 1 || (uint32_t)level > c->L) return CKKS_ELEVEL;
    switch (op) {
        case CKKS_OP_RELIN:
            if (!c->K) return CKKS_EINVAL;
            *bytes = ws_bytes_relin(c, batch, level);
            return CKKS_OK;
        case CKKS_OP_ROTATE:
            if (!c->K) return CKKS_EINVAL;
            *bytes = ws_bytes_rotate(c, batch, level);
            return CKKS_OK;
        case CKKS_OP_RESCALE:
            if (level < 2) return CKKS_ELEVEL;
            *bytes = ws_bytes_rescale(c, batch, level);
            return CKKS_OK;
        case CKKS_OP_MODRAISE:
            *bytes = ws_bytes_mod_raise(c, batch, level);
            return CKKS_OK;
        case CKKS_OP_EVALMOD:
            if (!c->K || bs < 1 || bs > 1024) return CKKS_EINVAL;
            *bytes = ws_bytes_eval_mod(c, batch, level, bs);
            return CKKS_OK;
        case CKKS_OP_BSGS:
            if (!c->K || bs < 1 || gs < 1) return CKKS_EINVAL;
            if (level < 2) return CKKS_ELEVEL;
            *bytes = ws_bytes_bsgs(c, batch, level, bs, gs);
            return CKKS_OK;
        default:
            return CKKS_EINVAL;
    }
}

static int ntt_common(const ckks_ctx *c, uint64_t *x, int count, int first, int nlimbs, void *stream, bool inv) {
    if (!c) return CKKS_EINVAL;
    if (count < 0 || nlimbs < 0 || first < 0 || (uint64_t)first + nlimbs > c->L + c->K) return CKKS_EINVAL;
    if (count == 0 || nlimbs == 0) return CKKS_OK;
    int e = check_ptr(x);
    if (e) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_ntt(c, x, count, first, nlimbs, inv, (hipStream_t)stream);
}

extern "C" int ckks_ntt_fwd(const ckks_ctx *c, uint64_t *x, int count, int first, int nlimbs, void *stream) {
    return ntt_common(c, x, count, first, nlimbs, stream, false);
}
extern "C" int ckks_ntt_inv(const ckks_ctx *c, uint64_t *x, int count, int first, int nlimbs, void *stream) {
    return ntt_common(c, x, count, first, nlimbs, stream, true);
}

extern "C" int ckks_pointwise_mul(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, uint64_t *out, int count,
                                  int first, int nlimbs, void *stream) {
    if (!c) return CKKS_EINVAL;
    int e;
    if (count < 0 || nlimbs < 0 || first < 0 || (uint64_t)first + nlimbs > c->L + c->K) return CKKS_EINVAL;
    if (count == 0 || nlimbs == 0) return CKKS_OK;
    if ((e = check_ptr(a)) || (e = check_ptr(b)) || (e = check_ptr(out))) return e;
    const size_t bytes = (size_t)count * nlimbs * c->n * 8;
    if ((out != a && overlaps(out, bytes, a, bytes)) || (out != b && overlaps(out, bytes, b, bytes)))
        return CKKS_EINVAL;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_pointwise_mul(c, a, b, out, count, first, nlimbs, (hipStream_t)stream);
}

extern "C" int ckks_count_unreduced(const ckks_ctx *c, const uint64_t *x, int count, int first, int nlimbs,
                                    uint32_t *out_count, void *stream) {
    if (!c) return CKKS_EINVAL;
    int e;
    if (count < 0 || nlimbs < 0 || first < 0 || (uint64_t)first + nlimbs > c->L + c->K) return CKKS_EINVAL;
    if ((e = check_ptr(out_count))) return e;  // 4-byte counter: the 8-byte alignment rule holds for it too
    if (count > 0 && nlimbs > 0 && (e = check_ptr(x))) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_count_unreduced(c, x, count, first, nlimbs, out_count, (hipStream_t)stream);
}

extern "C" int ckks_mul_tensor_relin(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, const ckks_swk *rlk,
                                     uint64_t *out, int batch, int level, void *ws, size_t ws_bytes, void *stream) {
    if (!c || !c->K) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(a)) || (e = check_ptr(b)) || (e = check_ptr(out))) return e;
    if ((e = check_key(c, rlk, true))) return e;
    if ((e = check_level(c, batch, level, 1))) return e;
    const size_t cb = ct_bytes(c, batch, level);
    if (overlaps(out, cb, a, cb) || overlaps(out, cb, b, cb)) return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_relin(c, batch, level)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    if ((e = check_ready(c, level, level))) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_mul_tensor_relin(c, a, b, rlk, out, batch, level, ws, (hipStream_t)stream);
}

extern "C" int ckks_rescale(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level, void *ws,
                            size_t ws_bytes, void *stream) {
    if (!c) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(in)) || (e = check_ptr(out))) return e;
    if ((e = check_level(c, batch, level, 2))) return e;
    if (overlaps(out, ct_bytes(c, batch, level - 1), in, ct_bytes(c, batch, level))) return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_rescale(c, batch, level)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    if ((e = check_ready(c, level, level))) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_rescale(c, in, out, batch, level, ws, (hipStream_t)stream);
}

extern "C" int ckks_rotate(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level,
                           uint32_t galois_elt, const ckks_swk *key, void *ws, size_t ws_bytes, void *stream) {
    if (!c || !c->K) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(in)) || (e = check_ptr(out))) return e;
    if ((e = check_key(c, key, true))) return e;
    if ((e = check_level(c, batch, level, 1))) return e;
    if ((galois_elt & 1) == 0 || galois_elt >= 2 * c->n) return CKKS_EINVAL;
    const size_t cb = ct_bytes(c, batch, level);
    if (overlaps(out, cb, in, cb)) return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_rotate(c, batch, level)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    if ((e = check_ready(c, level, level))) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_rotate(c, in, out, batch, level, galois_elt, key, ws, false, (hipStream_t)stream);
}

extern "C" int ckks_key_expand(const ckks_ctx *c, const ckks_swk *key, uint64_t *key_out, void *stream) {
    if (!c || !c->K) return CKKS_EINVAL;
    int e;
    if ((e = check_key(c, key, true)) || (e = check_ptr(key_out))) return e;
    if (!key->seeded) return CKKS_EKEY;
    const size_t out_bytes = (size_t)c->dnum * 2 * (c->L + c->K) * c->n * 8;
    if (overlaps(key->data, key_bytes(c, key), key_out, out_bytes)) return CKKS_EINVAL;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_key_expand(c, key, key_out, (hipStream_t)stream);
}

extern "C" int ckks_bsgs_linear_transform(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level,
                                          const uint64_t *diags, int bs, int gs, const ckks_swk *const *baby_keys,
                                          const ckks_swk *const *giant_keys, int do_rescale, void *ws,
                                          size_t ws_bytes, void *stream) {
    if (!c || !c->K) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(in)) || (e = check_ptr(out)) || (e = check_ptr(diags))) return e;
    if ((e = check_level(c, batch, level, do_rescale ? 2 : 1))) return e;
    if (bs < 1 || gs < 1 || (uint64_t)bs * gs > c->n / 2) return CKKS_EINVAL;
    if ((bs > 1 && !baby_keys) || (gs > 1 && !giant_keys)) return CKKS_EINVAL;
    for (int b = 1; b < bs; b++)
        if ((e = check_key(c, baby_keys[b], false))) return e;
    for (int g = 1; g < gs; g++)
        if ((e = check_key(c, giant_keys[g], false))) return e;
    const size_t ob = ct_bytes(c, batch, level - (do_rescale ? 1 : 0));
    if (overlaps(out, ob, in, ct_bytes(c, batch, level)) ||
        overlaps(out, ob, diags, (size_t)gs * bs * level * c->n * 8))
        return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_bsgs(c, batch, level, bs, gs)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    if ((e = check_ready(c, level, level))) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_bsgs(c, in, out, batch, level, diags, bs, gs, baby_keys, giant_keys, do_rescale != 0, ws,
                   (hipStream_t)stream);
}

extern "C" int ckks_fill_uniform(const ckks_ctx *c, uint64_t *dst, int count, int first, int nlimbs, uint64_t seed,
                                 uint64_t tag, uint64_t stream0, void *stream) {
    if (!c) return CKKS_EINVAL;
    if (count < 0 || nlimbs < 0 || first < 0 || (uint64_t)first + nlimbs > c->L + c->K) return CKKS_EINVAL;
    if (count == 0 || nlimbs == 0) return CKKS_OK;
    int e = check_ptr(dst);
    if (e) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_fill_uniform(c, dst, count, first, nlimbs, seed, tag, stream0, (hipStream_t)stream);
}

extern "C" int ckks_eval_mod(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level,
                             double scale_in, const double *cheb, int degree, double bound_k, int double_angles,
                             double out_factor, const ckks_swk *rlk, void *ws, size_t ws_bytes, double *scale_out,
                             int *level_out, void *stream) {
    if (!c || !c->K || !cheb) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(in)) || (e = check_ptr(out))) return e;
    if ((e = check_key(c, rlk, false))) return e;
    if (degree < 1 || degree > 1024 || double_angles < 0 || double_angles > 64) return CKKS_EINVAL;
    if (!(bound_k >= 0.5 && bound_k < 1e9) || !(scale_in > 0 && scale_in < 0x1p61) ||
        !(std::fabs(out_factor) < 2.0))
        return CKKS_EINVAL;
    for (int k = 0; k <= degree; k++)
        if (!(std::fabs(cheb[k]) < 2.0)) return CKKS_EINVAL;
    const int depth = eval_mod_depth(degree, double_angles);
    if ((e = check_level(c, batch, level, depth + 1))) return e;
    if (out != in && overlaps(out, ct_bytes(c, batch, level - depth), in, ct_bytes(c, batch, level)))
        return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_eval_mod(c, batch, level, degree)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    if ((e = check_ready(c, level - depth + 1, level))) return e;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_eval_mod(c, in, out, batch, level, scale_in, cheb, degree, bound_k,
                       double_angles, out_factor, rlk, ws, scale_out, level_out, (hipStream_t)stream);
}

extern "C" int ckks_mod_raise(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level_in,
                              int level_out, void *ws, size_t ws_bytes, void *stream) {
    if (!c) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(in)) || (e = check_ptr(out))) return e;
    if ((e = check_level(c, batch, level_in, 1))) return e;
    if (level_out < level_in || (uint32_t)level_out > c->L || level_in > 1000) return CKKS_ELEVEL;
    if (overlaps(out, ct_bytes(c, batch, level_out), in, ct_bytes(c, batch, level_in))) return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_mod_raise(c, batch, level_in)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    if (!find_raise(c, (uint32_t)level_in)) return CKKS_ENOTREADY;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    return op_mod_raise(c, in, out, batch, level_in, level_out, ws, (hipStream_t)stream);
}

namespace {
int check_boot(const ckks_ctx *c, int batch, int level_in, const ckks_boot_params *p) {
    if (!c || !c->K || !p || batch < 1) return CKKS_EINVAL;
    int e;
    if ((e = check_ptr(p->cts_diags)) || (e = check_ptr(p->stc_diags))) return e;
    if ((e = check_key(c, p->conj_key, false)) || (e = check_key(c, p->rlk, false))) return e;
    if (p->bs < 1 || p->gs < 1 || (uint64_t)p->bs * p->gs > c->n / 2) return CKKS_EINVAL;
    if ((p->bs > 1 && !p->baby_keys) || (p->gs > 1 && !p->giant_keys)) return CKKS_EINVAL;
    for (int b = 1; b < p->bs; b++)
        if ((e = check_key(c, p->baby_keys[b], false))) return e;
    for (int g = 1; g < p->gs; g++)
        if ((e = check_key(c, p->giant_keys[g], false))) return e;
    if (!p->cheb || p->degree < 1 || p->degree > 1024 || p->double_angles < 0 || p->double_angles > 64)
        return CKKS_EINVAL;
    if (!(p->bound_k >= 0.5 && p->bound_k < 1e9) || !(p->evalmod_scale > 0 && p->evalmod_scale < 0x1p61) ||
        !(std::fabs(p->out_factor) < 2.0))
        return CKKS_EINVAL;
    for (int k = 0; k <= p->degree; k++)
        if (!(std::fabs(p->cheb[k]) < 2.0)) return CKKS_EINVAL;
    if (level_in < 1 || level_in > 1000 || level_in > p->level_raise || (uint32_t)p->level_raise > c->L)
        return CKKS_ELEVEL;
    int lo = 0;
    boot_levels(p, &lo);
    if (lo < 1) return CKKS_ELEVEL;
    if (!find_raise(c, (uint32_t)level_in)) return CKKS_ENOTREADY;
    return check_ready(c, lo + 1, p->level_raise);
}
}  // namespace

extern "C" int ckks_bootstrap_workspace_size(const ckks_ctx *c, int batch, int level_in,
                                             const ckks_boot_params *p, size_t *bytes) {
    int e;
    if (!bytes) return CKKS_EINVAL;
    if ((e = check_boot(c, batch, level_in, p))) return e;
    *bytes = ws_bytes_bootstrap(c, batch, level_in, p);
    return CKKS_OK;
}

extern "C" int ckks_bootstrap(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level_in,
                              const ckks_boot_params *p, void *ws, size_t ws_bytes, double *scale_mid,
                              int *level_out, void *stream) {
    int e;
    if ((e = check_boot(c, batch, level_in, p))) return e;
    if ((e = check_ptr(in)) || (e = check_ptr(out))) return e;
    int lo = 0;
    boot_levels(p, &lo);
    if (overlaps(out, ct_bytes(c, batch, lo), in, ct_bytes(c, batch, level_in))) return CKKS_EINVAL;
    if (!ws || ws_bytes < ws_bytes_bootstrap(c, batch, level_in, p)) return CKKS_EWORKSPACE;
    if (!aligned(ws)) return CKKS_EALIGN;
    DeviceGuard g(c->device);
    if (!g.ok) return CKKS_EHIP;
    if (level_out) *level_out = lo;
    return op_bootstrap(c, in, out, batch, level_in, p, ws, scale_mid, (hipStream_t)stream);
}
