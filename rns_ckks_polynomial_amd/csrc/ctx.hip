// ctx.hip -- context creation: chain primes, roots, twiddles and exact
// base-conversion tables, generated on the host and kept resident in HBM.
#include <string.h>

#include <algorithm>
#include <new>

#include "ctx_internal.h"
#include "multipass.h"
#include "ops.h"

namespace ckks {

uint64_t h_mulmod(uint64_t a, uint64_t b, uint64_t q) { return host::mulmod(a, b, q); }
uint64_t h_powmod(uint64_t a, uint64_t e, uint64_t q) { return host::powmod(a, e, q); }
uint64_t h_invmod(uint64_t a, uint64_t q) { return host::invmod(a, q); }
uint64_t h_shoup(uint64_t w, uint64_t q) { return host::shoup(w, q); }

template <class T>
static T *dev_upload(const std::vector<T> &h, std::vector<void *> &owned, int *err) {
    T *d = nullptr;
    if (hipMalloc((void **)&d, std::max<size_t>(h.size(), 1) * sizeof(T)) != hipSuccess) {
        *err = CKKS_ENOMEM;
        return nullptr;
    }
    owned.push_back(d);
    if (!h.empty() && hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) {
        *err = CKKS_EHIP;
        return nullptr;
    }
    return d;
}

int build_basis(ckks_ctx *ctx, uint32_t first, uint32_t m, BasisDev *out, std::vector<void *> &owned,
                bool chain_targets, std::vector<uint64_t> *inv_hat_host) {
    host::BasisTables t;
    host::basis_tables(ctx->primes, ctx->L, ctx->K, first, m, chain_targets, t);
    int err = CKKS_OK;
    BasisDev d{};
    d.m = m;
    d.first = first;
    d.ntot = ctx->L + ctx->K;
    d.mk = t.mk;
    d.HD = dev_upload(t.HD, owned, &err);
    d.RC = dev_upload(t.RC, owned, &err);
    d.inv_hat = dev_upload(t.inv_hat, owned, &err);
    d.hat_mod = dev_upload(t.hat_mod, owned, &err);
    d.R = dev_upload(t.R, owned, &err);
    d.garner = dev_upload(t.garner, owned, &err);
    d.half = dev_upload(t.half, owned, &err);
    *out = d;
    if (inv_hat_host) *inv_hat_host = t.inv_hat;
    return err;
}

// n^-1 [Bhat_i^-1]_{q_i} (Shoup pairs) for the primes i of a basis, from its host inverses.
static void scaled_inv_hat(const ckks_ctx *ctx, uint32_t first, uint32_t m, const std::vector<uint64_t> &ih,
                           uint64_t *dst) {
    for (uint32_t i = 0; i < m; i++) {
        const uint64_t q = ctx->primes[first + i], v = h_mulmod(h_invmod(ctx->n % q, q), ih[2 * i], q);
        dst[2 * i] = v;
        dst[2 * i + 1] = h_shoup(v, q);
    }
}

int prepare_level(ckks_ctx *ctx, uint32_t l) {
    if (ctx->levels.count(l)) return CKKS_OK;
    LevelTables *lt = new LevelTables();
    lt->l = l;
    int err = CKKS_OK;
    if (ctx->K > 0) {
        lt->beta = (l + ctx->alpha - 1) / ctx->alpha;
        std::vector<uint64_t> sc(2 * l);
        for (uint32_t j = 0; j < lt->beta && !err; j++) {
            const uint32_t lo = j * ctx->alpha, hi = std::min(l, lo + ctx->alpha);
            std::vector<uint64_t> ih;
            if (hi - lo == ctx->full_digits[j].m) {
                lt->h_digits.push_back(ctx->full_digits[j]);
                ih = ctx->full_inv_hat[j];
            } else {
                BasisDev bd{};
                err = build_basis(ctx, lo, hi - lo, &bd, lt->owned, false, &ih);
                lt->h_digits.push_back(bd);
            }
            if (!err) scaled_inv_hat(ctx, lo, hi - lo, ih, sc.data() + 2 * lo);
        }
        if (!err) lt->d_digits = dev_upload(lt->h_digits, lt->owned, &err);
        if (!err) lt->d_modup_scale = dev_upload(sc, lt->owned, &err);
    }
    if (!err && l >= 2) {
        std::vector<uint64_t> ri(2 * (l - 1));
        const uint64_t ql = ctx->primes[l - 1];
        for (uint32_t i = 0; i + 1 < l; i++) {
            const uint64_t q = ctx->primes[i], v = h_invmod(ql % q, q);
            ri[2 * i] = v;
            ri[2 * i + 1] = h_shoup(v, q);
        }
        lt->d_rescale_inv = dev_upload(ri, lt->owned, &err);
    }
    if (err != CKKS_OK) {
        for (void *p : lt->owned) hipFree(p);
        delete lt;
        return err;
    }
    ctx->levels[l] = lt;
    return CKKS_OK;
}

int prepare_raise(ckks_ctx *ctx, uint32_t l0) {
    if (ctx->raise.count(l0)) return CKKS_OK;
    RaiseTables *rt = new RaiseTables();
    BasisDev bd{};
    std::vector<uint64_t> ih;
    int err = build_basis(ctx, 0, l0, &bd, rt->owned, true, &ih);
    std::vector<uint64_t> sc(2 * l0);
    if (!err) scaled_inv_hat(ctx, 0, l0, ih, sc.data());
    std::vector<BasisDev> one(1, bd);
    if (!err) rt->d_basis = dev_upload(one, rt->owned, &err);
    if (!err) rt->d_scale = dev_upload(sc, rt->owned, &err);
    if (err != CKKS_OK) {
        for (void *p : rt->owned) hipFree(p);
        delete rt;
        return err;
    }
    ctx->raise[l0] = rt;
    return CKKS_OK;
}

const LevelTables *find_level(const ckks_ctx *ctx, uint32_t l) {
    auto it = ctx->levels.find(l);
    return it == ctx->levels.end() ? nullptr : it->second;
}
const RaiseTables *find_raise(const ckks_ctx *ctx, uint32_t l0) {
    auto it = ctx->raise.find(l0);
    return it == ctx->raise.end() ? nullptr : it->second;
}

}  // namespace ckks

using namespace ckks;

extern "C" int ckks_ctx_create(ckks_ctx **out, const ckks_params *params, int device) {
    if (!out || !params) return CKKS_EINVAL;
    *out = nullptr;
    const ckks_params p = *params;
    if (p.n != 2048 && p.n != 65536) return CKKS_EUNSUPPORTED;
    if (p.L < 1 || p.L > 4096 || p.K > 4096) return CKKS_EINVAL;
    if (p.K > 0 && (p.dnum < 1 || p.dnum > p.L)) return CKKS_EINVAL;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return CKKS_EHIP;
    int dev_saved = 0;
    hipGetDevice(&dev_saved);
    if (hipSetDevice(device) != hipSuccess) return CKKS_EHIP;

    ckks_ctx *c = new (std::nothrow) ckks_ctx();
    if (!c) return CKKS_ENOMEM;
    c->n = p.n; c->L = p.L; c->K = p.K; c->dnum = p.K ? p.dnum : 1; c->device = device;
    c->alpha = (p.L + c->dnum - 1) / c->dnum;
    while ((1u << c->logn) < p.n) c->logn++;
    const uint32_t ntot = p.L + p.K, n = p.n;
    int err = CKKS_OK;
    if (!host::chain(n, ntot, c->primes)) err = CKKS_EINVAL;
    // the split multiply-accumulate bounds assume every prime is below 2^59 + 2^52,
    // and a base conversion sums at most 1000 products (digit width and K) so
    // that m (2^59 + 2^52)^2 plus the u [-B]_t term stays below 2^128
    if (!err && c->primes.back() >= (1ull << 59) + (1ull << 52)) err = CKKS_EUNSUPPORTED;
    if (!err && (c->alpha > 1000 || p.K > 1000)) err = CKKS_EUNSUPPORTED;
    if (!err) {
        c->psi.resize(ntot);
        std::vector<PrimeConsts> pc(ntot);
        std::vector<uint64_t> twf((size_t)ntot * n * 2), twi((size_t)ntot * n * 2), iota(ntot);
        for (uint32_t g = 0; g < ntot; g++) {
            c->psi[g] = host::min_root(n, c->primes[g]);
            host::prime_tables(n, c->primes[g], c->psi[g], pc[g], twf.data() + (size_t)g * n * 2,
                               twi.data() + (size_t)g * n * 2, iota[g]);
            if (n == 2048) host::ntt2048_twiddle_order(twf.data() + (size_t)g * n * 2, twi.data() + (size_t)g * n * 2);
        }
        c->d_pc = dev_upload(pc, c->owned, &err);
        c->d_tw_fwd = dev_upload(twf, c->owned, &err);
        c->d_tw_inv = dev_upload(twi, c->owned, &err);
        c->d_iota = dev_upload(iota, c->owned, &err);
        std::vector<uint64_t> prc((size_t)ntot * MF_RC);
        for (uint32_t g = 0; g < ntot; g++) host::recomb_row(c->primes[g], prc.data() + (size_t)g * MF_RC);
        c->d_prc = dev_upload(prc, c->owned, &err);
    }
    if (!err && p.K > 0) {
        // full digits at the top level, the special-prime basis and its constants
        for (uint32_t j = 0; j * c->alpha < p.L && !err; j++) {
            BasisDev bd{};
            std::vector<uint64_t> ih;
            err = build_basis(c, j * c->alpha, std::min(p.L, (j + 1) * c->alpha) - j * c->alpha, &bd, c->owned,
                              false, &ih);
            c->full_digits.push_back(bd);
            c->full_inv_hat.push_back(ih);
        }
        std::vector<uint64_t> ih;
        if (!err) err = build_basis(c, p.L, p.K, &c->h_pbasis, c->owned, false, &ih);
        if (!err) {
            std::vector<BasisDev> one(1, c->h_pbasis);
            c->d_pbasis = dev_upload(one, c->owned, &err);
            std::vector<uint64_t> sc(2 * p.K), pinv(2 * p.L), pmod(p.L);
            scaled_inv_hat(c, p.L, p.K, ih, sc.data());
            for (uint32_t i = 0; i < p.L; i++) {
                uint64_t q = c->primes[i], P = 1;
                for (uint32_t k = 0; k < p.K; k++) P = h_mulmod(P, c->primes[p.L + k] % q, q);
                uint64_t v = h_invmod(P, q);
                pmod[i] = P;
                pinv[2 * i] = v;
                pinv[2 * i + 1] = h_shoup(v, q);
            }
            c->d_moddown_scale = dev_upload(sc, c->owned, &err);
            c->d_pinv = dev_upload(pinv, c->owned, &err);
            c->d_pmod = dev_upload(pmod, c->owned, &err);
        }
    }
    if (!err && n > 2048) err = multipass_init(c);
    if (!err) err = noalloc_init(device);
    if (!err && p.L <= CKKS_PREPARE_ALL_MAX_L) {  // short chains: every level up front
        for (uint32_t l = 1; l <= p.L && !err; l++) err = prepare_level(c, l);
        for (uint32_t l = 1; l <= p.L && l <= 1000 && !err; l++) err = prepare_raise(c, l);
    } else if (!err) {
        err = prepare_level(c, p.L);
    }
    hipSetDevice(dev_saved);
    if (err) {
        ckks_ctx_destroy(c);
        return err;
    }
    *out = c;
    return CKKS_OK;
}

extern "C" void ckks_ctx_destroy(ckks_ctx *c) {
    if (!c) return;
    int dev_saved = 0;
    hipGetDevice(&dev_saved);
    hipSetDevice(c->device);
    hipDeviceSynchronize();
    for (auto &kv : c->levels) {
        for (void *p : kv.second->owned) hipFree(p);
        delete kv.second;
    }
    for (auto &kv : c->raise) {
        for (void *p : kv.second->owned) hipFree(p);
        delete kv.second;
    }
    if (c->mp) multipass_free(c);
    if (c->prof) {
        for (hipEvent_t e : c->prof->pool) (void)hipEventDestroy(e);
        delete c->prof;
    }
    for (void *p : c->owned) hipFree(p);
    hipSetDevice(dev_saved);
    delete c;
}

extern "C" int ckks_prepare_levels(ckks_ctx *c, int lo, int hi) {
    if (!c) return CKKS_EINVAL;
    if (lo < 1 || hi < lo || (uint32_t)hi > c->L) return CKKS_ELEVEL;
    int dev_saved = 0;
    hipGetDevice(&dev_saved);
    if (hipSetDevice(c->device) != hipSuccess) return CKKS_EHIP;
    int err = CKKS_OK;
    for (int l = lo; l <= hi && !err; l++) err = prepare_level(c, (uint32_t)l);
    hipSetDevice(dev_saved);
    return err;
}

extern "C" int ckks_prepare_raise(ckks_ctx *c, int level_in) {
    if (!c) return CKKS_EINVAL;
    if (level_in < 1 || (uint32_t)level_in > c->L || level_in > 1000) return CKKS_ELEVEL;
    int dev_saved = 0;
    hipGetDevice(&dev_saved);
    if (hipSetDevice(c->device) != hipSuccess) return CKKS_EHIP;
    const int err = prepare_raise(c, (uint32_t)level_in);
    hipSetDevice(dev_saved);
    return err;
}

extern "C" int ckks_ctx_primes(const ckks_ctx *c, uint64_t *hp, uint64_t *hpsi) {
    if (!c) return CKKS_EINVAL;
    if (hp) memcpy(hp, c->primes.data(), c->primes.size() * 8);
    if (hpsi) memcpy(hpsi, c->psi.data(), c->psi.size() * 8);
    return CKKS_OK;
}

extern "C" const char *ckks_strerror(int code) {
    switch (code) {
        case CKKS_OK: return "ok";
        case CKKS_EINVAL: return "invalid argument";
        case CKKS_ELEVEL: return "level out of range";
        case CKKS_ENOMEM: return "device allocation failed";
        case CKKS_EHIP: return "HIP runtime error";
        case CKKS_EALIGN: return "misaligned pointer";
        case CKKS_EWORKSPACE: return "workspace too small";
        case CKKS_EUNSUPPORTED: return "unsupported parameters";
        case CKKS_EKEY: return "switching key does not match the context";
        case CKKS_ENOTREADY: return "level tables not prepared";
        default: return "unknown error";
    }
}
