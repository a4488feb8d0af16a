// ctx.hip -- context creation: chain primes, roots, twiddles and exact
// base-conversion tables, generated on the host and kept resident in HBM.
#include <string.h>

#include <algorithm>
#include <new>

#include "ctx_internal.h"
#include "multipass.h"

namespace ckks {

typedef unsigned __int128 h128;

uint64_t h_mulmod(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)((h128)a * b % q); }
uint64_t h_powmod(uint64_t a, uint64_t e, uint64_t q) {
    uint64_t r = 1;
    a %= q;
    for (; e; e >>= 1, a = h_mulmod(a, a, q))
        if (e & 1) r = h_mulmod(r, a, q);
    return r;
}
// modular inverse by the extended Euclidean algorithm
uint64_t h_invmod(uint64_t a, uint64_t q) {
    __int128 t = 0, nt = 1, r = q, nr = a % q;
    while (nr) {
        __int128 qt = r / nr, tmp;
        tmp = t - qt * nt; t = nt; nt = tmp;
        tmp = r - qt * nr; r = nr; nr = tmp;
    }
    if (t < 0) t += q;
    return (uint64_t)t;
}
uint64_t h_shoup(uint64_t w, uint64_t q) { return (uint64_t)(((h128)w << 64) / q); }

// Miller-Rabin with the first 12 prime bases (exact below 3.3e24).
static bool h_is_prime(uint64_t x) {
    static const uint64_t P[12] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
    for (uint64_t p : P)
        if (x % p == 0) return x == p;
    uint64_t d = x - 1;
    int s = 0;
    for (; !(d & 1); d >>= 1) s++;
    for (uint64_t a : P) {
        uint64_t y = h_powmod(a, d, x);
        if (y == 1 || y == x - 1) continue;
        bool ok = false;
        for (int r = 1; r < s && !ok; r++) {
            y = h_mulmod(y, y, x);
            ok = (y == x - 1);
        }
        if (!ok) return false;
    }
    return true;
}

// Chain: the smallest primes in (2^59, 2^60) that are 1 mod 2n, ascending.
static bool h_chain(uint32_t n, uint32_t count, std::vector<uint64_t> &out) {
    out.clear();
    const uint64_t step = 2ull * n;
    for (uint64_t c = (1ull << 59) + 1; c < (1ull << 60) && out.size() < count; c += step)
        if (h_is_prime(c)) out.push_back(c);
    return out.size() == count;
}

// Smallest primitive 2n-th root of unity: any quadratic non-residue z gives
// w = z^((q-1)/2n) with w^n = -1; the odd powers of w are all such roots.
static uint64_t h_min_root(uint32_t n, uint64_t q) {
    uint64_t z = 2;
    while (h_powmod(z, (q - 1) / 2, q) != q - 1) z++;
    uint64_t w = h_powmod(z, (q - 1) / (2ull * n), q), w2 = h_mulmod(w, w, q), best = w, cur = w;
    for (uint32_t k = 0; k < n; k++, cur = h_mulmod(cur, w2, q)) best = std::min(best, cur);
    return best;
}

static uint32_t h_bitrev(uint32_t x, uint32_t bits) {
    uint32_t r = 0;
    for (uint32_t i = 0; i < bits; i++, x >>= 1) r = (r << 1) | (x & 1);
    return r;
}

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

// Little-endian multi-word helpers for (B-1)/2 in mixed radix.
static void big_mul(std::vector<uint64_t> &a, uint64_t m) {
    h128 c = 0;
    for (auto &w : a) {
        h128 t = (h128)w * m + c;
        w = (uint64_t)t;
        c = t >> 64;
    }
    if (c) a.push_back((uint64_t)c);
}
static uint64_t big_divmod(std::vector<uint64_t> &a, uint64_t m) {  // a /= m, returns a mod m
    h128 r = 0;
    for (size_t i = a.size(); i-- > 0;) {
        h128 cur = (r << 64) | a[i];
        a[i] = (uint64_t)(cur / m);
        r = cur % m;
    }
    while (a.size() > 1 && a.back() == 0) a.pop_back();
    return (uint64_t)r;
}

int build_basis(ckks_ctx *ctx, uint32_t first, uint32_t m, BasisDev *out, std::vector<void *> &owned,
                bool chain_targets) {
    const uint32_t ntot = ctx->L + ctx->K;
    const uint64_t *b = ctx->primes.data() + first;
    std::vector<uint64_t> inv_hat(2 * m), hat_mod(2 * m), R(m), H((size_t)ntot * m), negB(ntot),
        garner((size_t)2 * m * m, 0), half(m);
    // [Bhat_i]_t by prefix/suffix products, for every chain prime t
    std::vector<uint64_t> pre(m + 1), suf(m + 1);
    for (uint32_t t = 0; t < ntot; t++) {
        uint64_t qt = ctx->primes[t];
        pre[0] = 1;
        for (uint32_t i = 0; i < m; i++) pre[i + 1] = h_mulmod(pre[i], b[i] % qt, qt);
        suf[m] = 1;
        for (uint32_t i = m; i-- > 0;) suf[i] = h_mulmod(suf[i + 1], b[i] % qt, qt);
        for (uint32_t i = 0; i < m; i++) H[(size_t)t * m + i] = h_mulmod(pre[i], suf[i + 1], qt);
        negB[t] = (qt - pre[m]) % qt;
    }
    for (uint32_t i = 0; i < m; i++) {
        uint64_t bi = b[i];
        uint64_t hm = H[(size_t)(first + i) * m + i];  // [Bhat_i]_{b_i}
        uint64_t iv = h_invmod(hm, bi);
        inv_hat[2 * i] = iv;
        inv_hat[2 * i + 1] = h_shoup(iv, bi);
        hat_mod[2 * i] = hm;
        hat_mod[2 * i + 1] = h_shoup(hm, bi);
        R[i] = (uint64_t)(((h128)1 << 123) / bi);
        for (uint32_t k = 0; k < i; k++) {
            uint64_t v = h_invmod(b[k] % bi, bi);
            garner[((size_t)k * m + i) * 2] = v;
            garner[((size_t)k * m + i) * 2 + 1] = h_shoup(v, bi);
        }
    }
    // mixed-radix digits of (B - 1) / 2:  h = d_0 + d_1 b_0 + d_2 b_0 b_1 + ...
    std::vector<uint64_t> B(1, 1);
    for (uint32_t i = 0; i < m; i++) big_mul(B, b[i]);
    {  // B - 1 then halve (B odd)
        size_t i = 0;
        while (B[i] == 0) B[i++] = ~0ull;
        B[i] -= 1;
        uint64_t carry = 0;
        for (size_t j = B.size(); j-- > 0;) {
            uint64_t nc = B[j] & 1;
            B[j] = (B[j] >> 1) | (carry << 63);
            carry = nc;
        }
    }
    for (uint32_t i = 0; i < m; i++) half[i] = big_divmod(B, b[i]);

    // target positions (see BasisDev)
    std::vector<uint32_t> pos;  // position -> target prime
    if (first < ctx->L && !chain_targets) {
        for (uint32_t t = ctx->L; t < ntot; t++) pos.push_back(t);
        for (uint32_t t = 0; t < ctx->L; t++)
            if (t < first || t >= first + m) pos.push_back(t);
    } else {
        for (uint32_t t = 0; t < ctx->L; t++) pos.push_back(t);
    }
    // digit tables and reduction constants of the conversion (see BasisDev)
    const uint32_t mk = (m + 1 + 31) / 32 * 32, npos = (uint32_t)pos.size(), npad = (npos + 31) / 32 * 32;
    std::vector<int8_t> hd((size_t)npad * 8 * mk, 0);
    std::vector<uint64_t> rc((size_t)npad * MF_RC, 0);
    for (uint32_t p = 0; p < npos; p++) {
        const uint32_t t = pos[p];
        const uint64_t qt = ctx->primes[t];
        for (uint32_t r = 0; r <= m; r++) {
            const uint64_t v = digit_form(r < m ? H[(size_t)t * m + r] : negB[t]);
            for (uint32_t b = 0; b < 8; b++) hd[((size_t)p * 8 + b) * mk + r] = (int8_t)(uint8_t)(v >> (8 * b));
        }
        uint64_t *row = rc.data() + (size_t)p * MF_RC;
        uint64_t w = h_powmod(2, 64, qt);  // 256^8 mod t
        for (uint32_t s2 = 0; s2 < 7; s2++) {
            row[s2] = (w & ((1ull << 30) - 1)) | ((w >> 30) << 32);
            w = h_mulmod(w, 256, qt);
        }
        row[7] = h_powmod(2, 60, qt);
        row[8] = h_shoup(row[7], qt);
        row[9] = qt;
        row[10] = 8 * qt - h_powmod(2, 91, qt);
    }
    int err = CKKS_OK;
    BasisDev d{};
    d.m = m;
    d.first = first;
    d.ntot = ntot;
    d.mk = mk;
    d.HD = dev_upload(hd, owned, &err);
    d.RC = dev_upload(rc, owned, &err);
    d.inv_hat = dev_upload(inv_hat, owned, &err);
    d.hat_mod = dev_upload(hat_mod, owned, &err);
    d.R = dev_upload(R, owned, &err);
    d.garner = dev_upload(garner, owned, &err);
    d.half = dev_upload(half, owned, &err);
    *out = d;
    return err;
}

LevelTables *level_tables(ckks_ctx *ctx, uint32_t l, int *err) {
    std::lock_guard<std::mutex> g(ctx->mu);
    auto it = ctx->levels.find(l);
    if (it != ctx->levels.end()) return it->second;
    int dev_saved = 0;
    hipGetDevice(&dev_saved);
    hipSetDevice(ctx->device);
    LevelTables *lt = new LevelTables();
    lt->l = l;
    *err = CKKS_OK;
    if (ctx->K > 0) {
        lt->beta = (l + ctx->alpha - 1) / ctx->alpha;
        for (uint32_t j = 0; j < lt->beta; j++) {
            uint32_t lo = j * ctx->alpha, hi = std::min(l, lo + ctx->alpha);
            if (hi - lo == ctx->full_digits[j].m) {
                lt->h_digits.push_back(ctx->full_digits[j]);
            } else {
                BasisDev bd{};
                int e = build_basis(ctx, lo, hi - lo, &bd, lt->owned);
                if (e) *err = e;
                lt->h_digits.push_back(bd);
            }
        }
        lt->d_digits = dev_upload(lt->h_digits, lt->owned, err);
        // n^-1 [Bhat_i^-1]_{q_i} for the digit that contains prime i
        std::vector<uint64_t> sc(2 * l);
        for (uint32_t j = 0; j < lt->beta; j++) {
            const BasisDev &bd = lt->h_digits[j];
            std::vector<uint64_t> ih(2 * bd.m);
            hipMemcpy(ih.data(), bd.inv_hat, ih.size() * 8, hipMemcpyDeviceToHost);
            for (uint32_t i = 0; i < bd.m; i++) {
                uint32_t gidx = bd.first + i;
                uint64_t q = ctx->primes[gidx];
                uint64_t v = h_mulmod(h_invmod(ctx->n % q, q), ih[2 * i], q);
                sc[2 * gidx] = v;
                sc[2 * gidx + 1] = h_shoup(v, q);
            }
        }
        lt->d_modup_scale = dev_upload(sc, lt->owned, err);
    }
    if (l >= 2) {
        std::vector<uint64_t> ri(2 * (l - 1));
        uint64_t ql = ctx->primes[l - 1];
        for (uint32_t i = 0; i + 1 < l; i++) {
            uint64_t q = ctx->primes[i], v = h_invmod(ql % q, q);
            ri[2 * i] = v;
            ri[2 * i + 1] = h_shoup(v, q);
        }
        lt->d_rescale_inv = dev_upload(ri, lt->owned, err);
    }
    hipSetDevice(dev_saved);
    if (*err != CKKS_OK) {
        for (void *p : lt->owned) hipFree(p);
        delete lt;
        return nullptr;
    }
    ctx->levels[l] = lt;
    return lt;
}

RaiseTables *raise_tables(ckks_ctx *ctx, uint32_t l0, int *err) {
    std::lock_guard<std::mutex> g(ctx->mu);
    auto it = ctx->raise.find(l0);
    if (it != ctx->raise.end()) return it->second;
    int dev_saved = 0;
    hipGetDevice(&dev_saved);
    hipSetDevice(ctx->device);
    RaiseTables *rt = new RaiseTables();
    BasisDev bd{};
    *err = build_basis(ctx, 0, l0, &bd, rt->owned, true);
    std::vector<uint64_t> ih(2 * l0), sc(2 * l0);
    if (!*err) hipMemcpy(ih.data(), bd.inv_hat, ih.size() * 8, hipMemcpyDeviceToHost);
    for (uint32_t i = 0; i < l0; i++) {
        const uint64_t q = ctx->primes[i], v = h_mulmod(h_invmod(ctx->n % q, q), ih[2 * i], q);
        sc[2 * i] = v;
        sc[2 * i + 1] = h_shoup(v, q);
    }
    std::vector<BasisDev> one(1, bd);
    if (!*err) rt->d_basis = dev_upload(one, rt->owned, err);
    if (!*err) rt->d_scale = dev_upload(sc, rt->owned, err);
    hipSetDevice(dev_saved);
    if (*err != CKKS_OK) {
        for (void *p : rt->owned) hipFree(p);
        delete rt;
        return nullptr;
    }
    ctx->raise[l0] = rt;
    return rt;
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
    if (!h_chain(n, ntot, c->primes)) err = CKKS_EINVAL;
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
            const uint64_t q = c->primes[g];
            const uint64_t psi = h_min_root(n, q), ipsi = h_invmod(psi, q);
            c->psi[g] = psi;
            PrimeConsts &k = pc[g];
            k.q = q;
            k.mu = (uint64_t)(((h128)1 << 122) / q);
            k.r64 = (uint64_t)(((h128)1 << 64) % q);
            k.r64p = h_shoup(k.r64, q);
            k.m64 = (uint64_t)(((h128)1 << 64) / q);
            k.ninv = h_invmod(n % q, q);
            k.ninvp = h_shoup(k.ninv, q);
            k.r60 = (1ull << 60) % q;
            k.r60p = h_shoup(k.r60, q);
            // powers psi^e for e = 0..n-1, then place at bit-reversed slots
            uint64_t pw = 1, ipw = 1;
            std::vector<uint64_t> fp(n), ip(n);
            for (uint32_t e = 0; e < n; e++, pw = h_mulmod(pw, psi, q), ipw = h_mulmod(ipw, ipsi, q)) {
                fp[e] = pw;
                ip[e] = ipw;
            }
            iota[g] = fp[n / 2];  // psi^(n/2): a square root of -1
            uint64_t *tf = twf.data() + (size_t)g * n * 2, *ti = twi.data() + (size_t)g * n * 2;
            for (uint32_t k2 = 0; k2 < n; k2++) {
                uint32_t e = h_bitrev(k2, c->logn);
                tf[2 * k2] = fp[e];
                tf[2 * k2 + 1] = h_shoup(fp[e], q);
                ti[2 * k2] = ip[e];
                ti[2 * k2 + 1] = h_shoup(ip[e], q);
            }
        }
        c->d_pc = dev_upload(pc, c->owned, &err);
        c->d_tw_fwd = dev_upload(twf, c->owned, &err);
        c->d_tw_inv = dev_upload(twi, c->owned, &err);
        c->d_iota = dev_upload(iota, c->owned, &err);
    }
    if (!err && p.K > 0) {
        // full digits at the top level, the special-prime basis and its constants
        for (uint32_t j = 0; j * c->alpha < p.L && !err; j++) {
            BasisDev bd{};
            err = build_basis(c, j * c->alpha, std::min(p.L, (j + 1) * c->alpha) - j * c->alpha, &bd, c->owned);
            c->full_digits.push_back(bd);
        }
        if (!err) err = build_basis(c, p.L, p.K, &c->h_pbasis, c->owned);
        if (!err) {
            std::vector<BasisDev> one(1, c->h_pbasis);
            c->d_pbasis = dev_upload(one, c->owned, &err);
            std::vector<uint64_t> ih(2 * p.K);
            hipMemcpy(ih.data(), c->h_pbasis.inv_hat, ih.size() * 8, hipMemcpyDeviceToHost);
            std::vector<uint64_t> sc(2 * p.K), pinv(2 * p.L), pmod(p.L);
            for (uint32_t k = 0; k < p.K; k++) {
                uint64_t q = c->primes[p.L + k], v = h_mulmod(h_invmod(n % q, q), ih[2 * k], q);
                sc[2 * k] = v;
                sc[2 * k + 1] = h_shoup(v, q);
            }
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
        default: return "unknown error";
    }
}
