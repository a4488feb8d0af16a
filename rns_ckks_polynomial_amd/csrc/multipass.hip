// multipass.hip -- host tables of the four-step NTT (see multipass.h).
#include <vector>

#include "multipass.h"

namespace ckks {

int multipass_init(ckks_ctx *c) {
    if (c->n != MP_N1 * MP_N1) return CKKS_EUNSUPPORTED;
    MultipassPlan *mp = new MultipassPlan();
    c->mp = mp;
    const uint32_t ntot = c->L + c->K, n = c->n, m2 = 2 * n;
    std::vector<uint64_t> twf((size_t)ntot * MP_N1 * 2), twi((size_t)ntot * MP_N1 * 2);
    std::vector<uint64_t> taf((size_t)ntot * MP_N1 * 16 * 2), tai(taf.size());
    std::vector<uint64_t> rowf((size_t)ntot * 16 * MP_N1 * 2), rowi(rowf.size());
    std::vector<uint64_t> pw(m2);
    auto brev = [](uint32_t x, uint32_t bits) {
        uint32_t r = 0;
        for (uint32_t b = 0; b < bits; b++) r |= ((x >> b) & 1) << (bits - 1 - b);
        return r;
    };
    for (uint32_t g = 0; g < ntot; g++) {
        const uint64_t q = c->primes[g], psi = c->psi[g];
        pw[0] = 1;
        for (uint32_t e = 1; e < m2; e++) pw[e] = h_mulmod(pw[e - 1], psi, q);  // psi^e, e < 2n
        auto powe = [&](int64_t e) { e %= (int64_t)m2; if (e < 0) e += m2; return pw[(size_t)e]; };
        // a Shoup pair of psi^e at w[2 i], and of psi^-e at wi[2 i]
        auto put = [&](std::vector<uint64_t> &w, std::vector<uint64_t> &wi, size_t i, int64_t e) {
            const uint64_t f = powe(e), r = powe(-e);
            w[2 * i] = f;
            w[2 * i + 1] = h_shoup(f, q);
            wi[2 * i] = r;
            wi[2 * i + 1] = h_shoup(r, q);
        };
        for (uint32_t k = 0; k < MP_N1; k++)
            put(twf, twi, (size_t)g * MP_N1 + k, (int64_t)MP_N1 * brev(k, MP_LOG1));
        for (uint32_t i2 = 0; i2 < MP_N1; i2++)
            for (uint32_t t = 0; t < 16; t++)
                put(taf, tai, ((size_t)g * MP_N1 + i2) * 16 + t, (int64_t)i2 * (2 * (int64_t)t + 1 - (int64_t)MP_N1));
        for (uint32_t k = 0; k < 16; k++)
            for (uint32_t m = 1; m < MP_N1; m++) {
                uint32_t s = 0;
                while ((2u << s) <= m) s++;
                const uint32_t b = m - (1u << s);
                const int64_t e = (int64_t)(128 >> s) * (256 + 32 * (int64_t)k + 512 * (int64_t)brev(b, s));
                put(rowf, rowi, ((size_t)g * 16 + k) * MP_N1 + m, e);
            }
    }
    auto up = [&](const std::vector<uint64_t> &h, uint64_t **d) {
        if (hipMalloc((void **)d, h.size() * 8) != hipSuccess) return CKKS_ENOMEM;
        mp->owned.push_back(*d);
        return hipMemcpy(*d, h.data(), h.size() * 8, hipMemcpyHostToDevice) == hipSuccess ? CKKS_OK : CKKS_EHIP;
    };
    int e;
    if ((e = up(twf, &mp->d_tw256f)) || (e = up(twi, &mp->d_tw256i)) || (e = up(taf, &mp->d_taf)) ||
        (e = up(tai, &mp->d_tai)) || (e = up(rowf, &mp->d_rowf)) || (e = up(rowi, &mp->d_rowi)))
        return e;
    if (hipMalloc((void **)&mp->d_scratch, (size_t)MP_CHUNK * n * 8) != hipSuccess) return CKKS_ENOMEM;
    mp->owned.push_back(mp->d_scratch);
    if (hipEventCreateWithFlags(&mp->scratch_done, hipEventDisableTiming) != hipSuccess) return CKKS_EHIP;
    return CKKS_OK;
}

void multipass_free(ckks_ctx *c) {
    if (!c->mp) return;
    if (c->mp->scratch_done) (void)hipEventDestroy(c->mp->scratch_done);
    for (void *p : c->mp->owned) (void)hipFree(p);
    delete c->mp;
    c->mp = nullptr;
}

}  // namespace ckks
