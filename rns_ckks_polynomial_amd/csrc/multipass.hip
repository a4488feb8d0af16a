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
    std::vector<uint64_t> cr((size_t)ntot * n * 2), cri((size_t)ntot * n * 2);
    std::vector<uint64_t> pw(m2);
    for (uint32_t g = 0; g < ntot; g++) {
        const uint64_t q = c->primes[g], psi = c->psi[g];
        pw[0] = 1;
        for (uint32_t e = 1; e < m2; e++) pw[e] = h_mulmod(pw[e - 1], psi, q);  // psi^e, e < 2n
        auto powe = [&](int64_t e) { e %= (int64_t)m2; if (e < 0) e += m2; return pw[(size_t)e]; };
        for (uint32_t k = 0; k < MP_N1; k++) {
            uint32_t r = 0;
            for (uint32_t b = 0; b < MP_LOG1; b++) r |= ((k >> b) & 1) << (MP_LOG1 - 1 - b);
            const uint64_t wf = powe((int64_t)MP_N1 * r), wi = powe(-(int64_t)MP_N1 * r);
            twf[((size_t)g * MP_N1 + k) * 2] = wf;
            twf[((size_t)g * MP_N1 + k) * 2 + 1] = h_shoup(wf, q);
            twi[((size_t)g * MP_N1 + k) * 2] = wi;
            twi[((size_t)g * MP_N1 + k) * 2 + 1] = h_shoup(wi, q);
        }
        for (uint32_t j1 = 0; j1 < MP_N1; j1++)
            for (uint32_t i2 = 0; i2 < MP_N1; i2++) {
                const int64_t e = (int64_t)i2 * (2 * (int64_t)j1 + 1 - (int64_t)MP_N1);
                const uint64_t t = powe(e), ti = powe(-e);
                const size_t a = ((size_t)g * n + (size_t)j1 * MP_N1 + i2) * 2;
                const size_t b = ((size_t)g * n + (size_t)i2 * MP_N1 + j1) * 2;
                cr[a] = t;
                cr[a + 1] = h_shoup(t, q);
                cri[b] = ti;
                cri[b + 1] = h_shoup(ti, q);
            }
    }
    auto up = [&](const std::vector<uint64_t> &h, uint64_t **d) {
        if (hipMalloc((void **)d, h.size() * 8) != hipSuccess) return CKKS_ENOMEM;
        mp->owned.push_back(*d);
        return hipMemcpy(*d, h.data(), h.size() * 8, hipMemcpyHostToDevice) == hipSuccess ? CKKS_OK : CKKS_EHIP;
    };
    int e;
    if ((e = up(twf, &mp->d_tw256f)) || (e = up(twi, &mp->d_tw256i)) || (e = up(cr, &mp->d_cross)) ||
        (e = up(cri, &mp->d_crossinvT)))
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
