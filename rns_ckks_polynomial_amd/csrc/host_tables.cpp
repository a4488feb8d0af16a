// host_tables.cpp -- host-side number theory and constant tables (see host_tables.h).
#include "host_tables.h"

#include <algorithm>

namespace ckks {
namespace host {

typedef unsigned __int128 h128;

uint64_t mulmod(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)((h128)a * b % q); }
uint64_t powmod(uint64_t a, uint64_t e, uint64_t q) {
    uint64_t r = 1 % q;
    a %= q;
    for (; e; e >>= 1, a = mulmod(a, a, q))
        if (e & 1) r = mulmod(r, a, q);
    return r;
}
// modular inverse by the extended Euclidean algorithm
uint64_t invmod(uint64_t a, uint64_t q) {
    __int128 t = 0, nt = 1, r = q, nr = a % q;
    while (nr) {
        __int128 qt = r / nr, tmp;
        tmp = t - qt * nt; t = nt; nt = tmp;
        tmp = r - qt * nr; r = nr; nr = tmp;
    }
    if (t < 0) t += q;
    return (uint64_t)t;
}
uint64_t shoup(uint64_t w, uint64_t q) { return (uint64_t)(((h128)w << 64) / q); }

// Miller-Rabin with the first 12 prime bases (exact below 3.3e24).
bool is_prime(uint64_t x) {
    static const uint64_t P[12] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
    if (x < 2) return false;
    for (uint64_t p : P)
        if (x % p == 0) return x == p;
    uint64_t d = x - 1;
    int s = 0;
    for (; !(d & 1); d >>= 1) s++;
    for (uint64_t a : P) {
        uint64_t y = powmod(a, d, x);
        if (y == 1 || y == x - 1) continue;
        bool ok = false;
        for (int r = 1; r < s && !ok; r++) {
            y = mulmod(y, y, x);
            ok = (y == x - 1);
        }
        if (!ok) return false;
    }
    return true;
}

bool chain(uint32_t n, uint32_t count, std::vector<uint64_t> &out) {
    out.clear();
    const uint64_t step = 2ull * n;
    for (uint64_t c = (1ull << 59) + 1; c < (1ull << 60) && out.size() < count; c += step)
        if (is_prime(c)) out.push_back(c);
    return out.size() == count;
}

// Any quadratic non-residue z gives w = z^((q-1)/2n) with w^n = -1; the odd
// powers of w are all the primitive 2n-th roots.
uint64_t min_root(uint32_t n, uint64_t q) {
    uint64_t z = 2;
    while (powmod(z, (q - 1) / 2, q) != q - 1) z++;
    uint64_t w = powmod(z, (q - 1) / (2ull * n), q), w2 = mulmod(w, w, q), best = w, cur = w;
    for (uint32_t k = 0; k < n; k++, cur = mulmod(cur, w2, q)) best = std::min(best, cur);
    return best;
}

uint32_t bitrev(uint32_t x, uint32_t bits) {
    uint32_t r = 0;
    for (uint32_t i = 0; i < bits; i++, x >>= 1) r = (r << 1) | (x & 1);
    return r;
}

void prime_tables(uint32_t n, uint64_t q, uint64_t psi, PrimeConsts &k, uint64_t *tf, uint64_t *ti, uint64_t &iota) {
    uint32_t logn = 0;
    while ((1u << logn) < n) logn++;
    const uint64_t ipsi = invmod(psi, q);
    k.q = q;
    k.mu = (uint64_t)(((h128)1 << 122) / q);
    k.r64 = (uint64_t)(((h128)1 << 64) % q);
    k.r64p = shoup(k.r64, q);
    k.m64 = (uint64_t)(((h128)1 << 64) / q);
    k.ninv = invmod(n % q, q);
    k.ninvp = shoup(k.ninv, q);
    k.r60 = (1ull << 60) % q;
    k.r60p = shoup(k.r60, q);
    // powers psi^e for e = 0..n-1, then placed at bit-reversed slots
    std::vector<uint64_t> fp(n), ip(n);
    uint64_t pw = 1, ipw = 1;
    for (uint32_t e = 0; e < n; e++, pw = mulmod(pw, psi, q), ipw = mulmod(ipw, ipsi, q)) {
        fp[e] = pw;
        ip[e] = ipw;
    }
    iota = fp[n / 2];  // psi^(n/2): a square root of -1
    for (uint32_t k2 = 0; k2 < n; k2++) {
        const uint32_t e = bitrev(k2, logn);
        tf[2 * k2] = fp[e];
        tf[2 * k2 + 1] = shoup(fp[e], q);
        ti[2 * k2] = ip[e];
        ti[2 * k2 + 1] = shoup(ip[e], q);
    }
}

static void permute_stage(uint64_t *tw, uint32_t s) {
    const uint32_t c = 1u << (s - 8);
    std::vector<uint64_t> old(tw + 2 * (1u << s), tw + 4 * (1u << s));
    for (uint32_t t = 0; t < 256; t++)
        for (uint32_t h = 0; h < c; h++)
            for (uint32_t w = 0; w < 2; w++) tw[2 * ((1u << s) + c * t + h) + w] = old[2 * (c * bitrev(t, 8) + h) + w];
}

void ntt2048_twiddle_order(uint64_t *tf, uint64_t *ti) {
    permute_stage(tf, 9);
    permute_stage(tf, 10);
    permute_stage(ti, 8);
    permute_stage(ti, 9);
    permute_stage(ti, 10);
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

void basis_tables(const std::vector<uint64_t> &primes, uint32_t L, uint32_t K, uint32_t first, uint32_t m,
                  bool chain_targets, BasisTables &o) {
    const uint32_t ntot = L + K;
    const uint64_t *b = primes.data() + first;
    o.m = m;
    o.first = first;
    o.inv_hat.assign(2 * m, 0);
    o.hat_mod.assign(2 * m, 0);
    o.R.assign(m, 0);
    o.garner.assign((size_t)2 * m * m, 0);
    o.half.assign(m, 0);
    std::vector<uint64_t> H((size_t)ntot * m), negB(ntot);
    // [Bhat_i]_t by prefix/suffix products, for every chain prime t
    std::vector<uint64_t> pre(m + 1), suf(m + 1);
    for (uint32_t t = 0; t < ntot; t++) {
        const uint64_t qt = primes[t];
        pre[0] = 1;
        for (uint32_t i = 0; i < m; i++) pre[i + 1] = mulmod(pre[i], b[i] % qt, qt);
        suf[m] = 1;
        for (uint32_t i = m; i-- > 0;) suf[i] = mulmod(suf[i + 1], b[i] % qt, qt);
        for (uint32_t i = 0; i < m; i++) H[(size_t)t * m + i] = mulmod(pre[i], suf[i + 1], qt);
        negB[t] = (qt - pre[m]) % qt;
    }
    for (uint32_t i = 0; i < m; i++) {
        const uint64_t bi = b[i];
        const uint64_t hm = H[(size_t)(first + i) * m + i];  // [Bhat_i]_{b_i}
        const uint64_t iv = invmod(hm, bi);
        o.inv_hat[2 * i] = iv;
        o.inv_hat[2 * i + 1] = shoup(iv, bi);
        o.hat_mod[2 * i] = hm;
        o.hat_mod[2 * i + 1] = shoup(hm, bi);
        o.R[i] = (uint64_t)(((h128)1 << 123) / bi);
        for (uint32_t k = 0; k < i; k++) {
            const uint64_t v = invmod(b[k] % bi, bi);
            o.garner[((size_t)k * m + i) * 2] = v;
            o.garner[((size_t)k * m + i) * 2 + 1] = shoup(v, bi);
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
            const uint64_t nc = B[j] & 1;
            B[j] = (B[j] >> 1) | (carry << 63);
            carry = nc;
        }
    }
    for (uint32_t i = 0; i < m; i++) o.half[i] = big_divmod(B, b[i]);

    // target positions
    o.pos.clear();
    if (first < L && !chain_targets) {
        for (uint32_t t = L; t < ntot; t++) o.pos.push_back(t);
        for (uint32_t t = 0; t < L; t++)
            if (t < first || t >= first + m) o.pos.push_back(t);
    } else {
        for (uint32_t t = 0; t < L; t++) o.pos.push_back(t);
    }
    // rows r < mk (mk = m + 1 rounded up to 32): r < m is [Bhat_r]_t, r = m is [-B]_t, the rest zero
    o.mk = (m + 1 + 31) / 32 * 32;
    o.npos = (uint32_t)o.pos.size();
    const uint32_t npad = (o.npos + 31) / 32 * 32;
    o.HD.assign((size_t)npad * 8 * o.mk, 0);
    o.RC.assign((size_t)npad * MF_RC, 0);
    for (uint32_t p = 0; p < o.npos; p++) {
        const uint32_t t = o.pos[p];
        const uint64_t qt = primes[t];
        for (uint32_t r = 0; r <= m; r++) {
            const uint64_t v = digit_form(r < m ? H[(size_t)t * m + r] : negB[t]);
            for (uint32_t d = 0; d < 8; d++) o.HD[((size_t)p * 8 + d) * o.mk + r] = (int8_t)(uint8_t)(v >> (8 * d));
        }
        recomb_row(qt, o.RC.data() + (size_t)p * MF_RC);
    }
}

void recomb_row(uint64_t q, uint64_t *row) {
    uint64_t w = powmod(2, 64, q);  // 256^8 mod q
    for (uint32_t s2 = 0; s2 < 7; s2++) {
        row[s2] = (w & ((1ull << 30) - 1)) | ((w >> 30) << 32);
        w = mulmod(w, 256, q);
    }
    row[7] = powmod(2, 60, q);
    row[8] = shoup(row[7], q);
    row[9] = q;
    row[10] = 8 * q - powmod(2, 91, q);
}

}  // namespace host
}  // namespace ckks
