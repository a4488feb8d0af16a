// evalmod.hip -- homomorphic modular reduction for bootstrapping (the
// "sin_fold" stage of the Kestrel article's section 5.3 boot profile, the
// second-largest bootstrap cost there): slot values x in [-K, K] are mapped to
// sin(2 pi x) / (2 pi) (about x - round(x) near integers) by
//   u = x / K,  p(u) = sum_k c_k T_k(u)  (Chebyshev interpolant of
//   cos(2 pi (K u - 1/4) / 2^r)),  y <- 2 y^2 - 1 (r times),  out = f y.
// Every step is a ciphertext operation on the GPU (tensor + relinearise,
// rescale, and one elementwise kernel); the host only tracks scales and
// rounds the plaintext constants.
#include <algorithm>
#include <cmath>
#include <vector>

#include "ckks_common.h"
#include "ops.h"

namespace ckks {

// v mod q for a signed 64-bit v (q in (2^59, 2^60), so |v| < 16 q).
__device__ __forceinline__ uint64_t smod(int64_t v, uint64_t q) {
    uint64_t u = v < 0 ? 0 - (uint64_t)v : (uint64_t)v;
    u = u >= 8 * q ? u - 8 * q : u;
    u = u >= 4 * q ? u - 4 * q : u;
    u = u >= 2 * q ? u - 2 * q : u;
    u = u >= q ? u - q : u;
    return (v < 0 && u) ? q - u : u;
}

// out[p][i][k] = ma a[p][i][k] + mb b'[p][i][k] + (p even ? add : 0)  mod q_i,
// for polynomials p (2 per ciphertext: even = c0) and limbs i < lo; a has la
// limbs per polynomial, b lb (b may be null), so inputs above level lo are
// read truncated.  b' = b, or with iota (psi_i^(n/2) per prime) b X^(n/2),
// whose NTT is b[k] iota (-1)^k: multiplying the slots by the imaginary unit.
// In the NTT domain a constant polynomial is the constant in every
// coefficient, so `add` adds a plaintext constant.  out may alias a or b.
__global__ __launch_bounds__(256) void k_lincomb(const uint64_t *a, uint32_t la, const uint64_t *b, uint32_t lb,
                                                 uint64_t *out, uint32_t lo, uint32_t n, int64_t ma, int64_t mb,
                                                 int64_t add, const uint64_t *__restrict__ iota,
                                                 const PrimeConsts *__restrict__ pc) {
    const uint32_t i = blockIdx.x % lo, poly = blockIdx.x / lo;
    const PrimeConsts P = pc[i];
    const uint64_t wa = smod(ma, P.q), wc = (poly % 2 == 0) ? smod(add, P.q) : 0;
    uint64_t wb = smod(mb, P.q), wbn = wb;  // weights of b at even / odd k
    if (iota) {
        wb = mulm(wb, iota[i], P.q, P.mu);
        wbn = wb ? P.q - wb : 0;
    }
    const uint64_t *ar = a + ((size_t)poly * la + i) * n;
    const uint64_t *br = b ? b + ((size_t)poly * lb + i) * n : nullptr;
    uint64_t *o = out + ((size_t)poly * lo + i) * n;
    for (uint32_t k = threadIdx.x; k < n; k += blockDim.x) {
        uint64_t v = mulm(ar[k], wa, P.q, P.mu);
        if (br) v = addm(v, mulm(br[k], (k & 1) ? wbn : wb, P.q, P.mu), P.q);
        o[k] = addm(v, wc, P.q);
    }
}

int op_lincomb(const ckks_ctx *c, uint64_t *out, int lo, const uint64_t *a, int la, const uint64_t *b, int lb,
               int64_t ma, int64_t mb, int64_t add, bool mono_b, int B, hipStream_t s) {
    ProfScope ps_(c, "lincomb", s);
    hipLaunchKernelGGL(k_lincomb, dim3(B * 2 * lo), dim3(256), 0, s, a, (uint32_t)la, b, (uint32_t)lb, out,
                       (uint32_t)lo, c->n, ma, mb, add, mono_b ? (const uint64_t *)c->d_iota : nullptr, c->d_pc);
    return hipGetLastError() == hipSuccess ? CKKS_OK : CKKS_EHIP;
}

namespace {

// A batch of ciphertexts [B][2][l][n] with its (tracked) scale.
struct Ct {
    uint64_t *p = nullptr;
    int l = 0;
    double s = 0;
};

}  // namespace

// Constant c encoded at scale t: the integer nearest c t (ties to even);
// |c t| must stay below 2^62 (checked: *ok is cleared otherwise).
int64_t enc_const(double c, double t, bool *ok) {
    const double v = std::nearbyint(c * t);
    if (!(std::fabs(v) < 4611686018427387904.0)) {  // 2^62 (also rejects NaN)
        *ok = false;
        return 0;
    }
    return (int64_t)v;
}

namespace {

struct Eval {
    const ckks_ctx *c;
    int B;
    const ckks_swk *rlk;
    uint64_t *tmp_a, *tmp_b, *tmp_p;  // scratch ciphertexts, up to the input level
    void *ks_ws;                      // key-switch / rescale workspace
    hipStream_t s;
    bool ok = true;                   // every constant fitted in 62 bits
    int64_t enc(double cst, double t) { return enc_const(cst, t, &ok); }

    size_t words(int l) const { return (size_t)B * 2 * l * c->n; }
    double q(int idx) const { return (double)c->primes[idx]; }

    int lincomb(uint64_t *out, int lo, const Ct &a, const Ct *b, int64_t ma, int64_t mb, int64_t add) {
        ProfScope ps_(c, "eval_lincomb", s);
        hipLaunchKernelGGL(k_lincomb, dim3(B * 2 * lo), dim3(256), 0, s, a.p, (uint32_t)a.l, b ? b->p : nullptr,
                           b ? (uint32_t)b->l : 0u, out, (uint32_t)lo, c->n, ma, mb, add, (const uint64_t *)nullptr,
                           c->d_pc);
        return hipGetLastError() == hipSuccess ? CKKS_OK : CKKS_EHIP;
    }
    // out = Rescale(x * [cst at the scale of the prime the rescale drops]): level -1, scale kept
    int cmul_rescale(const Ct &x, double cst, Ct &out) {
        int e;
        if ((e = lincomb(tmp_p, x.l, x, nullptr, enc(cst, q(x.l - 1)), 0, 0))) return e;
        if ((e = op_rescale(c, tmp_p, out.p, B, x.l, ks_ws, s))) return e;
        out.l = x.l - 1;
        out.s = x.s;
        return CKKS_OK;
    }
    // out = Rescale(Relin(a (x) b)) at the lower of the two levels; scale s_a s_b / q
    int mul_rescale(const Ct &a, const Ct &b, Ct &out) {
        const int mu = std::min(a.l, b.l);
        int e;
        Ct ta = a, tb = b;
        if (a.l > mu) {
            if ((e = lincomb(tmp_a, mu, a, nullptr, 1, 0, 0))) return e;
            ta = Ct{tmp_a, mu, a.s};
        }
        if (b.p == a.p) {
            tb = ta;
        } else if (b.l > mu) {
            if ((e = lincomb(tmp_b, mu, b, nullptr, 1, 0, 0))) return e;
            tb = Ct{tmp_b, mu, b.s};
        }
        if ((e = op_mul_tensor_relin(c, ta.p, tb.p, rlk, tmp_p, B, mu, ks_ws, s))) return e;
        if ((e = op_rescale(c, tmp_p, out.p, B, mu, ks_ws, s))) return e;
        out.l = mu - 1;
        out.s = (a.s * b.s) / q(mu - 1);
        return CKKS_OK;
    }
};

int ceil_log2(int d) {
    int r = 0;
    while ((1 << r) < d) r++;
    return r;
}

}  // namespace

int eval_mod_depth(int degree, int double_angles) { return 3 + ceil_log2(degree) + double_angles; }

// Largest number of Chebyshev products in one generation (k in (2^(g-1), 2^g]).
static int max_generation(int d) {
    int m = 1;
    for (int lo = 2; lo <= d; lo = 2 * lo - 1) m = std::max(m, std::min(2 * (lo - 1), d) - lo + 1);
    return m;
}

// Products per batched key switch: a generation, capped so that the stacked
// key-switch workspace stays within an 8 GiB budget.
constexpr size_t EVAL_KS_BUDGET = 8ull << 30;
static int gen_chunk(const ckks_ctx *c, int B, int l, int d) {
    const size_t per = std::max<size_t>(1, ws_bytes_relin(c, B, l));
    return std::max(1, std::min(max_generation(d), (int)(EVAL_KS_BUDGET / per)));
}

size_t ws_bytes_eval_mod(const ckks_ctx *c, int B, int l, int degree) {
    const size_t ct = ((size_t)B * 2 * l * c->n * 8 + 255) & ~(size_t)255;
    const int G = gen_chunk(c, B, l, degree);
    const size_t ks = std::max(ws_bytes_relin(c, G * B, l), ws_bytes_rescale(c, G * B, l));
    // T_1..T_d, the running sum, the double-angle value, three scratch ciphertexts,
    // and the stacked left / right factors and products of one batch of products
    return ((size_t)degree + 5) * ct + 4 * (size_t)G * ct + ks;
}

int op_eval_mod(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, double scale_in, const double *cheb,
                int degree, double bound_k, int double_angles, double out_factor, const ckks_swk *rlk, void *ws,
                double *scale_out, int *level_out, hipStream_t s) {
    const int d = degree;
    const size_t slot = (((size_t)B * 2 * l * c->n * 8) + 255) & ~(size_t)255;
    const int G = gen_chunk(c, B, l, d);
    uint8_t *base = (uint8_t *)ws;
    auto take = [&](size_t slots) {
        uint64_t *p = (uint64_t *)base;
        base += slots * slot;
        return p;
    };
    std::vector<Ct> T(d + 1);
    for (int k = 1; k <= d; k++) T[k].p = take(1);
    Ct acc{take(1)}, y{take(1)};
    uint64_t *ta = take(1), *tb = take(1), *tp = take(1);
    uint64_t *left = take(G), *right = take(G), *prod = take(G), *prod_r = take(G);
    Eval ev{c, B, rlk, ta, tb, tp, base, s};
    int e;
    // u = x / K
    if ((e = ev.cmul_rescale(Ct{const_cast<uint64_t *>(in), l, scale_in}, 1.0 / bound_k, T[1]))) return e;
    // T_2j = 2 T_j^2 - 1,  T_2j+1 = 2 T_j T_j+1 - T_1, one generation k in
    // (2^(g-1), 2^g] at a time: its products are independent and share the
    // level T_1 - g + 1, so they go through one batched tensor + relinearise
    // and one rescale (the residues are those of separate products)
    for (int glo = 2, g = 1; glo <= d; glo = 2 * glo - 1, g++)
    for (int lo = glo, ghi = std::min(2 * (glo - 1), d); lo <= ghi; lo += G) {
        const int hi = std::min(lo + G - 1, ghi), cnt = hi - lo + 1;
        const int mu = T[1].l - (g - 1);
        const size_t per = (size_t)B * 2 * mu * c->n;       // words of B ciphertexts at level mu
        const size_t per_r = (size_t)B * 2 * (mu - 1) * c->n;
        for (int k = lo; k <= hi; k++) {
            const int j = k / 2, jr = k - j;
            if ((e = ev.lincomb(left + (k - lo) * per, mu, T[j], nullptr, 1, 0, 0))) return e;
            if ((e = ev.lincomb(right + (k - lo) * per, mu, T[jr], nullptr, 1, 0, 0))) return e;
        }
        if ((e = op_mul_tensor_relin(c, left, right, rlk, prod, cnt * B, mu, ev.ks_ws, s))) return e;
        if ((e = op_rescale(c, prod, prod_r, cnt * B, mu, ev.ks_ws, s))) return e;
        for (int k = lo; k <= hi; k++) {
            const int j = k / 2, jr = k - j;
            const Ct pk{prod_r + (k - lo) * per_r, mu - 1, (T[j].s * T[jr].s) / ev.q(mu - 1)};
            if (k % 2 == 0) {
                if ((e = ev.lincomb(T[k].p, pk.l, pk, nullptr, 2, 0, ev.enc(-1.0, pk.s)))) return e;
            } else {
                if ((e = ev.lincomb(T[k].p, pk.l, pk, &T[1], 2, -1, 0))) return e;
            }
            T[k].l = pk.l;
            T[k].s = pk.s;
        }
    }
    // p = c_0 + sum_k c_k T_k: every T_k truncated to T_d's level, weighted by
    // c_k at the scale of the prime dropped next, one rescale; scale of T_d
    const int lp = T[d].l;
    const double wq = ev.q(lp - 1);
    if ((e = ev.lincomb(ev.tmp_p, lp, T[1], nullptr, ev.enc(cheb[1], wq), 0, 0))) return e;
    for (int k = 2; k <= d; k++) {
        const Ct cur{ev.tmp_p, lp, 0};
        if ((e = ev.lincomb(ev.tmp_p, lp, cur, &T[k], 1, ev.enc(cheb[k], wq), 0))) return e;
    }
    if ((e = op_rescale(c, ev.tmp_p, acc.p, B, lp, ev.ks_ws, s))) return e;
    acc.l = lp - 1;
    acc.s = T[d].s;
    if ((e = ev.lincomb(acc.p, acc.l, acc, nullptr, 1, 0, ev.enc(cheb[0], acc.s)))) return e;
    // r double angles: y <- 2 y^2 - 1
    Ct cur = acc;
    for (int i = 0; i < double_angles; i++) {
        Ct prod{y.p};
        if ((e = ev.mul_rescale(cur, cur, prod))) return e;
        if ((e = ev.lincomb(y.p, prod.l, prod, nullptr, 2, 0, ev.enc(-1.0, prod.s)))) return e;
        y.l = prod.l;
        y.s = prod.s;
        cur = y;
    }
    // out = f y
    Ct res{out};
    if ((e = ev.cmul_rescale(cur, out_factor, res))) return e;
    if (!ev.ok) return CKKS_EINVAL;  // launches were queued with a zeroed constant: the output is invalid
    if (scale_out) *scale_out = res.s;
    if (level_out) *level_out = res.l;
    return CKKS_OK;
}

}  // namespace ckks
