// kernels.hip -- HIP kernels and their launch sequences for the hot path.
//
// Hybrid key switching (the Kestrel article's technique table: RNS base
// conversion, Galois keys, relinearisation) runs as this kernel sequence on
// one stream, all data resident in HBM:
//   prep        d = a1 b1 (relin) or sigma_g(c1) (rotation), NTT domain
//   iNTT        y_i = iNTT(d)_i [Bhat_i^-1]_{q_i}        (scale folded into n^-1)
//   u           u = round(sum_i y_i / q_i) per digit, exact
//   convert     ModUp: each digit to every other prime of Q_l u P (centered CRT)
//   NTT         of the converted limbs
//   inner       acc = sum_j ext_j (.) (b_j, a_j) over Q_l u P
//   iNTT        of the P limbs of acc, scaled by [Phat_k^-1]_{p_k}
//   u, convert  ModDown: P -> Q_l (centered)
//   NTT         of the converted limbs
//   final       out = (acc - conv) P^-1 (+ d0/d1, or sigma_g(c0))
#include <algorithm>

#include "ctx_internal.h"
#include "multipass.h"
#include "multipass_kernels.h"
#include "mfma_digits.h"
#include "ntt2048.h"
#include "ops.h"

namespace ckks {

#define HIP_TRY(x)                                      \
    do {                                                \
        if ((x) != hipSuccess) return CKKS_EHIP;        \
    } while (0)
#define LAUNCH_CHECK() HIP_TRY(hipGetLastError())

static inline size_t align_words(size_t w) { return (w + 31) & ~size_t(31); }  // 256-byte units
static inline dim3 grid_for(size_t total) {
    size_t b = (total + 255) / 256;
    return dim3((unsigned)std::min<size_t>(b, 1u << 20));
}

// =====================================================================
// Limb maps for the NTT launches.  get(blk, ...) gives the source and
// destination of limb blk, its prime index, and an optional Shoup pair that
// replaces n^-1 on the inverse.  src == nullptr skips the block.
// =====================================================================
struct MapStrided {  // [count][nl][n], limb r -> prime first + r
    static constexpr bool digit_out = false;
    const uint64_t *src;
    uint64_t *dst;
    uint32_t n, nl, first;
    const uint64_t *scale;  // optional, indexed by prime index
    __device__ __forceinline__ void get(int blk, const uint64_t *&s, uint64_t *&d, int &prime,
                                        const uint64_t *&sc) const {
        prime = first + blk % nl;
        s = src + (size_t)blk * n;
        d = dst + (size_t)blk * n;
        sc = scale ? scale + 2 * prime : nullptr;
    }
};

struct MapBatched {  // limb r of ciphertext b at src + b * src_stride + r * n -> dst [B][nl][n]
    static constexpr bool digit_out = true;  // ModUp inputs y: stored in digit form (digit_form)
    const uint64_t *src;
    size_t src_stride;
    uint64_t *dst;
    uint32_t n, nl;
    const uint64_t *scale;  // optional, indexed by prime index
    __device__ __forceinline__ void get(int blk, const uint64_t *&s, uint64_t *&d, int &prime,
                                        const uint64_t *&sc) const {
        const uint32_t b = blk / nl, r = blk % nl;
        prime = r;
        s = src + b * src_stride + (size_t)r * n;
        d = dst + (size_t)blk * n;
        sc = scale ? scale + 2 * prime : nullptr;
    }
};

struct MapExt {  // converted limbs [B][beta][l+K][n]; skips the digit's own primes
    static constexpr bool digit_out = false;
    uint64_t *ext;
    uint32_t n, l, L, K, beta, alpha;
    __device__ __forceinline__ void get(int blk, const uint64_t *&s, uint64_t *&d, int &prime,
                                        const uint64_t *&sc) const {
        const uint32_t el = l + K;
        const uint32_t e = blk % el, j = (blk / el) % beta;
        sc = nullptr;
        if (e >= j * alpha && e < min(l, (j + 1) * alpha)) {
            s = nullptr;
            d = nullptr;
            prime = 0;
            return;
        }
        prime = e < l ? e : L + (e - l);
        d = ext + (size_t)blk * n;
        s = d;
    }
};

struct MapPolyPairs {  // [B][2][l][n] in place, visited as u = (b l + i) 2 + c (the two polynomials adjacent)
    static constexpr bool digit_out = false;
    uint64_t *x;
    uint32_t n, l;
    __device__ __forceinline__ void get(int blk, const uint64_t *&s, uint64_t *&d, int &prime,
                                        const uint64_t *&sc) const {
        const uint32_t c = blk % 2, i = (blk / 2) % l, b = blk / (2 * l);
        prime = i;
        d = x + ((size_t)(b * 2 + c) * l + i) * n;
        s = d;
        sc = nullptr;
    }
};

struct MapLast {  // last limb of each polynomial [P][l][n] -> dense [P][n]
    static constexpr bool digit_out = false;
    const uint64_t *src;
    uint64_t *dst;
    uint32_t n, l;
    __device__ __forceinline__ void get(int blk, const uint64_t *&s, uint64_t *&d, int &prime,
                                        const uint64_t *&sc) const {
        s = src + ((size_t)blk * l + (l - 1)) * n;
        d = dst + (size_t)blk * n;
        prime = l - 1;
        sc = nullptr;
    }
};

struct MapAccP {  // P limbs of acc [B][2][l+K][n], scaled inverse -> ModDown inputs
    static constexpr bool digit_out = true;  // ModDown inputs y: stored in digit form (digit_form)
    uint64_t *acc;
    uint32_t n, l, L, K;
    const uint64_t *scale;  // [K][2]
    __device__ __forceinline__ void get(int blk, const uint64_t *&s, uint64_t *&d, int &prime,
                                        const uint64_t *&sc) const {
        const uint32_t k = blk % K, poly = blk / K;
        d = acc + ((size_t)poly * (l + K) + l + k) * n;
        s = d;
        prime = L + k;
        sc = scale + 2 * k;
    }
};

template <class Map, bool INV>
__global__ __launch_bounds__(256) void k_ntt2048(Map map, const PrimeConsts *__restrict__ pc,
                                                  const uint64_t *__restrict__ twf,
                                                  const uint64_t *__restrict__ twi) {
    __shared__ uint64_t lds[n2048::LDS_WORDS];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    map.get(blockIdx.x, src, dst, prime, sc);
    if (!src) return;
    const uint64_t q = pc[prime].q;
    const int t = threadIdx.x;
    uint64_t v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = src[t + 256 * k];
    if (!INV) {
        n2048::fwd(v, lds, twf + (size_t)prime * 2048 * 2, q);
#pragma unroll
        for (int k = 0; k < 8; k++) dst[t + 256 * k] = reduce_out(v[k], q);
    } else {
        n2048::inv(v, lds, twi + (size_t)prime * 2048 * 2, q);
        const uint64_t w = sc ? sc[0] : pc[prime].ninv, wp = sc ? sc[1] : pc[prime].ninvp;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const uint64_t r = shoup(v[k], w, wp, q);
            dst[t + 256 * k] = Map::digit_out ? digit_form(r) : r;
        }
    }
}

// mp_scratch: the operation's transpose buffer for rings above one LDS tile
// (mp_scratch_words words), or null for the context's (the bare NTT calls).
template <class Map>
// gal != 1 (forward, n > 2048 only): outputs permuted by the automorphism of that Galois element.
static int launch_ntt(const ckks_ctx *c, const Map &map, int nblk, bool inverse, hipStream_t s, const char *name,
                      uint64_t *mp_scratch, uint32_t gal = 1) {
    if (nblk <= 0) return CKKS_OK;
    ProfScope ps(c, name, s);
    if (c->n == 2048) {
        if (gal != 1) return CKKS_EUNSUPPORTED;
        if (inverse)
            hipLaunchKernelGGL((k_ntt2048<Map, true>), dim3(nblk), dim3(256), 0, s, map, c->d_pc, c->d_tw_fwd,
                               c->d_tw_inv);
        else
            hipLaunchKernelGGL((k_ntt2048<Map, false>), dim3(nblk), dim3(256), 0, s, map, c->d_pc, c->d_tw_fwd,
                               c->d_tw_inv);
        LAUNCH_CHECK();
        return CKKS_OK;
    }
    return multipass_ntt(c, map, nblk, inverse, s, mp_scratch, gal);
}

int op_ntt(const ckks_ctx *c, uint64_t *x, int count, int first, int nlimbs, bool inverse, hipStream_t s) {
    MapStrided m{x, x, c->n, (uint32_t)nlimbs, (uint32_t)first, nullptr};
    return launch_ntt(c, m, count * nlimbs, inverse, s, inverse ? "ntt_inv" : "ntt_fwd", nullptr);
}

// =====================================================================
// Elementwise kernels (grid-stride over [..][l][n] elements)
// =====================================================================
__global__ void k_pointwise(const uint64_t *__restrict__ a, const uint64_t *__restrict__ b, uint64_t *__restrict__ o,
                            const PrimeConsts *__restrict__ pc, uint32_t n, uint32_t nl, uint32_t first,
                            size_t total) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
        const PrimeConsts &P = pc[first + (e / n) % nl];
        o[e] = mulm(a[e], b[e], P.q, P.mu);
    }
}
__device__ __forceinline__ uint32_t galois_src(uint32_t j, uint32_t g, uint32_t n) {
    // NTT-domain automorphism: out[j] = in[(g(2j+1) mod 2n - 1) / 2]
    return (uint32_t)((((uint64_t)g * (2 * j + 1)) & (2ull * n - 1)) >> 1);
}

// Residues at or above their prime in [count][nl][n] (limb r modulo prime first + r): the
// count is added to *cnt (cleared by the first kernel, so the pair works under stream capture).
__global__ void k_clear_u32(uint32_t *p) { *p = 0; }
__global__ void k_count_unreduced(const uint64_t *__restrict__ x, const PrimeConsts *__restrict__ pc, uint32_t n,
                                  uint32_t nl, uint32_t first, size_t total, uint32_t *__restrict__ cnt) {
    uint32_t mine = 0;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x)
        mine += x[e] >= pc[first + (e / n) % nl].q;
    if (mine) atomicAdd(cnt, mine);
}

int op_count_unreduced(const ckks_ctx *c, const uint64_t *x, int count, int first, int nlimbs, uint32_t *out,
                       hipStream_t s) {
    const size_t total = (size_t)count * nlimbs * c->n;
    hipLaunchKernelGGL(k_clear_u32, dim3(1), dim3(1), 0, s, out);
    LAUNCH_CHECK();
    if (total) {
        hipLaunchKernelGGL(k_count_unreduced, grid_for(total), dim3(256), 0, s, x, c->d_pc, c->n, (uint32_t)nlimbs,
                           (uint32_t)first, total, out);
        LAUNCH_CHECK();
    }
    return CKKS_OK;
}

int op_pointwise_mul(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, uint64_t *out, int count, int first,
                     int nlimbs, hipStream_t s) {
    const size_t total = (size_t)count * nlimbs * c->n;
    if (!total) return CKKS_OK;
    {
        ProfScope ps_(c, "pointwise_mul", s);
        hipLaunchKernelGGL(k_pointwise, grid_for(total), dim3(256), 0, s, a, b, out, c->d_pc, c->n, (uint32_t)nlimbs,
                           (uint32_t)first, total);
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

// d[b][i][k] = a[b][1][i][k] * b[b][1][i][k]   (tensor component d2)
__global__ void k_prep_relin(const uint64_t *__restrict__ a, const uint64_t *__restrict__ b, uint64_t *__restrict__ d,
                             const PrimeConsts *__restrict__ pc, uint32_t n, uint32_t l, size_t total) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
        const size_t per = (size_t)l * n;
        const size_t bi = e / per, r = e % per;
        const uint32_t i = r / n;
        const size_t off = (bi * 2 + 1) * per + r;
        d[e] = mulm(a[off], b[off], pc[i].q, pc[i].mu);
    }
}

// ---------------------------------------------------------------------
// u = round(sum_i y_i / b_i) for one coefficient of one basis.
// Fixed point: f_i = floor((16 y_i) R_i / 2^64) with R_i = floor(2^123 / b_i)
// lies in (y_i 2^63 / b_i - 2, y_i 2^63 / b_i], so the 2^-63-unit sum S' is
// below the true sum T by less than 2m units.  round(T) = floor((S' + 2^62) /
// 2^63) unless the fractional part of S' + 2^62 is within 2m of 2^63; then an
// exact mixed-radix comparison of x with (B-1)/2 decides.
// ---------------------------------------------------------------------
__device__ __attribute__((noinline)) uint32_t exact_u_slow(const BasisDev &B, uint64_t *ycol, size_t stride,
                                                          uint32_t floor_s, const PrimeConsts *__restrict__ pc) {
    const uint32_t m = B.m;
    // x_i = y_i [Bhat_i]_{b_i}, in place (y arrives in digit form, x is plain)
    for (uint32_t i = 0; i < m; i++) {
        const uint64_t bi = pc[B.first + i].q;
        ycol[i * stride] = shoup(undigit(ycol[i * stride]), B.hat_mod[2 * i], B.hat_mod[2 * i + 1], bi);
    }
    // Garner, in place: after step i, slot i holds mixed-radix digit a_i and
    // slots k > i hold (x - a_0 - ... ) / (b_0 ... b_i) mod b_k.
    int cmp = 0;
    for (uint32_t i = 0; i < m; i++) {
        const uint64_t ai = ycol[i * stride];
        const uint64_t hi = B.half[i];
        cmp = ai > hi ? 1 : (ai < hi ? -1 : cmp);
        for (uint32_t k = i + 1; k < m; k++) {
            const uint64_t bk = pc[B.first + k].q;
            const uint64_t a = ai >= bk ? ai - bk : ai;  // a_i < b_i < 2 b_k
            const uint64_t t = subm(ycol[k * stride], a, bk);
            const size_t gi = ((size_t)i * m + k) * 2;
            ycol[k * stride] = shoup(t, B.garner[gi], B.garner[gi + 1], bk);
        }
    }
    // restore y_i: x_i = sum_{k<=i} a_k prod_{t<k} b_t mod b_i (Horner), then y_i = x_i [Bhat_i^-1]
    for (uint32_t i = m; i-- > 0;) {
        const PrimeConsts &P = pc[B.first + i];
        uint64_t r = ycol[i * stride];
        for (uint32_t k = i; k-- > 0;) {
            const uint64_t bk = pc[B.first + k].q % P.q;
            uint64_t ak = ycol[k * stride];
            ak = ak >= P.q ? ak - P.q : ak;
            r = addm(mulm(r, bk, P.q, P.mu), ak, P.q);
        }
        ycol[i * stride] = digit_form(shoup(r, B.inv_hat[2 * i], B.inv_hat[2 * i + 1], P.q));
    }
    return floor_s + (cmp > 0 ? 1u : 0u);
}

// Sets s = 0..nsets-1; set s reads m_s limbs at y + (s / inner) * so + (s % inner) * si + off
// and uses basis bases[per_set_basis ? s % inner : 0].
struct SetLayout {
    size_t so, si, off;
    uint32_t inner, per_set_basis;
};

__global__ void k_basis_u(const BasisDev *__restrict__ bases, SetLayout lay, uint64_t *__restrict__ y,
                          uint32_t *__restrict__ u, uint32_t n, const PrimeConsts *__restrict__ pc) {
    const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t s = blockIdx.y;
    if (k >= n) return;
    const BasisDev &B = bases[lay.per_set_basis ? s % lay.inner : 0];
    uint64_t *yb = y + (s / lay.inner) * lay.so + (s % lay.inner) * lay.si + lay.off + k;
    const uint32_t m = B.m;
    const uint64_t M63 = (1ull << 63) - 1;
    uint64_t frac = 0;
    uint32_t ip = 0;
    auto add = [&](uint64_t y, uint64_t r) {
        frac += mulhi64(y << 4, r);
        ip += (uint32_t)(frac >> 63);
        frac &= M63;
    };
    if (m <= 32) {
        // bases of up to 32 primes: every row is requested before the first is used
        uint64_t yv[32];
#pragma unroll
        for (int a = 0; a < 32; a++) yv[a] = yb[(size_t)min((uint32_t)a, m - 1) * n];
        // the empty asm takes every loaded value, so the loads cannot be sunk into the row guards
#pragma unroll
        for (int a = 0; a < 32; a++) asm volatile("" : "+v"(yv[a]));
#pragma unroll
        for (int a = 0; a < 32; a++)
            if ((uint32_t)a < m) add(undigit(yv[a]), gload(B.R + a));
    }
    // the sum is exact integer arithmetic, so inputs are taken 8 at a time
    // with all 8 loads in flight before the first is used
    for (uint32_t i0 = m <= 32 ? m : 0; i0 < m; i0 += 8) {
        uint64_t yv[8], rv[8];
#pragma unroll
        for (int a = 0; a < 8; a++) {
            const uint32_t i = min(i0 + a, m - 1);
            yv[a] = undigit(yb[(size_t)i * n]);
            rv[a] = gload(B.R + i);
        }
#pragma unroll
        for (int a = 0; a < 8; a++)
            if (i0 + a < m) add(yv[a], rv[a]);
    }
    uint64_t t = frac + (1ull << 62);
    uint32_t uu = ip + (uint32_t)(t >> 63);
    t &= M63;
    if (t >= (1ull << 63) - 2ull * m) uu = exact_u_slow(B, yb, n, ip, pc);
    u[(size_t)s * n + k] = uu;
}

// ---------------------------------------------------------------------
// Exact base conversion, out_t = sum_i y_i [Bhat_i]_t + u [-B]_t mod t, of
// "sets" of inputs (one per digit and ciphertext, or summed sets of several
// steps) onto target positions.
// ---------------------------------------------------------------------
struct ConvTargets {
    // MODE 0 (ModUp of digit [lo, lo+m)): target positions run over [L, L+K),
    // then [0, lo) u [lo+m, l); the outputs go to ext slots (special t -> l + t - L)
    // MODE 1 (ModDown, ModRaise): targets = [0, l) -> slot t
    uint32_t l, L, K;
    size_t out_so, out_si;  // output limb base of set s: (s / inner) * out_so + (s % inner) * out_si
    // Summed conversions (nsum > 1): the input sets s + j * sum_stride, j < nsum,
    // are split into parts of spp consecutive j; output set p * sum_stride + s
    // (s < sum_stride) is the sum of part p's conversions, each converted exactly
    // with its own u.
    uint32_t nsum = 1, sum_stride = 0, spp = 1;
};

template <int MODE>
__device__ __forceinline__ uint32_t conv_target(const ConvTargets &ct, uint32_t tn, uint32_t lo, uint32_t m) {
    if (MODE == 1) return tn;
    if (tn < ct.K) return ct.L + tn;
    const uint32_t c = tn - ct.K;
    return c < lo ? c : c + m;
}

// ---------------------------------------------------------------------
// Base conversion on the matrix cores: the exact conversion sums
//   out[k][t] = sum_r Y[k][r] H[r][t] mod t,
// with the rows r of every summed set = its m inputs y_i (H = [Bhat_i]_t), then
// its u (H = [-B]_t), then zeros up to BasisDev::mk.  Both operands are written
// in signed base-256 digits (digit_form), so the product is
//   sum_s 256^s S_s,   S_s = sum_{a+b=s} sum_r dY_a[k][r] dH_b[r][t],
// and each digit pair (a, b) is an exact int8 x int8 -> int32 product on the
// matrix cores adding into S_{a+b} (|S_s| <= 8 rows 2^14 <= 2^28 for rows <=
// MF_MAX_ROWS); two pairs of a diagonal share one 16x16x64 MFMA (mac_tile).
// One wave computes 16 coefficients x 16 target positions at a time: lane l
// supplies coefficient row l % 16 of Y and target column l % 16 of H, each with
// the 8 rows 8 (l / 16) + j of a 32-row chunk, and ends with target column
// l % 16 of the coefficient rows 4 (l / 16) + v (v < 4).
// ---------------------------------------------------------------------
constexpr uint32_t MF_COEF = 64;  // coefficients per workgroup (4 waves x 16)
constexpr uint32_t MF_TPB = 8;    // 16-position target tiles per workgroup
// The one-chunk variant stages 7 tiles (112 target positions): its 40320 bytes of tables let
// four workgroups share a CU's 160 KiB of LDS, matching its 128-VGPR budget of four waves per SIMD.
constexpr uint32_t MF_TPB1 = 7;
template <int OCC>
constexpr uint32_t mf_tpb() { return OCC == 3 ? MF_TPB1 : MF_TPB; }

constexpr uint32_t MF_HSTRIDE = 272;  // LDS bytes per target position (8 digits x 32 rows + bank padding)
// Byte offset, within a position, of the 8 rows of lane group g of digit b: the rows of digits
// 2h and 2h + 1 are adjacent, so mf_right's tuple h of a lane is one 16-byte read.
__device__ __forceinline__ constexpr uint32_t h_slot(uint32_t b, uint32_t g) { return 64 * (b / 2) + 16 * g + 8 * (b % 2); }

// OCC selects the variant: 3 when the whole contraction is one 32-row chunk
// (128 VGPRs and 7 staged tiles, so four waves per SIMD fit), 2 otherwise (two
// waves per SIMD).  STAGED: the basis rows fit
// one 32-row block (mk = 32), so the workgroup's digit table rows and
// reduction constants are staged in LDS once; otherwise the fragments come
// from the global table one chunk ahead of their use.
template <int MODE, int OCC, bool STAGED>
__global__ __launch_bounds__(256, OCC == 3 ? 4 : OCC) void k_convert_mfma(const BasisDev *__restrict__ bases, SetLayout lay,
                                                          const uint64_t *__restrict__ y,
                                                          const uint32_t *__restrict__ u, ConvTargets ct,
                                                          uint64_t *__restrict__ out, uint32_t n,
                                                          const PrimeConsts *__restrict__ pc) {
    constexpr uint32_t TPB = mf_tpb<OCC>();
    __shared__ __align__(16) int8_t sh_h[STAGED ? TPB * 16 * MF_HSTRIDE : 2 * 2 * 16 * MF_HSTRIDE];
    __shared__ uint64_t sh_rc[STAGED ? TPB * 16 * MF_RC : 1];
    constexpr bool FOLD_U = OCC == 3;  // u computed here rather than read (k_basis_u)
    const uint32_t s = blockIdx.z;
    const BasisDev &B = bases[lay.per_set_basis ? s % lay.inner : 0];
    const uint32_t m = B.m, lo = B.first, mk = B.mk;
    const uint32_t ntarget = MODE == 0 ? ct.l - m + ct.K : ct.l;
    const uint32_t tile0 = blockIdx.y * TPB;
    if (tile0 * 16 >= ntarget) return;
    const uint32_t tile_end = min(tile0 + TPB, (ntarget + 15) / 16), ntile = tile_end - tile0;
    const uint32_t lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const uint32_t kb = blockIdx.x * MF_COEF + (threadIdx.x >> 6) * 16;
    const uint32_t part = ct.nsum > 1 ? s / ct.sum_stride : 0;
    const size_t sfirst = ct.nsum > 1 ? s + (size_t)part * (ct.spp - 1) * ct.sum_stride : s;
    const uint32_t nsets = ct.nsum > 1 ? min(ct.spp, ct.nsum - part * ct.spp) : 1;
    // OCC 3 is launched only for one-chunk contractions (one set, mk = 32)
    const uint32_t cps = mk / 32, nch = OCC == 3 ? 1 : nsets * cps;  // 32-row chunks per set, in all
    const uint64_t *yb = y + (sfirst / lay.inner) * lay.so + (sfirst % lay.inner) * lay.si + lay.off + kb + col;
    const size_t set_step = (size_t)ct.sum_stride * lay.so;
    // rows 8 grp + j of chunk ch, loaded unconditionally (index clamped; the u row
    // and the padding rows are substituted when the fragments are built)
    auto load_rows = [&](uint64_t(&raw)[8], uint32_t &uraw, uint32_t ch) {
        const uint32_t js = ch / cps, r0 = (ch % cps) * 32 + 8 * grp;
        const uint64_t *ys = yb + js * set_step;
#pragma unroll
        for (int j = 0; j < 8; j++) raw[j] = ys[(size_t)min(r0 + j, m - 1) * n];
        if constexpr (!FOLD_U) uraw = u[(sfirst + (size_t)js * ct.sum_stride) * n + kb + col];
    };
    // One-chunk launches (a single set of at most 31 rows) take the set's u from its rows, as
    // k_basis_u does: the 4 lanes of a coefficient sum the fixed-point y_r / b_r of their 8 rows
    // and exchange the partial sums; a sum too close to a rounding boundary goes to the exact
    // path on a private copy of the column (other workgroups read the same rows).
    auto exact_u = [&](const uint64_t(&raw)[8], uint32_t ch) -> uint32_t {
        const uint64_t M63 = (1ull << 63) - 1;
        const uint32_t r0 = 8 * grp;
        uint64_t frac = 0;
        uint32_t ip = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t r = min(r0 + j, m - 1);
            const uint64_t rr = r0 + j < m ? gload(B.R + r) : 0;
            frac += mulhi64(undigit(raw[j]) << 4, rr);
            ip += (uint32_t)(frac >> 63);
            frac &= M63;
        }
#pragma unroll
        for (int off = 16; off <= 32; off *= 2) {
            const uint64_t f2 = __shfl_xor(frac, off);
            const uint32_t i2 = __shfl_xor(ip, off);
            const uint64_t sum = frac + f2;  // both below 2^63
            ip += i2 + (uint32_t)(sum >> 63);
            frac = sum & M63;
        }
        uint64_t t = frac + (1ull << 62);
        uint32_t uu = ip + (uint32_t)(t >> 63);
        t &= M63;
        if (t >= (1ull << 63) - 2ull * m) {
            uint64_t colv[32];
            const uint64_t *ys = yb + (ch / cps) * set_step;
            for (uint32_t r = 0; r < m; r++) colv[r] = ys[(size_t)r * n];
            uu = exact_u_slow(B, colv, 1, ip, pc);
        }
        return uu;
    };
    // the first rows are in flight while the tables are staged
    uint64_t rb[2][8];
    uint32_t ub[2];
    load_rows(rb[0], ub[0], 0);
    // rows are prefetched two chunks ahead whenever a set may have several chunks: always in
    // the unstaged variant (a compile-time condition there, so that no branch joins differing
    // load histories; a set of its launch with one chunk then reloads that chunk)
    const bool rows_ahead = OCC != 3 && (!STAGED || nch > 1);
    if (rows_ahead) load_rows(rb[1], ub[1], 1 % nch);
    if constexpr (STAGED) {
        // position p's 8 x 32 digit bytes are contiguous in HD (mk = 32), [digit b][row]; in LDS the
        // 8 rows of lane group grp of digits 2h and 2h + 1 sit together (h_slot): 8-byte copies
        const uint32_t np = ntile * 16;
        const int8_t *src = B.HD + (size_t)16 * tile0 * 256;
        for (uint32_t q = threadIdx.x; q < np * 32; q += 256) {
            const uint32_t b = (q % 32) / 4, gq = q % 4;
            *(uint2 *)(sh_h + (q / 32) * MF_HSTRIDE + h_slot(b, gq)) = *(const uint2 *)(src + (size_t)q * 8);
        }
        const uint64_t *rsrc = B.RC + (size_t)16 * tile0 * MF_RC;
        for (uint32_t q = threadIdx.x; q < np * MF_RC; q += 256) sh_rc[q] = rsrc[q];
        __syncthreads();
    }
    // the digit planes of the lane's 8 rows (byte j = row 8 grp + j) as the A operands of the
    // 64-deep products: mf_left's windows, except in the 128-VGPR one-chunk variant, which keeps
    // the windows on the per-tile operand (see mfma_digits.h)
    constexpr bool WIN_A = OCC != 3;
    mf_v4i AW[WIN_A ? MF_NW : MF_NT];
    auto build_a = [&](const uint64_t(&raw)[8], uint32_t uraw, uint32_t ch) {
        if constexpr (FOLD_U) uraw = exact_u(raw, ch);
        const uint32_t r0 = (ch % cps) * 32 + 8 * grp;
        // row r < m is input y_r (stored in digit form), row m the u row, the rest zero (whose digit
        // form is 0): selected without branches, so that no lane-divergent block waits for every
        // load in flight (the prefetched chunks)
        const uint64_t zu = digit_form(uraw);
        uint64_t z[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t r = r0 + j;
            uint64_t v = r < m ? raw[j] : zu;
            z[j] = r <= m ? v : 0;
        }
        long pl[8];
        mf_planes(z, pl);
        mf_left(pl, AW);
    };
    // TT target tiles share each chunk's A fragments (2 when the contraction has
    // several chunks, so the rows are fetched and transposed once per 2 tiles)
    constexpr uint32_t TT = OCC == 3 ? 1 : 2;
    // H fragments of a tile (mf_right's tuples): from LDS.  Staged: the workgroup's whole
    // table, loaded once (the one-chunk variant reads a tile's fragments once, the
    // two-wave variant at every chunk).
    // Otherwise the digit-table slice of each (pass, chunk), 2 tiles x 16
    // positions x 8 digits x 32 rows, goes through a double-buffered LDS slice
    // that the workgroup fills one step ahead (all its waves run the same steps).
    // The staged two-wave variant (summed sets) reads a tile's tuples from LDS again at every
    // chunk rather than keeping both tiles' tuples for the whole pass, which keeps it within
    // 256 VGPRs.
    constexpr int NH = WIN_A ? MF_NT : MF_NW;  // 4-VGPR H registers per tile
    mf_v4i hb[TT][NH];
    auto load_h = [&](mf_v4i(&H)[NH], uint32_t tile, uint32_t buf) {
        const int8_t *h = STAGED ? sh_h + ((tile - tile0) * 16 + col) * MF_HSTRIDE
                                 : sh_h + ((buf * 2 + (tile - tile0) % 2) * 16 + col) * MF_HSTRIDE;
        if constexpr (WIN_A) {
#pragma unroll
            for (int p = 0; p < NH; p++) H[p] = *(const mf_v4i *)(h + h_slot(2 * p, grp));
        } else {
            long pl[8];
#pragma unroll
            for (int b = 0; b < 8; b++) pl[b] = *(const long *)(h + h_slot(b, grp));
            mf_right(pl, H);
        }
    };
    // the slice of step g: thread x copies 16-byte pieces q = x and x + 256 of the
    // 2 x 16 x 8 x 32 bytes (tiles past tile_end read padded, in-bounds positions).  The two
    // pieces live in named registers (an array captured by the lambdas went to scratch memory,
    // and its store waited for every load in flight), read through a global-address-space
    // pointer (a generic one makes flat loads, which count against the LDS counter too).
    u32x4 hs0{}, hs1{};
    const uint32_t sl_pos = (threadIdx.x / 16) % 16, sl_b = (threadIdx.x / 2) % 8, sl_hf = threadIdx.x % 2;
    auto fetch_slice = [&](uint32_t g) {
        const uint32_t t0 = tile0 + (g / nch) * TT, c0 = (g % nch % cps) * 32;
        const uint32_t ta = min(t0, tile_end - 1), tb = min(t0 + 1, tile_end - 1);
        hs0 = gload((const u32x4 *)(B.HD + ((size_t)(16 * ta + sl_pos) * 8 + sl_b) * mk + c0 + 16 * sl_hf));
        hs1 = gload((const u32x4 *)(B.HD + ((size_t)(16 * tb + sl_pos) * 8 + sl_b) * mk + c0 + 16 * sl_hf));
    };
    auto store_slice = [&](uint32_t buf) {  // the piece's rows 16 sl_hf .. + 16 are lane groups 2 sl_hf, + 1
        const uint32_t o0 = sl_pos * MF_HSTRIDE + h_slot(sl_b, 2 * sl_hf), o1 = o0 + h_slot(0, 1);
        int8_t *d0 = sh_h + ((buf * 2 + 0) * 16) * MF_HSTRIDE, *d1 = sh_h + ((buf * 2 + 1) * 16) * MF_HSTRIDE;
        *(uint2 *)(d0 + o0) = uint2{hs0.x, hs0.y};
        *(uint2 *)(d0 + o1) = uint2{hs0.z, hs0.w};
        *(uint2 *)(d1 + o0) = uint2{hs1.x, hs1.y};
        *(uint2 *)(d1 + o1) = uint2{hs1.z, hs1.w};
    };
    const MfW2 w2 = mf_w2();
    auto recombine = [&](uint32_t tile, const mf_v4i(&acc)[15]) {
        const uint32_t p = 16 * tile + col;
        if (p >= ntarget) return;  // padding columns: every MFMA ran on the whole wave
        const uint64_t *rc = STAGED ? sh_rc + ((tile - tile0) * 16 + col) * MF_RC : B.RC + (size_t)p * MF_RC;
        const MfRecomb k = mf_recomb_consts([&](int d) -> uint64_t { return STAGED ? rc[d] : gload(rc + d); });
        const uint32_t t = conv_target<MODE>(ct, p, lo, m);
        const uint32_t slot = (MODE == 0 && t >= ct.L) ? ct.l + (t - ct.L) : t;
        uint64_t *ob = out + (s / lay.inner) * ct.out_so + (s % lay.inner) * ct.out_si + (size_t)slot * n + kb + 4 * grp;
        if constexpr (OCC == 3) {  // one chunk of at most 32 rows
#pragma unroll
            for (int v = 0; v < 4; v++) ob[v] = mf_recombine32(acc, v, w2, k);
        } else {
#pragma unroll
            for (int v = 0; v < 4; v++) ob[v] = mf_recombine(acc, v, w2, k);
        }
    };
    mf_v4i acc[TT][15];
    // the flat sequence g = pass nch + ch over passes of TT tiles; rows are
    // fetched two chunks ahead
    const uint32_t total = (ntile + TT - 1) / TT * nch;
    if (!rows_ahead) build_a(rb[0], ub[0], 0);
    if constexpr (!STAGED) {
        fetch_slice(0);
        store_slice(0);
        __syncthreads();
    }
    auto step = [&](uint64_t(&raw)[8], uint32_t &uraw, uint32_t g) {
        const uint32_t t0 = tile0 + (g / nch) * TT, ch = g % nch;
        if (ch == 0) {
#pragma unroll
            for (uint32_t tt = 0; tt < TT; tt++)
#pragma unroll
                for (int d = 0; d < 15; d++) acc[tt][d] = mf_v4i{0, 0, 0, 0};
        }
        if (rows_ahead) build_a(raw, uraw, ch);
        // the next slice is requested before the row prefetch: loads complete in order, so
        // storing the slice then leaves the prefetched rows in flight.  Both are issued on every
        // step (past the end they fetch clamped, valid addresses that nobody uses): branches
        // around them make the compiler drain every load in flight at the loop's joins.
        if constexpr (!STAGED) fetch_slice(g + 1);
        asm volatile("" ::: "memory");  // keeps the slice loads ahead of the row loads
        if (rows_ahead) load_rows(raw, uraw, (g + 2) % nch);
#pragma unroll
        for (uint32_t tt = 0; tt < TT; tt++) {
            if (t0 + tt >= tile_end) break;  // workgroup-uniform
            if (!STAGED || ch == 0 || OCC == 2) load_h(hb[tt], t0 + tt, g & 1);  // OCC 2: see NH
            mf_mac_tile(acc[tt], AW, hb[tt]);
        }
        if constexpr (!STAGED) {
            // the next slice goes to the other buffer, whose last readers (step g - 1)
            // passed the barrier at its end; this barrier publishes it for step g + 1
            store_slice((g + 1) & 1);
            __syncthreads();
        }
        if (ch + 1 < nch) return;
#pragma unroll
        for (uint32_t tt = 0; tt < TT; tt++)
            if (t0 + tt < tile_end) recombine(t0 + tt, acc[tt]);
    };
    for (uint32_t g = 0; g < total; g += 2) {
        step(rb[0], ub[0], g);
        if (g + 1 < total) step(rb[1], ub[1], g + 1);
    }
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Maps dispatch index i to (group g, member j < B) so that the B members of a
// group (the B ciphertexts that read one key row) run on one XCD back to back:
// launch xcd_blocks(ngroups, B) workgroups; those with g >= ngroups exit.
constexpr uint32_t NXCD = 8;
__device__ __forceinline__ void xcd_group(uint32_t i, uint32_t B, uint32_t &g, uint32_t &j) {
    const uint32_t x = i % NXCD, k = i / NXCD;
    g = x + NXCD * (k / B);
    j = k % B;
}
static inline uint32_t xcd_blocks(uint32_t ngroups, uint32_t B) {
    return (ngroups + NXCD - 1) / NXCD * NXCD * B;
}

// A batched key switch runs S "steps" of B ciphertexts each: output
// ciphertext cb = s * B + b uses key[s] and Galois element g[s].  With
// shared = 1 every step switches the same B inputs (hoisted baby steps);
// otherwise step s has its own inputs (ciphertext cb).
constexpr int MAX_STEPS = 32;
struct Steps {
    const uint64_t *key[MAX_STEPS];  // [dnum][2][L + K][n], or the b rows [dnum][L + K][n] when seeded
    uint32_t g[MAX_STEPS];
    uint64_t root[MAX_STEPS];        // seeded keys: key_seed_root(seed) of each step's key
    uint32_t count, B, shared, seeded;
};

// acc[cb][c][e][k] = sum_j v_j[e][galois_src(k)] key[j][c][gidx(e)][k], where
// v_j[e] = d[ct][e] (NTT domain, own digit) or ext[ct][j][e] (ModUp of digit j).
// With g = 1 the gather is the identity.  With g != 1 this is the key switch
// of sigma_g(d): exact centered ModUp commutes with the automorphism, so
// permuting the extended digits equals extending the permuted polynomial.
// One workgroup per (output ciphertext, extended limb): each digit's limb is
// loaded into LDS with coalesced reads and permuted from there; the key rows
// are read in order.  (n = 2048: 8 coefficients per thread.)  SEEDED: the keys
// hold their b rows only and each a-row residue is regenerated from its seed.
template <bool SEEDED>
__global__ __launch_bounds__(256) void k_inner2048(const uint64_t *__restrict__ d, size_t d_stride,
                                                    const uint64_t *__restrict__ ext, const Steps st,
                                                    uint64_t *__restrict__ acc, const PrimeConsts *__restrict__ pc,
                                                    uint32_t l, uint32_t L, uint32_t K, uint32_t beta,
                                                    uint32_t alpha, uint32_t e0, uint32_t ne) {
    constexpr uint32_t n = 2048;
    __shared__ uint64_t buf[2][n];
    const uint32_t el = l + K;
    // group = (step, limb of the range [e0, e0 + ne)), member = ciphertext: the
    // B blocks reading one key row share an XCD's L2, one step's key at a time
    uint32_t grp, bl;
    xcd_group(blockIdx.x, st.B, grp, bl);
    if (grp >= st.count * ne) return;
    const uint32_t e = e0 + grp % ne;
    const uint32_t step = grp / ne;
    const size_t cb = (size_t)step * st.B + bl;
    const size_t b = st.shared ? bl : cb;  // input ciphertext
    const uint64_t *key = st.key[step];
    const uint32_t g = st.g[step];
    const uint32_t gi = e < l ? e : L + (e - l);
    const uint32_t t = threadIdx.x;
    Split3 s0[8], s1[8];
#pragma unroll
    for (int m = 0; m < 8; m++) s0[m] = s1[m] = {0, 0, 0, 0};
    for (uint32_t j = 0; j < beta; j++) {
        const bool own = e >= j * alpha && e < min(l, (j + 1) * alpha);
        const uint64_t *src = own ? d + b * d_stride + (size_t)e * n : ext + ((b * beta + j) * el + e) * n;
        const uint64_t *kb = key + ((size_t)j * (SEEDED ? 1 : 2) * (L + K) + gi) * n;
        const uint64_t *ka = kb + (size_t)(L + K) * n;
        // the key rows are requested with the digit row, before the barrier (which the
        // compiler does not move loads across), so both arrive in one memory latency
        uint64_t sv[8], kbv[8], kav[8];
#pragma unroll
        for (int m = 0; m < 8; m++) sv[m] = src[t + 256 * m];
#pragma unroll
        for (int m = 0; m < 8; m++) {
            kbv[m] = kb[t + 256 * m];
            if (!SEEDED) kav[m] = ka[t + 256 * m];
        }
        uint64_t *lb = buf[j & 1];
#pragma unroll
        for (int m = 0; m < 8; m++) lb[t + 256 * m] = sv[m];
        __syncthreads();
        const uint64_t row = SEEDED ? sm_at(st.root[step], (uint64_t)j * (L + K) + gi) : 0;
        const uint64_t qa = pc[gi].q;
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const uint32_t k = t + 256 * m;
            const uint64_t v = lb[galois_src(k, g, n)];
            const uint32_t vl = (uint32_t)(v & M30), vh = (uint32_t)(v >> 30);
            smac(s0[m], vl, vh, split30(kbv[m]));
            smac(s1[m], vl, vh, split30(SEEDED ? seeded_a(row, k, qa) : kav[m]));
        }
        if ((j + 1) % SPLIT_CHUNK == 0) {  // more than 15 digits: keep the sums in bounds
#pragma unroll
            for (int m = 0; m < 8; m++) {
                snorm(s0[m]);
                snorm(s1[m]);
            }
            if ((j + 1) % (4 * SPLIT_CHUNK) == 0) {
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    sreduce(s0[m], pc[gi]);
                    sreduce(s1[m], pc[gi]);
                }
            }
        }
    }
    const PrimeConsts P = pc[gi];
    uint64_t *o0 = acc + ((cb * 2 + 0) * el + e) * n, *o1 = acc + ((cb * 2 + 1) * el + e) * n;
#pragma unroll
    for (int m = 0; m < 8; m++) {
        o0[t + 256 * m] = sreduce60(s0[m], P);  // a2 < 2^64: sreduce at least every 60 products
        o1[t + 256 * m] = sreduce60(s1[m], P);
    }
}

// Hoisted baby steps (n = 2048): every step of the batch switches the same B
// inputs, so a workgroup (extended limb e, group of HOIST_SPW steps; member =
// input ciphertext) stages limb e of the input's beta digits in LDS once and
// runs its steps on them: each step gathers sigma_g of the digits from LDS and
// takes the inner product with that step's key rows.  The B members of a group
// share an XCD, so each key row is fetched once per XCD.  Same sums and output
// layout as k_inner2048 with shared = 1.
constexpr uint32_t HOIST_SPW = 16;
constexpr uint32_t HOIST_MAX_BETA = 4;  // beta digit limbs of 16 KiB in at most 64 KiB of LDS
__global__ __launch_bounds__(256) void k_inner_hoisted2048(const uint64_t *__restrict__ d, size_t d_stride,
                                                            const uint64_t *__restrict__ ext, const Steps st,
                                                            uint64_t *__restrict__ acc,
                                                            const PrimeConsts *__restrict__ pc, uint32_t l, uint32_t L,
                                                            uint32_t K, uint32_t beta, uint32_t alpha) {
    constexpr uint32_t n = 2048;
    __shared__ uint64_t dig[HOIST_MAX_BETA * n];
    const uint32_t el = l + K;
    uint32_t grp, b;
    xcd_group(blockIdx.x, st.B, grp, b);
    const uint32_t ngroups = (st.count + HOIST_SPW - 1) / HOIST_SPW;
    if (grp >= el * ngroups) return;
    const uint32_t e = grp % el, s0 = (grp / el) * HOIST_SPW, s1 = min(st.count, s0 + HOIST_SPW);
    const uint32_t gi = e < l ? e : L + (e - l);
    const uint32_t t = threadIdx.x;
    {  // every digit row is requested before the first is stored (rows past beta repeat the last)
        uint64_t dv[HOIST_MAX_BETA][8];
#pragma unroll
        for (uint32_t j = 0; j < HOIST_MAX_BETA; j++) {
            const uint32_t jj = min(j, beta - 1);
            const bool own = e >= jj * alpha && e < min(l, (jj + 1) * alpha);
            const uint64_t *src = own ? d + b * d_stride + (size_t)e * n : ext + ((b * beta + jj) * el + e) * n;
#pragma unroll
            for (int m = 0; m < 8; m++) dv[j][m] = src[t + 256 * m];
        }
#pragma unroll
        for (uint32_t j = 0; j < HOIST_MAX_BETA; j++)
#pragma unroll
            for (int m = 0; m < 8; m++) dig[j * n + t + 256 * m] = dv[j][m];
    }
    __syncthreads();
    const PrimeConsts P = pc[gi];
    // (step, digit) pairs run flattened, it = (step - s0) beta + j; the key rows of pair it + 1 are
    // in flight while pair it is multiplied (buffers A / B alternate; past the last pair the last
    // rows are fetched again)
    const uint32_t T = (s1 - s0) * beta;
    Split3c a0[8], a1[8];
    // byte offsets of sigma_g's sources in a digit row, computed once per step
    // (at its first digit) and shared by its beta digits
    uint32_t sidx[8];
    auto kload = [&](uint32_t it, uint64_t (&kbv)[8], uint64_t (&kav)[8]) {
        it = min(it, T - 1);
        const uint32_t step = s0 + it / beta, j = it % beta;
        const uint64_t *kb = st.key[step] + ((size_t)j * 2 * (L + K) + gi) * n;
        const uint64_t *ka = kb + (size_t)(L + K) * n;
#pragma unroll
        for (int m = 0; m < 8; m++) {
            kbv[m] = kb[t + 256 * m];
            kav[m] = ka[t + 256 * m];
        }
    };
    auto pair = [&](uint32_t it, const uint64_t (&kbv)[8], const uint64_t (&kav)[8]) {
        const uint32_t step = s0 + it / beta, j = it % beta;
        if (j == 0) {
            const uint32_t g = st.g[step];
#pragma unroll
            for (int m = 0; m < 8; m++) {
                a0[m] = a1[m] = {0, 0, 0};
                sidx[m] = galois_src(t + 256 * m, g, n) * 8;
            }
        }
        const char *row = (const char *)(dig + j * n);
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const uint64_t v = *(const uint64_t *)(row + sidx[m]);
            const uint32_t vl = (uint32_t)(v & M30), vh = (uint32_t)(v >> 30);
            smac(a0[m], vl, vh, split30(kbv[m]));
            smac(a1[m], vl, vh, split30(kav[m]));
        }
        if (j == beta - 1 && it < T) {  // beta <= HOIST_MAX_BETA products per sum: within the snorm-free bound
            const size_t cb = (size_t)step * st.B + b;
            uint64_t *o0 = acc + ((cb * 2 + 0) * el + e) * n, *o1 = acc + ((cb * 2 + 1) * el + e) * n;
#pragma unroll
            for (int m = 0; m < 8; m++) {
                o0[t + 256 * m] = sreduce60(a0[m], P);
                o1[t + 256 * m] = sreduce60(a1[m], P);
            }
        }
    };
    // the empty asm with a memory clobber is a compiler-only fence: the prefetch stays ahead of
    // the pair it overlaps instead of being sunk next to its use
    uint64_t kbA[8], kaA[8], kbB[8], kaB[8];
    kload(0, kbA, kaA);
    for (uint32_t it = 0; it < T; it += 2) {
        kload(it + 1, kbB, kaB);
        asm volatile("" ::: "memory");
        pair(it, kbA, kaA);
        kload(it + 2, kbA, kaA);
        asm volatile("" ::: "memory");
        pair(it + 1, kbB, kaB);  // it + 1 = T (T odd) multiplies the repeated last rows and stores nothing
    }
}

// Giant-step inner product summed over the steps of a batch (n = 2048, limbs
// e < l).  Block (part p, ciphertext b, limb e) covers the steps
// [p * spp, min(count, (p + 1) * spp)) and writes
//   acc[p B + b][c][e][k] = sum_s ( sum_j v_{s,j}[e][src_s(k)] key_s[j][c][e][k]
//                                   + [c = 0] [P]_{q_e} c0_s[e][src_s(k)] ),
// src_s = galois_src(., g_s).  A rotation's result is
//   (acc_s - NTT(ModDown conversion of acc_s's P-part)) P^-1 + sigma_{g_s}(c0_s),
// which is linear in acc_s's Q-part and in sigma(c0_s) (carried as P sigma(c0_s)
// inside the accumulator); only the conversion, which lifts each step's P-part
// exactly, must stay per step.  So the Q-part of the giant-step sum is formed
// here without storing the individual rotations.
__global__ __launch_bounds__(256) void k_inner_sum2048(const uint64_t *__restrict__ d, size_t d_stride,
                                                        const uint64_t *__restrict__ c0, size_t c0_stride,
                                                        const uint64_t *__restrict__ ext, const Steps st,
                                                        uint32_t spp, uint32_t nparts, uint64_t *__restrict__ acc,
                                                        const PrimeConsts *__restrict__ pc,
                                                        const uint64_t *__restrict__ pmod, uint32_t l, uint32_t K,
                                                        uint32_t L, uint32_t beta, uint32_t alpha) {
    constexpr uint32_t n = 2048;
    __shared__ uint64_t buf[2][n];
    const uint32_t el = l + K;
    uint32_t grp, bl;  // group = (part, limb), member = ciphertext (see xcd_group)
    xcd_group(blockIdx.x, st.B, grp, bl);
    if (grp >= nparts * l) return;
    const uint32_t e = grp % l;
    const uint32_t part = grp / l;
    const uint32_t s_end = min(st.count, (part + 1) * spp);
    const uint32_t t = threadIdx.x;
    const PrimeConsts P = pc[e];
    const uint64_t pm = split30(pmod[e]);
    Split3c s0[8], s1[8];
#pragma unroll
    for (int m = 0; m < 8; m++) s0[m] = s1[m] = {0, 0, 0};
    uint32_t cnt = 0, rounds = 0, bi = 0;
    // called before each product: at most 15 products between snorm, at most
    // 4 snorm rounds between full reductions
    auto guard = [&]() {
        if (cnt == SPLIT_CHUNK) {
#pragma unroll
            for (int m = 0; m < 8; m++) {
                snorm(s0[m]);
                snorm(s1[m]);
            }
            cnt = 0;
            if (++rounds == 4) {
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    sreduce(s0[m], P);
                    sreduce(s1[m], P);
                }
                rounds = 0;
            }
        }
        cnt++;
    };
    for (uint32_t step = part * spp; step < s_end; step++) {
        const size_t cb = (size_t)step * st.B + bl;
        const uint64_t *key = st.key[step];
        const uint32_t g = st.g[step];
        for (uint32_t j = 0; j < beta; j++) {
            const bool own = e >= j * alpha && e < min(l, (j + 1) * alpha);
            const uint64_t *src = own ? d + cb * d_stride + (size_t)e * n : ext + ((cb * beta + j) * el + e) * n;
            const uint64_t *kb = key + ((size_t)j * 2 * (L + K) + e) * n;
            const uint64_t *ka = kb + (size_t)(L + K) * n;
            // the key rows are requested with the digit row, before the barrier (which the
            // compiler does not move loads across), so both arrive in one memory latency
            uint64_t sv[8], kbv[8], kav[8];
#pragma unroll
            for (int m = 0; m < 8; m++) sv[m] = src[t + 256 * m];
#pragma unroll
            for (int m = 0; m < 8; m++) {
                kbv[m] = kb[t + 256 * m];
                kav[m] = ka[t + 256 * m];
            }
            uint64_t *lb = buf[bi];
            bi ^= 1;
#pragma unroll
            for (int m = 0; m < 8; m++) lb[t + 256 * m] = sv[m];
            __syncthreads();
            guard();
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const uint32_t k = t + 256 * m;
                const uint64_t v = lb[galois_src(k, g, n)];
                const uint32_t vl = (uint32_t)(v & M30), vh = (uint32_t)(v >> 30);
                smac(s0[m], vl, vh, split30(kbv[m]));
                smac(s1[m], vl, vh, split30(kav[m]));
            }
        }
        {  // P sigma_g(c0) joins the c = 0 sum
            const uint64_t *src = c0 + cb * c0_stride + (size_t)e * n;
            uint64_t *lb = buf[bi];
            bi ^= 1;
#pragma unroll
            for (int m = 0; m < 8; m++) lb[t + 256 * m] = src[t + 256 * m];
            __syncthreads();
            guard();
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const uint64_t v = lb[galois_src(t + 256 * m, g, n)];
                smac(s0[m], (uint32_t)(v & M30), (uint32_t)(v >> 30), pm);
            }
        }
    }
    const size_t ob = (size_t)part * st.B + bl;
    uint64_t *o0 = acc + ((ob * 2 + 0) * el + e) * n, *o1 = acc + ((ob * 2 + 1) * el + e) * n;
#pragma unroll
    for (int m = 0; m < 8; m++) {
        o0[t + 256 * m] = sreduce60(s0[m], P);  // a2 < 2^64: sreduce at least every 60 products
        o1[t + 256 * m] = sreduce60(s1[m], P);
    }
}

// Generic-n version: one thread per (extended limb, coefficient) for all B
// ciphertexts of the step, gathered global reads.  The thread loads its key
// values once and reuses them for every ciphertext (consecutive threads take
// consecutive coefficients, so the reads stay coalesced and each key row
// leaves memory once per launch instead of once per ciphertext).
constexpr uint32_t INNER_UNROLL = 8;  // digits held in registers (beta up to this; larger beta loops)
template <bool SEEDED>
__global__ void k_inner(const uint64_t *__restrict__ d, size_t d_stride, const uint64_t *__restrict__ ext,
                        const uint64_t *__restrict__ key, uint64_t *__restrict__ acc,
                        const PrimeConsts *__restrict__ pc, uint32_t n, uint32_t l, uint32_t L, uint32_t K,
                        uint32_t beta, uint32_t alpha, uint32_t g, uint32_t ge, uint64_t root, uint32_t B) {
    const uint32_t el = l + K;
    const size_t total = (size_t)el * n;
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const uint32_t k = idx % n;
        const uint32_t e = idx / n;
        const uint32_t gi = e < l ? e : L + (e - l);
        const uint32_t ks = galois_src(k, g, n), kx = galois_src(k, ge, n);
        auto digit = [&](size_t b, uint32_t j) -> uint64_t {
            const bool own = e >= j * alpha && e < min(l, (j + 1) * alpha);
            return own ? d[b * d_stride + (size_t)e * n + ks] : ext[((b * beta + j) * el + e) * n + kx];
        };
        auto key_b = [&](uint32_t j) -> uint64_t {
            return key[((size_t)j * (SEEDED ? 1 : 2) * (L + K) + gi) * n + k];
        };
        auto key_a = [&](uint32_t j) -> uint64_t {
            return SEEDED ? seeded_a(sm_at(root, (uint64_t)j * (L + K) + gi), k, pc[gi].q)
                          : key[((size_t)j * 2 * (L + K) + gi) * n + k + (size_t)(L + K) * n];
        };
        if (beta <= INNER_UNROLL) {
            // rows past beta repeat the last digit's (in-bounds) and are zeroed before the product
            uint64_t kb[INNER_UNROLL], ka[INNER_UNROLL];
#pragma unroll
            for (uint32_t j = 0; j < INNER_UNROLL; j++) {
                const uint32_t jj = min(j, beta - 1);
                kb[j] = key_b(jj);
                ka[j] = key_a(jj);
            }
            for (uint32_t b = 0; b < B; b++) {
                uint64_t v[INNER_UNROLL];
#pragma unroll
                for (uint32_t j = 0; j < INNER_UNROLL; j++) v[j] = digit(b, min(j, beta - 1));
                Split3 s0{0, 0, 0, 0}, s1{0, 0, 0, 0};
#pragma unroll
                for (uint32_t j = 0; j < INNER_UNROLL; j++) {
                    const uint64_t x = j < beta ? v[j] : 0;  // at most 8 products: within the snorm-free bound
                    const uint32_t vl = (uint32_t)(x & M30), vh = (uint32_t)(x >> 30);
                    smac(s0, vl, vh, split30(kb[j]));
                    smac(s1, vl, vh, split30(ka[j]));
                }
                acc[((b * 2 + 0) * el + e) * n + k] = sreduce60(s0, pc[gi]);
                acc[((b * 2 + 1) * el + e) * n + k] = sreduce60(s1, pc[gi]);
            }
            continue;
        }
        for (uint32_t b = 0; b < B; b++) {
            Split3 s0{0, 0, 0, 0}, s1{0, 0, 0, 0};
            for (uint32_t j = 0; j < beta; j++) {
                const uint64_t v = digit(b, j);
                const uint32_t vl = (uint32_t)(v & M30), vh = (uint32_t)(v >> 30);
                smac(s0, vl, vh, split30(key_b(j)));
                smac(s1, vl, vh, split30(key_a(j)));
                if ((j + 1) % SPLIT_CHUNK == 0) {  // more than 15 digits: keep the sums in bounds
                    snorm(s0);
                    snorm(s1);
                    if ((j + 1) % (4 * SPLIT_CHUNK) == 0) {
                        sreduce(s0, pc[gi]);
                        sreduce(s1, pc[gi]);
                    }
                }
            }
            // a2 stays below 2^64: sreduce runs at least every 60 digits
            acc[((b * 2 + 0) * el + e) * n + k] = sreduce60(s0, pc[gi]);
            acc[((b * 2 + 1) * el + e) * n + k] = sreduce60(s1, pc[gi]);
        }
    }
}

// Fused ModDown tail for n > 2048 (four-step NTT): the row pass of the converted
// P-part's forward NTT (its column pass left it in the transpose buffer), then
//   out[b][c][i][k] = (acc[b][c][i][k] - NTT(conv)[b][c][i][k]) P^-1 + extra
//   MODE 1: relin (c0: a0 b0, c1: a0 b1 + a1 b0); 2: rotate (c0: in[b][0][i][galois]);
//   ACCUM: out += result instead of out = result.
// Row index y: pair index u = limb0 + y (MapPolyPairs order: the two polynomials of
// one (ciphertext, limb) are neighbours, so the workgroups that both read a0 and b0
// of a relinearisation run back to back on one XCD and the second finds them in
// L2); the NTT values meet their accumulator in registers instead of a round trip
// through memory.
template <int MODE, bool ACCUM>
__global__ __launch_bounds__(mp::NT) void k_rows_final(uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                          const uint64_t *__restrict__ rowf,
                                                          const uint64_t *__restrict__ scratch,
                                                          const uint64_t *__restrict__ acc,
                                                          const uint64_t *__restrict__ pinv,
                                                          const uint64_t *__restrict__ xa,
                                                          const uint64_t *__restrict__ xb, uint32_t g,
                                                          uint64_t *__restrict__ out, uint32_t l, uint32_t K) {
    using namespace mp;
    constexpr uint32_t n = MP_N1 * MP_N1;
    __shared__ uint64_t lds[V * VSTRIDE];
    // MODE 2: the 32 row blocks of a pair of limbs (c0 and c1 of one ciphertext limb) share one XCD
    // (workgroups are dealt to the 8 XCDs in turn), so the gather of c0 over its whole limb is served by
    // that XCD's L2; a last group of fewer than 16 limbs keeps the plain order.
    uint32_t by = blockIdx.y, bx = blockIdx.x;
    if (MODE == 2 && by < (gridDim.y & ~15u)) {
        const uint32_t id = by * 16 + bx, r = id & 255;
        by = (id >> 8) * 16 + 2 * (r & 7) + (r >> 7);
        bx = (r >> 3) & 15;
    }
    const uint32_t u = limb0 + by, c = u % 2, i = (u / 2) % l;
    const size_t b = u / (2 * l);
    const size_t limb = (b * 2 + c) * l + i;
    const uint64_t q = pc[i].q, mu = pc[i].mu;
    const int r0 = bx * V;
    // output lanes run across rows (128-byte runs of the limb); their accumulator values and extra
    // terms are requested and formed before the row transform, so the loads are in flight while
    // its butterflies run (its barriers keep the compiler from sinking them)
    const int vo = threadIdx.x % V, to = threadIdx.x / V;
    const size_t per = (size_t)l * n;
    const uint64_t *ap = acc + ((b * 2 + c) * (l + K) + i) * n;
    const uint64_t *x0 = xa + (b * 2) * per + (size_t)i * n;  // MODE 1: a0 (a1 one polynomial on); 2: c0
    const uint64_t *y0 = MODE == 1 ? xb + (b * 2) * per + (size_t)i * n : nullptr;
    auto pos = [&](int k) -> uint32_t { return (uint32_t)(r0 + vo) + MP_N1 * (uint32_t)(to + 16 * k); };
    uint64_t av[E], ex[E];
#pragma unroll
    for (int k = 0; k < E; k++) av[k] = ap[pos(k)];
    if (MODE == 1) {
        if (c == 0) {  // workgroup-uniform
#pragma unroll
            for (int k = 0; k < E; k++) ex[k] = mulm(x0[pos(k)], y0[pos(k)], q, mu);
        } else {
#pragma unroll
            for (int k = 0; k < E; k++) {
                const uint32_t j = pos(k);
                ex[k] = addm(mulm(x0[j], y0[j + per], q, mu), mulm(x0[j + per], y0[j], q, mu), q);
            }
        }
    } else if (MODE == 2 && c == 0) {
#pragma unroll
        for (int k = 0; k < E; k++) ex[k] = x0[galois_src(pos(k), g, n)];
    }
    {
        const BfConsts bc = bf_consts(q);
        const uint64_t *in = scratch + (size_t)by * n;
        const int t = threadIdx.x % 16, v = threadIdx.x / 16;  // lanes along a row
        uint64_t x[E];
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = in[sidx(r0 + v, t + 16 * k)];
        fwd(x, lds, v, t, rowf + ((size_t)i * 16 + ((r0 + v) >> 4)) * MP_N1 * 2, bc);
    }
    uint64_t *op = out + limb * n;
    const uint64_t w = pinv[2 * i], wp = pinv[2 * i + 1];
    const uint64_t *lb = lds + slot(vo, to);
#pragma unroll
    for (int k = 0; k < E; k++) {
        const uint32_t j = pos(k);
        const uint64_t nt = reduce_out(lb[islot(16 * k)], q);
        uint64_t r = shoup(subm(av[k], nt, q), w, wp, q);
        if (MODE == 1 || (MODE == 2 && c == 0)) r = addm(r, ex[k], q);
        if (ACCUM) r = addm(r, op[j], q);
        op[j] = r;
    }
}

// conv, acc: the key switch's converted P-part and accumulators; mps: its transpose buffer.
template <int MODE, bool ACCUM>
static int moddown_final_mp(const ckks_ctx *c, uint64_t *conv, const uint64_t *acc, uint64_t *mps, size_t nout,
                            int l, const uint64_t *xa, const uint64_t *xb, uint32_t g, uint64_t *out, hipStream_t s) {
    const MultipassPlan *p = c->mp;
    if (!p || !mps) return CKKS_EUNSUPPORTED;
    const int nblk = (int)(nout * 2 * l);
    MapPolyPairs m{conv, c->n, (uint32_t)l};
    for (int l0 = 0, ch = mp_chunk(nblk); l0 < nblk; l0 += ch) {
        const dim3 grid(MP_N1 / mp::V, (unsigned)std::min<int>(ch, nblk - l0)), blk(mp::NT);
        hipLaunchKernelGGL(mp::k_fwd_cols<MapPolyPairs>, grid, blk, 0, s, m, (uint32_t)l0, c->d_pc, p->d_tw256f,
                           p->d_taf, mps);
        hipLaunchKernelGGL((k_rows_final<MODE, ACCUM>), grid, blk, 0, s, (uint32_t)l0, c->d_pc, p->d_rowf,
                           (const uint64_t *)mps, acc, c->d_pinv, xa, xb, g, out, (uint32_t)l, c->K);
        LAUNCH_CHECK();
    }
    return CKKS_OK;
}

// n = 2048 fused ModDown tail: one workgroup per (output ciphertext cb,
// polynomial, limb i): NTT of the converted P-part in LDS, then
//   out = (acc - NTT(conv)) P^-1 + extra   (MODE / ACCUM as k_moddown_final);
// for rotations c0 (of the step's input ciphertext) is staged in LDS and
// permuted with the step's Galois element.
template <int MODE, bool ACCUM>
__global__ __launch_bounds__(256) void k_final2048(const uint64_t *__restrict__ acc, const uint64_t *__restrict__ conv,
                                                    const uint64_t *__restrict__ pinv,
                                                    const PrimeConsts *__restrict__ pc,
                                                    const uint64_t *__restrict__ twf, const uint64_t *__restrict__ xa,
                                                    const uint64_t *__restrict__ xb, const Steps st,
                                                    uint64_t *__restrict__ out, uint32_t l, uint32_t K) {
    constexpr uint32_t n = 2048;
    __shared__ uint64_t lds[n2048::LDS_WORDS];
    const uint32_t i = blockIdx.x % l;
    const uint32_t c = (blockIdx.x / l) % 2;
    const size_t cb = blockIdx.x / (2 * l);
    const size_t b = st.shared ? cb % st.B : cb;  // input ciphertext of the extra term
    const uint32_t g = st.g[cb / st.B];
    const uint32_t t = threadIdx.x;
    const PrimeConsts P = pc[i];
    const uint64_t q = P.q;
    const size_t per = (size_t)l * n;
    uint64_t v[8];
    const uint64_t *cv = conv + (size_t)blockIdx.x * n;
#pragma unroll
    for (int m = 0; m < 8; m++) v[m] = cv[t + 256 * m];
    // the accumulator row (and for rotations c0) are loaded before the transform, so they arrive
    // while it runs instead of after it (its barriers keep the compiler from hoisting them)
    const uint64_t *ar = acc + ((cb * 2 + c) * (l + K) + i) * n;
    uint64_t av[8], c0v[8];
#pragma unroll
    for (int m = 0; m < 8; m++) av[m] = ar[t + 256 * m];
    if (MODE == 2 && c == 0) {  // workgroup-uniform: only the c0 rows take the rotated input
        const uint64_t *c0 = xa + (b * 2) * per + (size_t)i * n;
#pragma unroll
        for (int m = 0; m < 8; m++) c0v[m] = c0[t + 256 * m];
    }
    n2048::fwd(v, lds, twf + (size_t)i * n * 2, q);
    if (MODE == 2 && c == 0) {  // stage c0 of this limb for the Galois gather
#pragma unroll
        for (int m = 0; m < 8; m++) lds[t + 256 * m] = c0v[m];
        __syncthreads();
    }
    uint64_t *o = out + (size_t)blockIdx.x * n;
    const uint64_t w = pinv[2 * i], wp = pinv[2 * i + 1];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const uint32_t k = t + 256 * m;
        const uint64_t x = reduce_out(v[m], q);
        uint64_t r = shoup(subm(av[m], x, q), w, wp, q);
        if (MODE == 1) {
            const size_t o0 = (b * 2) * per + (size_t)i * n + k, o1 = o0 + per;
            uint64_t y;
            if (c == 0) y = mulm(xa[o0], xb[o0], q, P.mu);
            else y = addm(mulm(xa[o0], xb[o1], q, P.mu), mulm(xa[o1], xb[o0], q, P.mu), q);
            r = addm(r, y, q);
        } else if (MODE == 2) {
            if (c == 0) r = addm(r, lds[galois_src(k, g, n)], q);
        }
        if (ACCUM) r = addm(r, o[k], q);
        o[k] = r;
    }
}

// n = 2048 giant-step tail: one workgroup per (ciphertext b, polynomial c, limb i):
//   out[b][c][i] += (sum_p acc[p B + b][c][i] - NTT(sum_p conv[p B + b][c][i])) P^-1
// with the parts' accumulators from k_inner_sum2048 and the parts of the
// batch's ModDown conversions, summed in the coefficient domain (the NTT is
// linear, so one transform serves the whole batch).
__global__ __launch_bounds__(256) void k_final_giant2048(const uint64_t *__restrict__ acc,
                                                          const uint64_t *__restrict__ conv,
                                                          const uint64_t *__restrict__ pinv,
                                                          const PrimeConsts *__restrict__ pc,
                                                          const uint64_t *__restrict__ twf, uint32_t nparts,
                                                          uint32_t nconv, uint32_t B, uint64_t *__restrict__ out,
                                                          uint32_t l, uint32_t K) {
    constexpr uint32_t n = 2048;
    __shared__ uint64_t lds[n2048::LDS_WORDS];
    const uint32_t i = blockIdx.x % l;
    const uint32_t c = (blockIdx.x / l) % 2;
    const size_t b = blockIdx.x / (2 * l);
    const uint32_t t = threadIdx.x;
    const PrimeConsts P = pc[i];
    const uint64_t q = P.q;
    uint64_t v[8];
    const uint64_t *cv = conv + (size_t)blockIdx.x * n;
    const size_t cstride = (size_t)B * 2 * l * n;
    // parts outer, coefficients inner: each part's 8 loads are in flight together; the
    // accumulator parts and the output row are requested before the transform starts
#pragma unroll
    for (int m = 0; m < 8; m++) v[m] = cv[t + 256 * m];
    for (uint32_t p = 1; p < nconv; p++)
#pragma unroll
        for (int m = 0; m < 8; m++) v[m] = addm(v[m], cv[p * cstride + t + 256 * m], q);
    const size_t pstride = (size_t)B * 2 * (l + K) * n;
    const uint64_t *ar = acc + ((b * 2 + c) * (l + K) + i) * n;
    uint64_t *o = out + (size_t)blockIdx.x * n;
    uint64_t a[8], ov[8];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        a[m] = ar[t + 256 * m];
        ov[m] = o[t + 256 * m];
    }
    for (uint32_t p = 1; p < nparts; p++)
#pragma unroll
        for (int m = 0; m < 8; m++) a[m] = addm(a[m], ar[p * pstride + t + 256 * m], q);
    n2048::fwd(v, lds, twf + (size_t)i * n * 2, q);
    const uint64_t w = pinv[2 * i], wp = pinv[2 * i + 1];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const uint64_t x = reduce_out(v[m], q);
        o[t + 256 * m] = addm(ov[m], shoup(subm(a[m], x, q), w, wp, q), q);
    }
}

// n = 2048 fused rescale tail: per (ciphertext, polynomial, limb i < l-1):
// centered lift of t = iNTT(c_{l-1}) to q_i, NTT in LDS, out = (c_i - .) q_{l-1}^-1.
__global__ __launch_bounds__(256) void k_rescale2048(const uint64_t *__restrict__ in, const uint64_t *__restrict__ tl,
                                                      const uint64_t *__restrict__ rinv,
                                                      const PrimeConsts *__restrict__ pc,
                                                      const uint64_t *__restrict__ twf, uint64_t *__restrict__ out,
                                                      uint32_t l) {
    constexpr uint32_t n = 2048;
    __shared__ uint64_t lds[n2048::LDS_WORDS];
    const uint32_t i = blockIdx.x % (l - 1);
    const size_t bc = blockIdx.x / (l - 1);
    const uint32_t t = threadIdx.x;
    const uint64_t q = pc[i].q, ql = pc[l - 1].q;
    const uint64_t qlm = ql >= q ? ql - q : ql;
    uint64_t v[8];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const uint64_t x = tl[bc * n + t + 256 * m];  // in [0, q_{l-1}), q_{l-1} < 2 q_i
        uint64_t y = x >= q ? x - q : x;
        if (x > (ql - 1) / 2) y = subm(y, qlm, q);
        v[m] = y;
    }
    n2048::fwd(v, lds, twf + (size_t)i * n * 2, q);
    const uint64_t *ci = in + (bc * l + i) * n;
    uint64_t *o = out + (bc * (l - 1) + i) * n;
    const uint64_t w = rinv[2 * i], wp = rinv[2 * i + 1];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const uint32_t k = t + 256 * m;
        const uint64_t x = reduce_out(v[m], q);
        o[k] = shoup(subm(ci[k], x, q), w, wp, q);
    }
}

// ---------------------------------------------------------------------
// Rescale (drop q_{l-1}): r = centered t mod q_i, then out = (c_i - NTT(r)) q_{l-1}^-1.
// ---------------------------------------------------------------------
__global__ void k_rescale_lift(const uint64_t *__restrict__ t, uint64_t *__restrict__ r,
                               const PrimeConsts *__restrict__ pc, uint32_t n, uint32_t l, size_t total) {
    const uint64_t ql = pc[l - 1].q;
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const uint32_t k = idx % n;
        const uint32_t i = (idx / n) % (l - 1);
        const size_t bc = idx / ((size_t)n * (l - 1));
        const uint64_t q = pc[i].q;
        const uint64_t v = t[bc * n + k];
        // t < q_{l-1} < 2 q_i for all chain primes here; centered: t or t - q_{l-1}
        uint64_t x = v >= q ? v - q : v;
        if (v > (ql - 1) / 2) {
            uint64_t qlm = ql >= q ? ql - q : ql;
            x = subm(x, qlm, q);
        }
        r[idx] = x;
    }
}

__global__ void k_rescale_final(const uint64_t *__restrict__ in, const uint64_t *__restrict__ r,
                                const uint64_t *__restrict__ rinv, const PrimeConsts *__restrict__ pc,
                                uint64_t *__restrict__ out, uint32_t n, uint32_t l, size_t total) {
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const uint32_t k = idx % n;
        const uint32_t i = (idx / n) % (l - 1);
        const size_t bc = idx / ((size_t)n * (l - 1));
        const uint64_t q = pc[i].q;
        const uint64_t c = in[(bc * l + i) * n + k];
        out[idx] = shoup(subm(c, r[idx], q), rinv[2 * i], rinv[2 * i + 1], q);
    }
}

// ---------------------------------------------------------------------
// BSGS multiply-accumulate for every giant step at once:
//   inner[g][col][i][k] = sum_bb pt[g][bb][i][k] rot_bb[col][i][k]
// (col = ciphertext * 2 + polynomial; rot_0 is the input itself, rot_bb for
// bb >= 1 at rot + (bb - 1) * ctsize).  A workgroup owns limb i, 16
// coefficients and 16 columns; thread (k, col) keeps its rotated inputs for up
// to MAC_B baby steps in registers (split30).  The diagonals of giant step g
// (MAC_B x 16 values, 128-byte runs) are staged in LDS, double-buffered and
// prefetched two giant steps ahead, and read as broadcasts: every diagonal
// element leaves HBM once.  Baby steps beyond MAC_B are added in further
// passes (ACC: the pass adds into inner).  Every global load is issued
// unconditionally (addresses clamped to valid rows, unused values masked
// afterwards) so that loads stay in flight together instead of each waiting
// behind a per-lane branch; FULL marks launches whose columns are all active.
// ---------------------------------------------------------------------
constexpr int MAC_K = 16, MAC_C = 16, MAC_B = 32, MAC_R = 4;
static_assert(MAC_B <= 4 * SPLIT_CHUNK, "one split sum per giant step without a 128-bit fold");
static_assert(MAC_B % MAC_R == 0, "diagonal rows are read from LDS in groups of MAC_R");

template <bool FULL, bool ACC>
__global__ __launch_bounds__(256) void k_bsgs_mac(const uint64_t *__restrict__ pt, const uint64_t *__restrict__ in,
                                                   const uint64_t *__restrict__ rot, uint64_t *__restrict__ inner,
                                                   const PrimeConsts *__restrict__ pc, uint32_t n, uint32_t l,
                                                   uint32_t bs, uint32_t gs, uint32_t ncols, size_t ctsize,
                                                   uint32_t b0) {
    __shared__ uint64_t ps[2][MAC_B * MAC_K];
    const uint32_t t = threadIdx.x;
    const uint32_t i = blockIdx.y;
    const uint32_t k0 = blockIdx.x * MAC_K;
    const uint32_t kl = t % MAC_K;
    const uint32_t col = blockIdx.z * MAC_C + t / MAC_K;
    const bool active = FULL || col < ncols;
    const PrimeConsts P = pc[i];
    const uint32_t nb = min((uint32_t)MAC_B, bs - b0);
    const size_t off = ((size_t)(active ? col : 0) * l + i) * n + k0 + kl;
    uint64_t r[MAC_B];
#pragma unroll
    for (int bb = 0; bb < MAC_B; bb++) {
        const uint32_t b = b0 + min((uint32_t)bb, nb - 1);
        r[bb] = (b == 0 ? in : rot + (size_t)(b - 1) * ctsize)[off];
    }
    // the empty asm takes every loaded value, so the loads cannot be sunk into per-row branches
#pragma unroll
    for (int bb = 0; bb < MAC_B; bb++) asm volatile("" : "+v"(r[bb]));
#pragma unroll
    for (int bb = 0; bb < MAC_B; bb++) r[bb] = (active && bb < (int)nb) ? split30(r[bb]) : 0;
    const size_t pstride = (size_t)l * n;
    // staging: thread t loads elements x = t and t + 256 of the MAC_B x MAC_K tile
    auto pt_addr = [&](uint32_t g, uint32_t x) -> const uint64_t * {
        const uint32_t bb = x / MAC_K, kk = x % MAC_K;
        return pt + ((size_t)g * bs + b0 + min(bb, nb - 1)) * pstride + (size_t)i * n + k0 + kk;
    };
    // diagonal tiles are prefetched two giant steps ahead (registers a: even g, b: odd g);
    // past the last giant step the last tile is fetched again, so every step issues its loads
    const uint32_t g1 = min(1u, gs - 1);
    uint64_t a0 = *pt_addr(0, t), a1 = *pt_addr(0, t + 256);
    uint64_t b0v = *pt_addr(g1, t), b1v = *pt_addr(g1, t + 256);
    auto step = [&](uint32_t g, uint64_t &s0, uint64_t &s1) {
        uint64_t *buf = ps[g & 1];
        buf[t] = split30(s0);  // stored split: low 30 bits | high 30 bits << 32
        buf[t + 256] = split30(s1);
        __syncthreads();
        const uint32_t gn = min(g + 2, gs - 1);
        s0 = *pt_addr(gn, t);
        s1 = *pt_addr(gn, t + 256);
        Split3c sp{0, 0, 0};
#pragma unroll
        for (int c = 0; c < MAC_B; c += MAC_R) {
            // rows bb >= nb hold a valid (clamped) diagonal and a zero rotation: no guard needed
            uint64_t p[MAC_R];
#pragma unroll
            for (int j = 0; j < MAC_R; j++) p[j] = buf[(c + j) * MAC_K + kl];
#pragma unroll
            for (int j = 0; j < MAC_R; j++) asm volatile("" : "+v"(p[j]));  // the group's reads issue together
#pragma unroll
            for (int j = 0; j < MAC_R; j++) {
                smac(sp, (uint32_t)p[j], (uint32_t)(p[j] >> 32), r[c + j]);
                if ((c + j) % SPLIT_CHUNK == SPLIT_CHUNK - 1) snorm(sp);
            }
        }
        uint64_t v = sreduce60(sp, P);
        uint64_t *o = inner + (size_t)g * ctsize + off;
        if (ACC) v = addm(v, *o, P.q);
        if (active) *o = v;
    };
    // the LDS buffer of step g is rewritten at step g + 2, after the barrier of step g + 1
    for (uint32_t g = 0; g < gs; g += 2) {
        step(g, a0, a1);
        if (g + 1 < gs) step(g + 1, b0v, b1v);
    }
}

// ---------------------------------------------------------------------
// The same multiply-accumulate on the matrix cores: for limb i and coefficient k,
//   inner[g][c][i][k] (+)= sum_{bb < nb} P[g][b0 + bb][i][k] R[b0 + bb][c][i][k]  mod q_i,
// a (gs x 32) x (32 x cols) product per (i, k), taken in signed base-256 digits
// (mfma_digits.h): the rows of a 16 x 16 tile are giant steps, its columns the
// ciphertext polynomials c < cols <= 16, the contraction the baby steps.  A
// workgroup takes 16 consecutive coefficients of one limb, wave w the
// coefficients 4w .. 4w + 3.  Every global access is a 128-byte run of 16
// coefficients, turned in one LDS buffer: first the rotations (whose digit
// planes then stay in registers), then per tile of 16 giant steps the diagonals
// (16 x 32 x 16 values), read back in the operand layout, and the tile's sums on
// their way out.  Two workgroups share a CU, so one's loads overlap the other's
// products.
// ---------------------------------------------------------------------
constexpr int MM_K = 16;                  // coefficients per workgroup
constexpr int MM_ROW = 34;                // LDS words per staged (k, row) run of 32 + 2 pad
constexpr int MM_SLAB = 16 * MM_ROW + 2;  // LDS words per staged coefficient (16 rows) + 2 pad
constexpr int MM_OC = 17;                 // LDS words per (g, c) row of the sums: 16 + 1 pad

template <bool ACC>
__global__ __launch_bounds__(256, 2) void k_bsgs_mac_mfma(const uint64_t *__restrict__ pt,
                                                           const uint64_t *__restrict__ in,
                                                           const uint64_t *__restrict__ rot,
                                                           uint64_t *__restrict__ inner,
                                                           const uint64_t *__restrict__ prc, uint32_t n, uint32_t l,
                                                           uint32_t bs, uint32_t gs, uint32_t ncols, size_t ctsize,
                                                           uint32_t b0) {
    __shared__ __align__(16) uint64_t sp[MM_K * MM_SLAB];
    const uint32_t i = blockIdx.y, k0 = blockIdx.x * MM_K;
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t col = lane & 15, grp = lane >> 4;
    const uint32_t nb = min(32u, bs - b0);
    const size_t pstride = (size_t)l * n;
    // staging lanes: coefficient k0 + kk_s and runs r_s + 16 mm (r_s < 16)
    const uint32_t kk_s = threadIdx.x % 16, r_s = threadIdx.x / 16;
    uint64_t *const sdst = sp + kk_s * MM_SLAB + r_s;
    // the rotations: run (c = r_s, baby step mm) at sp[k][c][bb]; rows past nb and columns
    // past ncols are zero (their loads clamped)
    {
        const size_t rofs = ((size_t)min(r_s, ncols - 1) * l + i) * n + k0 + kk_s;
        uint64_t x[32];
#pragma unroll
        for (int mm = 0; mm < 32; mm++) {
            const uint32_t b = b0 + min((uint32_t)mm, nb - 1);
            x[mm] = (b == 0 ? in : rot + (size_t)(b - 1) * ctsize)[rofs];
        }
        const bool colok = r_s < ncols;
        uint64_t *d = sp + kk_s * MM_SLAB + r_s * MM_ROW;
#pragma unroll
        for (int mm = 0; mm < 32; mm++) d[mm] = (colok && (uint32_t)mm < nb) ? x[mm] : 0;
    }
    __syncthreads();
    // right operand: digit planes of baby steps 8 grp + j of polynomial col at this wave's 4
    // coefficients (rp[q][a] = plane a), so that mf_right's tuples {plane 2p | plane 2p + 1}
    // are consecutive registers
    long rp[4][8];
#pragma unroll
    for (int qk = 0; qk < 4; qk++) {
        const uint64_t *a = sp + (4 * wave + qk) * MM_SLAB + col * MM_ROW + 8 * grp;
        uint64_t z[8];
#pragma unroll
        for (int j = 0; j < 8; j++) z[j] = digit_form(a[j]);
        long pl[8];
        mf_planes(z, pl);
#pragma unroll
        for (int a2 = 0; a2 < 8; a2++) rp[qk][a2] = pl[a2];
    }
    const MfW2 w2 = mf_w2();
    const MfRecomb rk = mf_recomb_consts([&](int d) -> uint64_t { return prc[(size_t)i * MF_RC + d]; });
    // diagonal runs of a tile: r_s + 16 mm = giant step mm >> 1, baby step r_s + 16 (mm & 1)
    const size_t gstride = (size_t)bs * pstride;
    const uint64_t *pb0 = pt + (size_t)(b0 + min(r_s, nb - 1)) * pstride + (size_t)i * n + k0 + kk_s;
    const uint64_t *pb1 = pt + (size_t)(b0 + min(r_s + 16, nb - 1)) * pstride + (size_t)i * n + k0 + kk_s;
    for (uint32_t g0 = 0; g0 < gs; g0 += 16) {
        __syncthreads();  // sp is free: the previous contents are all read
        {
            uint64_t x[32];
#pragma unroll
            for (int mm = 0; mm < 32; mm++) {
                const size_t g = min(g0 + (uint32_t)(mm >> 1), gs - 1);
                x[mm] = ((mm & 1) ? pb1 : pb0)[g * gstride];
            }
#pragma unroll
            for (int mm = 0; mm < 32; mm++) sdst[(mm >> 1) * MM_ROW + 16 * (mm & 1)] = x[mm];
        }
        __syncthreads();
        uint64_t res[4][4];
#pragma unroll
        for (int qk = 0; qk < 4; qk++) {
            // left operand: giant step g0 + col, baby steps 8 grp + j
            const uint64_t *a = sp + (4 * wave + qk) * MM_SLAB + col * MM_ROW + 8 * grp;
            uint64_t z[8];
#pragma unroll
            for (int j = 0; j < 8; j++) z[j] = digit_form(a[j]);
            long pl[8];
            mf_planes(z, pl);
            mf_v4i AW[MF_NW], H[MF_NT];
            mf_left(pl, AW);
            mf_right(rp[qk], H);
            mf_v4i acc[15];
#pragma unroll
            for (int d = 0; d < 15; d++) acc[d] = mf_v4i{0, 0, 0, 0};
            mf_mac_tile(acc, AW, H);
#pragma unroll
            for (int v = 0; v < 4; v++) res[qk][v] = mf_recombine32(acc, v, w2, rk);  // at most 32 baby steps
        }
        __syncthreads();  // every wave is done with the diagonals
        // the sums of (giant step g0 + 4 grp + v, polynomial col) at sp[(g c)][k]
#pragma unroll
        for (int qk = 0; qk < 4; qk++)
#pragma unroll
            for (int v = 0; v < 4; v++) sp[((4 * grp + v) * 16 + col) * MM_OC + 4 * wave + qk] = res[qk][v];
        __syncthreads();
        // out: polynomial r_s, giant steps g0 + mm
        if (r_s < ncols) {
            uint64_t *ob = inner + ((size_t)r_s * l + i) * n + k0 + kk_s;
#pragma unroll 4
            for (int mm = 0; mm < 16; mm++) {
                if (g0 + mm >= gs) break;
                uint64_t *o = ob + (size_t)(g0 + mm) * ctsize;
                uint64_t v = sp[(mm * 16 + r_s) * MM_OC + kk_s];
                if (ACC) v = addm(v, *o, rk.tq);
                *o = v;
            }
        }
    }
}

__global__ void k_copy(const uint64_t *__restrict__ a, uint64_t *__restrict__ b, size_t total) {
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x)
        b[idx] = a[idx];
}


// =====================================================================
// Key switching core
// =====================================================================
struct KsWs {
    uint64_t *d, *y, *ext, *acc, *conv;
    uint32_t *u, *uP;
    uint64_t *mp;  // transpose buffer of the n > 2048 NTT
};

static size_t ks_words(const ckks_ctx *c, int B, int l, KsWs *w, uint64_t *base) {
    const size_t n = c->n, el = (size_t)l + c->K;
    const size_t beta = (l + c->alpha - 1) / c->alpha;
    size_t off = 0;
    auto take = [&](size_t words) {
        uint64_t *p = base ? base + off : nullptr;
        off += align_words(words);
        return p;
    };
    uint64_t *d = take(B * (size_t)l * n);
    uint64_t *y = take(B * (size_t)l * n);
    uint64_t *ext = take(B * beta * el * n);
    uint64_t *acc = take(B * 2 * el * n);
    uint64_t *conv = take(B * 2 * (size_t)l * n);
    uint64_t *u = take((B * beta * n + 1) / 2);
    uint64_t *uP = take((B * 2 * n + 1) / 2);
    uint64_t *mp = take(mp_scratch_words(c->n));
    if (w) *w = KsWs{d, y, ext, acc, conv, (uint32_t *)u, (uint32_t *)uP, mp};
    return off;
}

// ModUp of d ([B][l][n], NTT domain, ciphertext b at d + b * d_stride):
// fills w.y, w.u and the NTT-domain extended digits w.ext.
// Exact base conversion of `sets` input sets (bases of at most mmax primes)
// onto up to maxt target positions.  The one-chunk conversion (bases of up to
// 31 primes, no summed sets) takes its correction u itself; the others read it
// from k_basis_u.
static inline bool conv_needs_u(uint32_t mmax, uint32_t nsum = 1) { return mmax + 1 > 32 || nsum > 1; }
template <int MODE>
static void launch_convert(const ckks_ctx *c, const BasisDev *bases, const SetLayout &lay, const uint64_t *y,
                           const uint32_t *u, const ConvTargets &ct, uint64_t *out, uint32_t maxt, uint32_t sets,
                           uint32_t mmax, hipStream_t s) {
    const uint32_t n = c->n;
    // every basis of the launch has at most mmax rows: mk = 32 for all or none
    const uint32_t tpb = mmax + 1 > 32 || ct.nsum > 1 ? mf_tpb<2>() : mf_tpb<3>();
    const dim3 grid(n / MF_COEF, ((maxt + 15) / 16 + tpb - 1) / tpb, sets);
    if (mmax + 1 > 32)
        hipLaunchKernelGGL((k_convert_mfma<MODE, 2, false>), grid, dim3(256), 0, s, bases, lay, y, u, ct, out, n,
                           c->d_pc);
    else if (ct.nsum > 1)
        hipLaunchKernelGGL((k_convert_mfma<MODE, 2, true>), grid, dim3(256), 0, s, bases, lay, y, u, ct, out, n,
                           c->d_pc);
    else
        hipLaunchKernelGGL((k_convert_mfma<MODE, 3, true>), grid, dim3(256), 0, s, bases, lay, y, u, ct, out, n,
                           c->d_pc);
}

// gal != 1 (n > 2048): the extended digits come out of their NTT already permuted by that
// automorphism (the own-prime limbs, which the NTT does not touch, stay unpermuted).
static int ks_modup(const ckks_ctx *c, const LevelTables *lt, int B, int l, const uint64_t *d, size_t d_stride, const KsWs &w,
                    hipStream_t s, uint32_t gal = 1) {
    const uint32_t n = c->n, K = c->K, L = c->L, el = l + K, beta = lt->beta;
    int e;
    {  // y = iNTT(d) scaled by [Bhat_i^-1]
        MapBatched m{d, d_stride, w.y, n, (uint32_t)l, lt->d_modup_scale};
        if ((e = launch_ntt(c, m, B * l, true, s, "ks_intt_modup", w.mp))) return e;
    }
    SetLayout lay_up{(size_t)l * n, (size_t)c->alpha * n, 0, beta, 1};
    if (conv_needs_u(c->alpha)) {
        ProfScope ps_(c, "ks_modup_u", s);
        hipLaunchKernelGGL(k_basis_u, dim3((n + 255) / 256, B * beta), dim3(256), 0, s, lt->d_digits, lay_up, w.y,
                           w.u, n, c->d_pc);
        LAUNCH_CHECK();
    }
    {
        ConvTargets ct{(uint32_t)l, L, K, (size_t)beta * el * n, (size_t)el * n};
        const uint32_t maxt = l + K;  // upper bound on targets per digit
        ProfScope ps_(c, "ks_modup_convert", s);
        launch_convert<0>(c, lt->d_digits, lay_up, w.y, w.u, ct, w.ext, maxt, B * beta, c->alpha, s);
    }
    LAUNCH_CHECK();
    {
        MapExt m{w.ext, n, (uint32_t)l, L, K, beta, c->alpha};
        if ((e = launch_ntt(c, m, B * beta * el, false, s, "ks_ntt_ext", w.mp, gal))) return e;
    }
    return CKKS_OK;
}

// Inner product of sigma_g(ModUp(d)) with the key, then ModDown up to the
// NTT-domain conversion: leaves the Q-limbs of the accumulators in w.acc and
// the converted P-part in w.conv; the caller runs the final kernel.
static Steps one_step(const ckks_swk *key, uint32_t g, int B) {
    Steps st{};
    st.key[0] = key->data;
    st.g[0] = g;
    st.count = 1;
    st.B = (uint32_t)B;
    st.shared = 0;
    if (key->seeded) {
        st.seeded = 1;
        st.root[0] = key_seed_root(key->seed);
    }
    return st;
}

// Inner product of sigma_g(ModUp(d)) with the keys of a batch of steps:
// leaves st.count * st.B accumulator pairs in w.acc.
// ext_permuted (generic n, one step): ks_modup already applied the step's automorphism
// to the extended digits, which are then read in place.
static int ks_inner(const ckks_ctx *c, const LevelTables *lt, int l, const uint64_t *d, size_t d_stride, const Steps &st,
                    const KsWs &w, hipStream_t s, bool ext_permuted = false) {
    const uint32_t n = c->n, K = c->K, L = c->L, el = l + K, beta = lt->beta;
    const size_t nout = (size_t)st.count * st.B;
    ProfScope ps_(c, st.shared ? "ks_inner_product_hoisted" : "ks_inner_product", s);
    if (n == 2048 && st.shared && !st.seeded && beta <= HOIST_MAX_BETA) {
        const uint32_t ngroups = (st.count + HOIST_SPW - 1) / HOIST_SPW;
        hipLaunchKernelGGL(k_inner_hoisted2048, dim3(xcd_blocks(el * ngroups, st.B)), dim3(256), 0, s, d, d_stride,
                           w.ext, st, w.acc, c->d_pc, (uint32_t)l, L, K, beta, c->alpha);
    } else if (n == 2048) {
        auto kern = st.seeded ? k_inner2048<true> : k_inner2048<false>;
        hipLaunchKernelGGL(kern, dim3(xcd_blocks(st.count * el, st.B)), dim3(256), 0, s, d, d_stride, w.ext, st,
                           w.acc, c->d_pc, (uint32_t)l, L, K, beta, c->alpha, 0u, el);
    } else {  // generic n: one launch per step
        if (ext_permuted && st.count != 1) return CKKS_EINVAL;
        auto kern = st.seeded ? k_inner<true> : k_inner<false>;
        for (uint32_t j = 0; j < st.count; j++) {
            const size_t in_off = st.shared ? 0 : (size_t)j * st.B;
            hipLaunchKernelGGL(kern, grid_for((size_t)el * n), dim3(256), 0, s, d + in_off * d_stride, d_stride,
                               w.ext + in_off * beta * el * n, st.key[j], w.acc + (size_t)j * st.B * 2 * el * n,
                               c->d_pc, n, (uint32_t)l, L, K, beta, c->alpha, st.g[j], ext_permuted ? 1u : st.g[j],
                               st.root[j], st.B);
        }
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

// Giant-step inner products of a batch (n = 2048), x = the steps' input
// ciphertexts (c0 at x + cb x_stride, c1 one polynomial further): the P-limbs
// of every step go to w.acc as usual, the Q-limbs are summed over the steps
// into *nparts partial sums (k_inner_sum2048).
static int ks_inner_giant(const ckks_ctx *c, const LevelTables *lt, int l, const uint64_t *x, size_t x_stride, const Steps &st,
                          const KsWs &w, uint32_t *nparts, hipStream_t s) {
    const uint32_t K = c->K, L = c->L, beta = lt->beta;
    const size_t per = (size_t)l * c->n;
    {
        ProfScope ps_(c, "ks_inner_product", s);
        hipLaunchKernelGGL(k_inner2048<false>, dim3(xcd_blocks(st.count * K, st.B)), dim3(256), 0, s, x + per, x_stride,
                           w.ext, st, w.acc, c->d_pc, (uint32_t)l, L, K, beta, c->alpha, (uint32_t)l, K);
    }
    LAUNCH_CHECK();
    // up to 4 partial sums: enough workgroups to fill the chip at ~1 wave per SIMD each
    const uint32_t parts = std::min(st.count, 4u), spp = (st.count + parts - 1) / parts;
    *nparts = (st.count + spp - 1) / spp;
    {
        ProfScope ps_(c, "ks_inner_product_sum", s);
        hipLaunchKernelGGL(k_inner_sum2048, dim3(xcd_blocks(*nparts * l, st.B)), dim3(256), 0, s, x + per, x_stride,
                           x, x_stride, w.ext, st, spp, *nparts, w.acc, c->d_pc, c->d_pmod, (uint32_t)l, K, L, beta,
                           c->alpha);
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

// ModDown of nout accumulator pairs up to the converted P-part in w.conv, in
// coefficient form: the final kernels transform it (k_final2048, or the fused
// row pass of moddown_final_mp).
// With nsum > 1 the conversions of accumulators o + j (nout / nsum), j < nsum,
// are summed (n = 2048 giant steps) in *nparts partial sums: part p of output
// o at w.conv pair p (nout / nsum) + o.
static int ks_moddown_conv(const ckks_ctx *c, size_t nout, int l, const KsWs &w, hipStream_t s, uint32_t nsum = 1,
                           uint32_t *nparts = nullptr) {
    const uint32_t n = c->n, K = c->K, L = c->L, el = l + K;
    int e;
    {
        MapAccP m{w.acc, n, (uint32_t)l, L, K, c->d_moddown_scale};
        if ((e = launch_ntt(c, m, (int)(nout * 2 * K), true, s, "ks_intt_moddown", w.mp))) return e;
    }
    SetLayout lay_dn{(size_t)el * n, 0, (size_t)l * n, 1, 0};
    if (conv_needs_u(K, nsum)) {
        ProfScope ps_(c, "ks_moddown_u", s);
        hipLaunchKernelGGL(k_basis_u, dim3((n + 255) / 256, (unsigned)(nout * 2)), dim3(256), 0, s, c->d_pbasis,
                           lay_dn, w.acc, w.uP, n, c->d_pc);
        LAUNCH_CHECK();
    }
    {
        ConvTargets ct{(uint32_t)l, L, K, (size_t)l * n, 0};
        // lay_dn.inner == 1: the summed sets are evenly spaced, as k_convert_mfma assumes
        ct.nsum = nsum;
        ct.sum_stride = (uint32_t)(nout / nsum * 2);
        // up to 4 parts: long summed workgroups need enough of them to fill the chip
        const uint32_t parts = std::min(nsum, 4u);
        ct.spp = (nsum + parts - 1) / parts;
        const uint32_t np = (nsum + ct.spp - 1) / ct.spp;
        if (nparts) *nparts = np;
        ProfScope ps_(c, "ks_moddown_convert", s);
        launch_convert<1>(c, c->d_pbasis, lay_dn, w.acc, w.uP, ct, w.conv, (uint32_t)l, np * ct.sum_stride, c->K, s);
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

// ModRaise: the exact centered lift of every coefficient from the primes
// [0, l0) to the primes [0, lt) (bootstrapping's first step): scaled iNTT of
// the l0 limbs, exact u, conversion to every target, NTT of the lt limbs.
size_t ws_bytes_mod_raise(const ckks_ctx *c, int B, int l0) {
    return (align_words((size_t)2 * B * l0 * c->n) + align_words(((size_t)2 * B * c->n + 1) / 2) +
            mp_scratch_words(c->n)) * 8;
}

int op_mod_raise(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l0, int lt, void *ws,
                 hipStream_t s) {
    int e = CKKS_OK;
    const RaiseTables *rt = find_raise(c, (uint32_t)l0);
    if (!rt) return CKKS_ENOTREADY;
    const uint32_t n = c->n, P = 2 * (uint32_t)B;
    uint64_t *y = (uint64_t *)ws;
    uint32_t *u = (uint32_t *)(y + align_words((size_t)P * l0 * n));
    uint64_t *mp = y + align_words((size_t)P * l0 * n) + align_words(((size_t)P * n + 1) / 2);
    {
        MapBatched m{in, (size_t)l0 * n, y, n, (uint32_t)l0, rt->d_scale};
        if ((e = launch_ntt(c, m, (int)(P * l0), true, s, "raise_intt", mp))) return e;
    }
    SetLayout lay{(size_t)l0 * n, 0, 0, 1, 0};
    if (conv_needs_u((uint32_t)l0)) {
        ProfScope ps_(c, "raise_u", s);
        hipLaunchKernelGGL(k_basis_u, dim3((n + 255) / 256, P), dim3(256), 0, s, rt->d_basis, lay, y, u, n,
                           c->d_pc);
        LAUNCH_CHECK();
    }
    {
        ConvTargets ct{(uint32_t)lt, c->L, c->K, (size_t)lt * n, 0};
        ProfScope ps_(c, "raise_convert", s);
        launch_convert<1>(c, rt->d_basis, lay, y, u, ct, out, (uint32_t)lt, P, (uint32_t)l0, s);
    }
    LAUNCH_CHECK();
    MapStrided m2{out, out, n, (uint32_t)lt, 0, nullptr};
    return launch_ntt(c, m2, (int)(P * lt), false, s, "raise_ntt", mp);
}

size_t ws_bytes_relin(const ckks_ctx *c, int B, int l) { return ks_words(c, B, l, nullptr, nullptr) * 8; }
size_t ws_bytes_rotate(const ckks_ctx *c, int B, int l) { return ks_words(c, B, l, nullptr, nullptr) * 8; }
size_t ws_bytes_rescale(const ckks_ctx *c, int B, int l) {
    return (align_words((size_t)B * 2 * c->n) + align_words((size_t)B * 2 * (l - 1) * c->n) +
            mp_scratch_words(c->n)) * 8;
}

// Steps per batched key switch inside BSGS: as many as fit a workspace budget.
constexpr size_t BSGS_KS_BUDGET = 8ull << 30;
static int bsgs_chunk(const ckks_ctx *c, int B, int l, int bs, int gs) {
    if (c->n != 2048) return 1;
    const size_t per = ks_words(c, B, l, nullptr, nullptr) * 8;
    int sc = (int)std::max<size_t>(1, BSGS_KS_BUDGET / std::max<size_t>(per, 1));
    // a giant batch sums sc conversions of K inputs each: sc K <= 1000 keeps it in 128 bits
    sc = std::min<int>(sc, (int)std::max<uint32_t>(1, 1000 / std::max<uint32_t>(c->K, 1)));
    return std::max(1, std::min({sc, MAX_STEPS, std::max(bs, gs) - 1}));
}
static size_t bsgs_words(const ckks_ctx *c, int B, int l, int bs, int gs) {
    const size_t ct = (size_t)B * 2 * l * c->n;
    const int sc = bsgs_chunk(c, B, l, bs, gs);
    return align_words(ct * (bs - 1)) + align_words(ct * gs) + ks_words(c, sc * B, l, nullptr, nullptr) +
           ws_bytes_rescale(c, B, l) / 8;
}
size_t ws_bytes_bsgs(const ckks_ctx *c, int B, int l, int bs, int gs) { return bsgs_words(c, B, l, bs, gs) * 8; }

int op_mul_tensor_relin(const ckks_ctx *c, const uint64_t *a, const uint64_t *b, const ckks_swk *rlk, uint64_t *out,
                        int B, int l, void *ws, hipStream_t s) {
    int e = CKKS_OK;
    const LevelTables *lt = find_level(c, l);
    if (!lt) return CKKS_ENOTREADY;
    KsWs w;
    ks_words(c, B, l, &w, (uint64_t *)ws);
    const uint32_t n = c->n;
    size_t tot = (size_t)B * l * n;
    {
        ProfScope ps_(c, "relin_tensor_d2", s);
        hipLaunchKernelGGL(k_prep_relin, grid_for(tot), dim3(256), 0, s, a, b, w.d, c->d_pc, n, (uint32_t)l, tot);
    }
    LAUNCH_CHECK();
    const size_t per = (size_t)l * n;
    const Steps st = one_step(rlk, 1, B);
    if ((e = ks_modup(c, lt, B, l, w.d, per, w, s))) return e;
    if ((e = ks_inner(c, lt, l, w.d, per, st, w, s))) return e;
    if ((e = ks_moddown_conv(c, B, l, w, s))) return e;
    {
        ProfScope ps_(c, "relin_final", s);
        if (n == 2048)
            hipLaunchKernelGGL((k_final2048<1, false>), dim3(B * 2 * l), dim3(256), 0, s, w.acc, w.conv, c->d_pinv,
                               c->d_pc, c->d_tw_fwd, a, b, st, out, (uint32_t)l, c->K);
        else if ((e = moddown_final_mp<1, false>(c, w.conv, w.acc, w.mp, B, l, a, b, 0u, out, s)))
            return e;
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

// Final kernel of a batch of rotations: out[cb] (+)= (acc - conv) P^-1 + (sigma_g(c0), 0).
static int rotate_final(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int l, const Steps &st, const KsWs &w,
                        bool accumulate, hipStream_t s) {
    const size_t nout = (size_t)st.count * st.B;
    const uint64_t *nul = nullptr;
    ProfScope ps_(c, accumulate ? "rotate_final_acc" : "rotate_final", s);
    if (c->n == 2048) {
        if (accumulate)
            hipLaunchKernelGGL((k_final2048<2, true>), dim3(nout * 2 * l), dim3(256), 0, s, w.acc, w.conv,
                               c->d_pinv, c->d_pc, c->d_tw_fwd, in, nul, st, out, (uint32_t)l, c->K);
        else
            hipLaunchKernelGGL((k_final2048<2, false>), dim3(nout * 2 * l), dim3(256), 0, s, w.acc, w.conv,
                               c->d_pinv, c->d_pc, c->d_tw_fwd, in, nul, st, out, (uint32_t)l, c->K);
    } else {  // larger rings: single step
        const int e = accumulate ? moddown_final_mp<2, true>(c, w.conv, w.acc, w.mp, nout, l, in, nul, st.g[0], out, s)
                                 : moddown_final_mp<2, false>(c, w.conv, w.acc, w.mp, nout, l, in, nul, st.g[0], out, s);
        if (e) return e;
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

// Rotation: ModUp of c1 as stored (no permuted copy).  At n = 2048 the automorphism
// is a gather of the extended digits inside the key inner product; for larger rings
// the row pass of the extended digits' NTT writes them permuted (a gather there
// would touch a different line per residue), and only the digit's own limbs, read
// from c1, are gathered.
int op_rotate(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, uint32_t g, const ckks_swk *key,
              void *ws, bool accumulate, hipStream_t s) {
    int e = CKKS_OK;
    const LevelTables *lt = find_level(c, l);
    if (!lt) return CKKS_ENOTREADY;
    KsWs w;
    ks_words(c, B, l, &w, (uint64_t *)ws);
    const size_t per = (size_t)l * c->n;
    const uint64_t *c1 = in + per;
    const Steps st = one_step(key, g, B);
    const bool fold = c->n > 2048;
    if ((e = ks_modup(c, lt, B, l, c1, 2 * per, w, s, fold ? g : 1u))) return e;
    if ((e = ks_inner(c, lt, l, c1, 2 * per, st, w, s, fold))) return e;
    if ((e = ks_moddown_conv(c, B, l, w, s))) return e;
    return rotate_final(c, in, out, l, st, w, accumulate, s);
}

// Seed-expanded key -> stored format: out[j][0] = b[j], out[j][1][i][k] = the
// seeded a-part residue of (digit j, key prime i).
__global__ void k_key_expand(const uint64_t *__restrict__ kb, uint64_t *__restrict__ out,
                             const PrimeConsts *__restrict__ pc, uint32_t n, uint32_t tot, uint64_t root,
                             size_t total) {
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const uint32_t k = idx % n;
        const size_t row = idx / n;  // j * tot + i
        const uint32_t i = row % tot;
        const size_t j = row / tot;
        out[((j * 2 + 0) * tot + i) * n + k] = kb[idx];
        out[((j * 2 + 1) * tot + i) * n + k] = seeded_a(sm_at(root, row), k, pc[i].q);
    }
}

int op_key_expand(const ckks_ctx *c, const ckks_swk *key, uint64_t *key_out, hipStream_t s) {
    const uint32_t tot = c->L + c->K;
    const size_t total = (size_t)c->dnum * tot * c->n;
    hipLaunchKernelGGL(k_key_expand, grid_for(total), dim3(256), 0, s, key->data, key_out, c->d_pc, c->n, tot,
                       key_seed_root(key->seed), total);
    LAUNCH_CHECK();
    return CKKS_OK;
}

int op_rescale(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, void *ws, hipStream_t s) {
    int e = CKKS_OK;
    const LevelTables *lt = find_level(c, l);
    if (!lt) return CKKS_ENOTREADY;
    const uint32_t n = c->n;
    uint64_t *t = (uint64_t *)ws;
    uint64_t *r = t + align_words((size_t)B * 2 * n);
    uint64_t *mp = r + align_words((size_t)B * 2 * (l - 1) * n);
    // t[b][c] = iNTT(in[b][c][l-1])
    {
        MapLast ml{in, t, n, (uint32_t)l};
        if ((e = launch_ntt(c, ml, B * 2, true, s, "rescale_intt", mp))) return e;
    }
    size_t tot = (size_t)B * 2 * (l - 1) * n;
    if (n == 2048) {
        ProfScope ps_(c, "rescale_final", s);
        hipLaunchKernelGGL(k_rescale2048, dim3(B * 2 * (l - 1)), dim3(256), 0, s, in, t, lt->d_rescale_inv, c->d_pc,
                           c->d_tw_fwd, out, (uint32_t)l);
        LAUNCH_CHECK();
        return CKKS_OK;
    }
    {
        ProfScope ps_(c, "rescale_lift", s);
        hipLaunchKernelGGL(k_rescale_lift, grid_for(tot), dim3(256), 0, s, t, r, c->d_pc, n, (uint32_t)l, tot);
    }
    LAUNCH_CHECK();
    {
        MapStrided m{r, r, n, (uint32_t)(l - 1), 0, nullptr};
        if ((e = launch_ntt(c, m, B * 2 * (l - 1), false, s, "rescale_ntt", mp))) return e;
    }
    {
        ProfScope ps_(c, "rescale_final", s);
        hipLaunchKernelGGL(k_rescale_final, grid_for(tot), dim3(256), 0, s, in, r, lt->d_rescale_inv, c->d_pc, out, n,
                           (uint32_t)l, tot);
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

static uint32_t rot_elt(uint32_t n, uint64_t k) {
    uint64_t m = 2ull * n, r = 1, b = 5;
    k %= n / 2;
    for (; k; k >>= 1, b = b * b % m)
        if (k & 1) r = r * b % m;
    return (uint32_t)r;
}

int op_bsgs(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int B, int l, const uint64_t *diags, int bs, int gs,
            const ckks_swk *const *baby, const ckks_swk *const *giant, bool rescale, void *ws, hipStream_t s) {
    const size_t ct = (size_t)B * 2 * l * c->n;
    const size_t per = (size_t)l * c->n;
    const int sc = bsgs_chunk(c, B, l, bs, gs);
    uint64_t *rot = (uint64_t *)ws;
    uint64_t *inner = rot + align_words(ct * (bs - 1));
    uint64_t *ksws = inner + align_words(ct * gs);
    uint64_t *rsws = ksws + ks_words(c, sc * B, l, nullptr, nullptr);
    int e = CKKS_OK;
    const LevelTables *lt = find_level(c, l);
    if (!lt) return CKKS_ENOTREADY;
    KsWs w;
    ks_words(c, sc * B, l, &w, ksws);
    if (bs > 1) {
        // baby steps hoisted: one ModUp of c1, then batches of steps sharing it
        if ((e = ks_modup(c, lt, B, l, in + per, 2 * per, w, s))) return e;
        for (int b0 = 1; b0 < bs; b0 += sc) {
            Steps st{};
            st.count = (uint32_t)std::min(sc, bs - b0);
            st.B = (uint32_t)B;
            st.shared = 1;
            for (uint32_t j = 0; j < st.count; j++) {
                st.key[j] = baby[b0 + j]->data;
                st.g[j] = rot_elt(c->n, b0 + j);
            }
            if ((e = ks_inner(c, lt, l, in + per, 2 * per, st, w, s))) return e;
            if ((e = ks_moddown_conv(c, (size_t)st.count * B, l, w, s))) return e;
            if ((e = rotate_final(c, in, rot + (size_t)(b0 - 1) * ct, l, st, w, false, s))) return e;
        }
    }
    for (int b0 = 0; b0 < bs; b0 += MAC_B) {
        ProfScope ps_(c, "bsgs_mac", s);
        if (2 * B <= 16) {  // the polynomials fit the columns of one matrix-core tile
            const dim3 grid(c->n / MM_K, l);
            hipLaunchKernelGGL(b0 ? k_bsgs_mac_mfma<true> : k_bsgs_mac_mfma<false>, grid, dim3(256), 0, s, diags, in,
                               rot, inner, c->d_prc, c->n, (uint32_t)l, (uint32_t)bs, (uint32_t)gs, (uint32_t)(2 * B),
                               ct, (uint32_t)b0);
        } else {
            const dim3 grid(c->n / MAC_K, l, (2 * B + MAC_C - 1) / MAC_C);
            const bool full = (2 * B) % MAC_C == 0;
            auto kern = b0 ? (full ? k_bsgs_mac<true, true> : k_bsgs_mac<false, true>)
                           : (full ? k_bsgs_mac<true, false> : k_bsgs_mac<false, false>);
            hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, diags, in, rot, inner, c->d_pc, c->n, (uint32_t)l,
                               (uint32_t)bs, (uint32_t)gs, (uint32_t)(2 * B), ct, (uint32_t)b0);
        }
        LAUNCH_CHECK();
    }
    // giant steps: batches of independent rotations of inner[g], summed into inner[0]
    for (int g0 = 1; g0 < gs; g0 += sc) {
        Steps st{};
        st.count = (uint32_t)std::min(sc, gs - g0);
        st.B = (uint32_t)B;
        st.shared = 0;
        for (uint32_t j = 0; j < st.count; j++) {
            st.key[j] = giant[g0 + j]->data;
            st.g[j] = rot_elt(c->n, (uint64_t)(g0 + j) * bs);
        }
        const uint64_t *src = inner + (size_t)g0 * ct;  // ciphertexts (g0 + j, b), consecutive
        const int nb = (int)st.count * B;
        if (c->n == 2048) {
            uint32_t nparts = 0, nconv = 0;
            if ((e = ks_modup(c, lt, nb, l, src + per, 2 * per, w, s))) return e;
            if ((e = ks_inner_giant(c, lt, l, src, 2 * per, st, w, &nparts, s))) return e;
            if ((e = ks_moddown_conv(c, nb, l, w, s, st.count, &nconv))) return e;
            ProfScope ps_(c, "giant_final", s);
            hipLaunchKernelGGL(k_final_giant2048, dim3(B * 2 * l), dim3(256), 0, s, w.acc, w.conv, c->d_pinv,
                               c->d_pc, c->d_tw_fwd, nparts, nconv, (uint32_t)B, inner, (uint32_t)l, c->K);
            LAUNCH_CHECK();
        } else {
            for (uint32_t j = 0; j < st.count; j++)
                if ((e = op_rotate(c, src + (size_t)j * ct, inner, B, l, st.g[j], giant[g0 + j], ksws, true, s)))
                    return e;
        }
    }
    if (rescale) return op_rescale(c, inner, out, B, l, rsws, s);
    {
        ProfScope ps_(c, "copy", s);
        hipLaunchKernelGGL(k_copy, grid_for(ct), dim3(256), 0, s, inner, out, ct);
    }
    LAUNCH_CHECK();
    return CKKS_OK;
}

}  // namespace ckks
