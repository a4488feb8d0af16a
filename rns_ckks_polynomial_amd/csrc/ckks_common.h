// ckks_common.h -- device arithmetic and table layouts shared by the kernels.
//
// All moduli are primes in (2^59, 2^60) with q = 1 (mod 2n) (the 60-bit RNS
// primes of the Kestrel relay README, section 1).  Residues at API boundaries
// are fully reduced to [0, q).  Inside kernels values may be "lazy" in
// [0, 2q) or [0, 4q) (4q < 2^62).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_tables.h"  // PrimeConsts, MF_RC

namespace ckks {

typedef unsigned __int128 u128;

// Loads through table pointers that the kernels read from device structs (BasisDev):
// such pointers are generic to the compiler, which then emits flat loads; these count
// against the LDS counter as well, so every LDS wait also waits for them.  Reading
// through the global address space gives global loads.
template <class T>
__device__ __forceinline__ T gload(const T *p) {
    return *(const T __attribute__((address_space(1))) *)p;
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ scalar
__device__ __forceinline__ uint64_t mulhi64(uint64_t a, uint64_t b) { return __umul64hi(a, b); }

// Shoup product: w < q, wp = floor(w 2^64 / q), any 64-bit x -> x w mod q in [0, 2q).
__device__ __forceinline__ uint64_t shoup_lazy(uint64_t x, uint64_t w, uint64_t wp, uint64_t q) {
    return x * w - mulhi64(x, wp) * q;
}
__device__ __forceinline__ uint64_t csub(uint64_t x, uint64_t q) { return x >= q ? x - q : x; }

// Shoup product with the quotient floor(y wp / 2^64) truncated to the three
// high 32x32 partial products: the dropped carries make it at most 2 too
// small, so y w - Q q lands in [0, 4q) (instead of [0, 2q)) for any 64-bit y.
// The remainder is formed as y w + Q (2^64 - q) mod 2^64 (nq = 2^64 - q), so
// the subtraction rides on the multiply-adds.
__device__ __forceinline__ uint64_t shoup_lazy4(uint64_t y, uint64_t w, uint64_t wp, uint64_t nq) {
    const uint32_t yl = (uint32_t)y, yh = (uint32_t)(y >> 32);
    const uint32_t pl = (uint32_t)wp, ph = (uint32_t)(wp >> 32);
    // the two high halves are summed with an explicit carry (add, add-with-carry) into the
    // 64-bit addend of the yh ph multiply-add, instead of two zero-extended 64-bit adds
    uint32_t c;
    const uint32_t hs = __builtin_addc(__umulhi(yh, pl), __umulhi(yl, ph), 0u, &c);
    const uint64_t qt = (uint64_t)yh * ph + (((uint64_t)c << 32) | hs);
    const uint32_t ql = (uint32_t)qt, qh = (uint32_t)(qt >> 32);
    const uint32_t wl = (uint32_t)w, wh = (uint32_t)(w >> 32);
    const uint32_t nl = (uint32_t)nq, nh = (uint32_t)(nq >> 32);
    const uint64_t r = (uint64_t)ql * nl + (uint64_t)yl * wl;  // mod 2^64
    // the high word is a 32-bit sum (the empty asm keeps it from being rewritten as a
    // 64-bit add of a shifted value)
    uint32_t rh = (uint32_t)(r >> 32);
    asm("" : "+v"(rh));
    const uint32_t hi = rh + yl * wh + yh * wl + ql * nh + qh * nl;
    return ((uint64_t)hi << 32) | (uint32_t)r;
}

// x mod q for x < 2^64 - 2^59 with q in (2^59, 2^59 + 2^52) (every chain prime): x >> 59 is
// floor(x / q) or one more, so x - (x >> 59) q lies in [-q, q) and one conditional add of q
// finishes.  nq = 2^64 - q.
__device__ __forceinline__ uint64_t reduce59(uint64_t x, uint64_t q, uint64_t nq) {
    const uint32_t qt = (uint32_t)(x >> 59);
    const int64_t r = (int64_t)(x + (uint64_t)qt * nq);
    return r < 0 ? (uint64_t)r + q : (uint64_t)r;
}

// x - c if x >= c else x, for x, c < 2^63 with |x - c| < 2^63 (nc = 2^64 - c): add, then select on the sign.
__device__ __forceinline__ uint64_t csub_sign(uint64_t x, uint64_t nc) {
    const uint64_t m = x + nc;
    return (int64_t)m < 0 ? x : m;
}

__device__ __forceinline__ uint64_t shoup(uint64_t x, uint64_t w, uint64_t wp, uint64_t q) {
    return csub(shoup_lazy(x, w, wp, q), q);
}
__device__ __forceinline__ uint64_t addm(uint64_t a, uint64_t b, uint64_t q) { return csub(a + b, q); }
__device__ __forceinline__ uint64_t subm(uint64_t a, uint64_t b, uint64_t q) { return a >= b ? a - b : a + q - b; }

// Barrett product for a, b < q, q in (2^59, 2^60), mu = floor(2^122 / q).
// With p = a b < 2^120, qhat = floor((p >> 58) mu / 2^64) is within 1 of
// floor(p / q), so one conditional subtraction finishes.
__device__ __forceinline__ uint64_t mulm(uint64_t a, uint64_t b, uint64_t q, uint64_t mu) {
    u128 p = (u128)a * b;
    uint64_t x1 = (uint64_t)(p >> 58);
    uint64_t qh = mulhi64(x1, mu);
    uint64_t r = (uint64_t)p - qh * q;
    return csub(r, q);
}

// Reduce a 128-bit value (hi:lo) modulo q: hi 2^64 + lo = shoup(hi, 2^64 mod q) + shoup(lo, 1).
__device__ __forceinline__ uint64_t reduce128(uint64_t lo, uint64_t hi, const PrimeConsts &c) {
    uint64_t a = shoup_lazy(hi, c.r64, c.r64p, c.q);  // [0, 2q)
    uint64_t b = lo - mulhi64(lo, c.m64) * c.q;       // [0, 2q)
    uint64_t s = a + b;                               // [0, 4q)
    s = s >= 2 * c.q ? s - 2 * c.q : s;
    return csub(s, c.q);
}

struct Acc128 {
    uint64_t lo, hi;
};
__device__ __forceinline__ void mac(Acc128 &acc, uint64_t a, uint64_t b) {
    u128 p = (u128)a * b;
    u128 s = ((u128)acc.hi << 64 | acc.lo) + p;
    acc.lo = (uint64_t)s;
    acc.hi = (uint64_t)(s >> 64);
}

// Split-operand multiply-accumulate for sums of many 60-bit products.
// With x = xa 2^30 + xb (xb < 2^30), four 64-bit partial sums
//   a0 += xb yb,  a1 += xb ya,  a1b += xa yb,  a2 += xa ya
// are each one v_mad_u64_u32 per product (independent chains, no carry
// handling): for operands below 2^59 + 2^52 (every chain prime is), 15
// products fit in 64 bits.  sflush folds a0 + (a1 + a1b) 2^30 + a2 2^60 into a
// 128-bit accumulator.
constexpr uint64_t M30 = (1ull << 30) - 1;
constexpr int SPLIT_CHUNK = 15;
struct Split3 {
    uint64_t a0, a1, a1b, a2;
};
__device__ __forceinline__ uint64_t split30(uint64_t v) { return (v & M30) | ((v >> 30) << 32); }
__device__ __forceinline__ void smac(Split3 &s, uint32_t xb, uint32_t xa, uint64_t ysplit) {
    const uint32_t yb = (uint32_t)ysplit, ya = (uint32_t)(ysplit >> 32);
    s.a0 += (uint64_t)xb * yb;
    s.a1 += (uint64_t)xb * ya;
    s.a1b += (uint64_t)xa * yb;
    s.a2 += (uint64_t)xa * ya;
}
// Three-sum variant (a1 takes both middle products): two fewer VGPRs per sum,
// for kernels whose occupancy is register-bound.
struct Split3c {
    uint64_t a0, a1, a2;
};
__device__ __forceinline__ void smac(Split3c &s, uint32_t xb, uint32_t xa, uint64_t ysplit) {
    const uint32_t yb = (uint32_t)ysplit, ya = (uint32_t)(ysplit >> 32);
    s.a0 += (uint64_t)xb * yb;
    s.a1 += (uint64_t)xb * ya + (uint64_t)xa * yb;
    s.a2 += (uint64_t)xa * ya;
}
__device__ __forceinline__ void sflush(Acc128 &acc, Split3c &s) {
    u128 v = ((u128)acc.hi << 64 | acc.lo) + s.a0 + ((u128)s.a1 << 30) + ((u128)s.a2 << 60);
    acc.lo = (uint64_t)v;
    acc.hi = (uint64_t)(v >> 64);
    s.a0 = s.a1 = s.a2 = 0;
}
__device__ __forceinline__ void sflush(Acc128 &acc, Split3 &s) {
    u128 v = ((u128)acc.hi << 64 | acc.lo) + s.a0 + ((u128)s.a1 << 30) + ((u128)s.a1b << 30) + ((u128)s.a2 << 60);
    acc.lo = (uint64_t)v;
    acc.hi = (uint64_t)(v >> 64);
    s.a0 = s.a1 = s.a1b = s.a2 = 0;
}

// Carry normalisation inside the 64-bit lanes (value-preserving):
// afterwards a0, a1 < 2^30 and a1b = 0, so 15 more smac fit before the next
// snorm; a2 (weight 2^60) gains below 2^62 per round, so a full reduction
// (sreduce) is due at least every 4 rounds.
__device__ __forceinline__ void snorm(Split3 &s) {
    s.a1 += s.a1b + (s.a0 >> 30);
    s.a0 &= M30;
    s.a1b = 0;
    s.a2 += s.a1 >> 30;
    s.a1 &= M30;
}
// The 128-bit value a0 + 2^30 (a1 + a1b) + 2^60 (a2 + hi).
__device__ __forceinline__ Acc128 sfinal(const Acc128 &hi, Split3 s) {
    snorm(s);
    const u128 h = ((u128)hi.hi << 64 | hi.lo) + s.a2;
    const u128 v = (h << 60) + (s.a0 | (s.a1 << 30));
    return Acc128{(uint64_t)v, (uint64_t)(v >> 64)};
}
// Three-sum form: a1 takes two products per smac, so at most 15 smac between
// snorm; a2 stays below 2^64 for up to 60 smac.
__device__ __forceinline__ void snorm(Split3c &s) {
    s.a1 += s.a0 >> 30;
    s.a0 &= M30;
    s.a2 += s.a1 >> 30;
    s.a1 &= M30;
}
// a0 + 2^30 (a1 + a1b) + 2^60 a2 mod q for a split sum kept within the
// snorm / sreduce bounds (a2 < 2^64): after snorm the low part is below 2^60 < 2q.
template <class S>
__device__ __forceinline__ uint64_t sreduce60(S s, const PrimeConsts &P) {
    snorm(s);
    uint64_t r = shoup_lazy(s.a2, P.r60, P.r60p, P.q) + (s.a0 | (s.a1 << 30));  // < 4q
    r = r >= 2 * P.q ? r - 2 * P.q : r;
    return csub(r, P.q);
}

// Full reduction of a split sum modulo P.q, left in normalised split form
// (a0, a1 < 2^30, a2 = 0): restarts the growth bounds of snorm.
__device__ __forceinline__ void sreduce(Split3 &s, const PrimeConsts &P) {
    const Acc128 v = sfinal(Acc128{0, 0}, s);
    const uint64_t r = reduce128(v.lo, v.hi, P);
    s = Split3{r & M30, r >> 30, 0, 0};
}
__device__ __forceinline__ void sreduce(Split3c &s, const PrimeConsts &P) {
    const uint64_t r = sreduce60(s, P);
    s = Split3c{r & M30, r >> 30, 0};
}

// ------------------------------------------------------------------ tables
// Exact base conversion from a contiguous run of primes (a "basis": one
// key-switching digit, or the special primes P) to any other chain prime.
// The centered CRT value x_c of residues x_i modulo B = prod b_i is
//   x_c = sum_i y_i Bhat_i - u B,   y_i = [x_i Bhat_i^-1]_{b_i},
//   u = round(sum_i y_i / b_i)  (= floor(sum) + [x > (B-1)/2]).
struct BasisDev {
    uint32_t m;            // number of primes in the basis
    uint32_t first;        // global index of the first basis prime
    uint32_t ntot;         // number of chain primes (L + K)
    uint32_t pad;
    const uint64_t *inv_hat;  // [m][2]  Shoup pair of [Bhat_i^-1]_{b_i}
    const uint64_t *hat_mod;  // [m][2]  Shoup pair of [Bhat_i]_{b_i}   (recovers x_i from y_i)
    const uint64_t *R;        // [m]     floor(2^123 / b_i)                (fixed-point 1/b_i)
    const uint64_t *garner;   // [m][m][2]  Shoup pair of b_k^-1 mod b_i (k < i used)
    const uint64_t *half;     // [m]        mixed-radix digits of (B-1)/2
    // Conversion tables.  Target positions: for a chain digit, the special primes
    // first, then the chain primes outside the digit (so the targets at any level
    // are a prefix); for the special basis or a chain prefix, the chain primes.
    // Rows r < mk (mk = m + 1 rounded up to 32): r < m is [Bhat_r]_t, r = m is
    // [-B]_t (the u row), the rest zero.
    //   HD[p][b][r]: signed base-256 digit b of row r's value at target position p
    //               (positions padded to a multiple of 32 with zero digits);
    //   RC[p][MF_RC]: the target's reduction constants (see k_convert_mfma).
    const int8_t *HD;
    const uint64_t *RC;
    uint32_t mk;
};
// Signed base-256 digits of a value below 2^63: byte a of digit_form(v), read as
// an int8, is d_a with v = sum_a d_a 256^a and -128 <= d_a <= 127 (adding 128 in
// every byte position, then flipping each byte's top bit, subtracts it back).
__host__ __device__ __forceinline__ uint64_t digit_form(uint64_t v) {
    return (v + 0x8080808080808080ull) ^ 0x8080808080808080ull;
}
// The value back from its digit form.
__host__ __device__ __forceinline__ uint64_t undigit(uint64_t z) {
    return (z ^ 0x8080808080808080ull) - 0x8080808080808080ull;
}
constexpr uint32_t MF_MAX_ROWS = 2048;  // |S_s| <= 8 rows 2^14 <= 2^28

// ------------------------------------------------------------------ SplitMix64
// Counter-based generator (G. Steele, D. Lea, C. Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014): output i (i = 0, 1, ...) of the
// generator seeded with s is mix64(s + (i + 1) gamma).  Used by the seeded fill
// of synthetic inputs and by seed-expanded switching keys.
__host__ __device__ __forceinline__ uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
__host__ __device__ __forceinline__ uint64_t sm_at(uint64_t s, uint64_t i) {
    return sm_mix(s + (i + 1) * 0x9e3779b97f4a7c15ull);
}

// Seed-expanded switching keys: residue k of the a-part row (digit j, key prime
// i) is floor(w q_i / 2^64), w = sm_at(row, k), row = sm_at(root, j (L + K) + i),
// root = sm_at(seed, KEY_SEED_TAG).  One mix and one high product per residue:
// no rejection loop, so a wavefront never diverges.
constexpr uint64_t KEY_SEED_TAG = 10;
inline uint64_t key_seed_root(uint64_t seed) { return sm_at(seed, KEY_SEED_TAG); }
__device__ __forceinline__ uint64_t seeded_a(uint64_t row, uint32_t k, uint64_t q) {
    return mulhi64(sm_at(row, k), q);
}

}  // namespace ckks
