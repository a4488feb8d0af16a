// mfma_digits.h -- exact sums of products of residues on the int8 matrix cores.
//
// A value below 2^63 is written in signed base-256 digits (digit_form), so a sum
// of products over rows r is
//   sum_r x_r y_r = sum_s 256^s S_s,   S_s = sum_{a+b=s} sum_r dx_a[r] dy_b[r],
// each S_s an exact int32 sum of int8 x int8 products.  One wave computes a
// 16 x 16 tile: lane l supplies row l % 16 of the left operand and column l % 16
// of the right one, each with 8 contraction rows 8 (l / 16) + j (one byte per row
// in every digit plane), and ends with column l % 16 of the rows 4 (l / 16) + v
// (v < 4).  The base conversion and the baby-step giant-step multiply-accumulate
// share these pieces.
#pragma once
#include "ckks_common.h"

namespace ckks {

typedef int mf_v4i __attribute__((ext_vector_type(4)));
typedef long mf_v2l __attribute__((ext_vector_type(2)));

// 4x4 byte transpose: o_b holds byte b of x0, x1, x2, x3 (in that order).
__device__ __forceinline__ void bt4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t &o0, uint32_t &o1,
                                    uint32_t &o2, uint32_t &o3) {
    const uint32_t p01l = __builtin_amdgcn_perm(x1, x0, 0x05010400u), p01h = __builtin_amdgcn_perm(x1, x0, 0x07030602u);
    const uint32_t p23l = __builtin_amdgcn_perm(x3, x2, 0x05010400u), p23h = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
    o0 = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
    o1 = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
    o2 = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
    o3 = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
}

// Digit planes of a lane's 8 rows (z[j] = digit_form of row j): pl[a] holds digit
// a of rows 0..7 in its bytes 0..7.
__device__ __forceinline__ void mf_planes(const uint64_t (&z)[8], long (&pl)[8]) {
    uint32_t o[2][8];
    bt4((uint32_t)z[0], (uint32_t)z[1], (uint32_t)z[2], (uint32_t)z[3], o[0][0], o[0][1], o[0][2], o[0][3]);
    bt4((uint32_t)(z[0] >> 32), (uint32_t)(z[1] >> 32), (uint32_t)(z[2] >> 32), (uint32_t)(z[3] >> 32), o[0][4],
        o[0][5], o[0][6], o[0][7]);
    bt4((uint32_t)z[4], (uint32_t)z[5], (uint32_t)z[6], (uint32_t)z[7], o[1][0], o[1][1], o[1][2], o[1][3]);
    bt4((uint32_t)(z[4] >> 32), (uint32_t)(z[5] >> 32), (uint32_t)(z[6] >> 32), (uint32_t)(z[7] >> 32), o[1][4],
        o[1][5], o[1][6], o[1][7]);
#pragma unroll
    for (int a = 0; a < 8; a++) pl[a] = (long)(((uint64_t)o[1][a] << 32) | o[0][a]);
}

// Operand register tuples.  A 16x16x64 product of {X_a | X_a'} and {Y_b | Y_b'} adds the digit
// pairs (a, b) and (a', b') (the two halves of each operand take the same K positions, so the
// product is the sum of the two 32-deep ones); both pairs must lie on one diagonal s.  Two
// pairings do that with 36 instructions per tile and chunk instead of 64:
//  - windows on the left, tuples on the right: {A_a | A_a-1} x {H_2p | H_2p+1} adds (a, 2p) and
//    (a-1, 2p+1), s = a + 2p; the 7 windows are built once per left operand and the 4 tuples of
//    each tile are four 16-byte reads when its planes are stored pairwise (h_slot);
//  - tuples on the left, windows on the right: {A_2i | A_2i+1} x {H_b | H_b-1} adds (2i, b) and
//    (2i+1, b-1); the per-tile windows are transient, which suits a 128-VGPR budget in which
//    the left windows would stay live across the tiles and spill.
// The mf_left / mf_right / mf_mac_tile overloads pick the pairing from the array sizes.
constexpr int MF_NW = 7, MF_NT = 4;
__device__ __forceinline__ void mf_left(const long (&pl)[8], mf_v4i (&AW)[MF_NW]) {  // windows {w+1 | w}
#pragma unroll
    for (int w = 0; w < MF_NW; w++) AW[w] = __builtin_bit_cast(mf_v4i, mf_v2l{pl[w + 1], pl[w]});
}
__device__ __forceinline__ void mf_left(const long (&pl)[8], mf_v4i (&AT)[MF_NT]) {  // tuples {2i | 2i+1}
#pragma unroll
    for (int i = 0; i < MF_NT; i++) AT[i] = __builtin_bit_cast(mf_v4i, mf_v2l{pl[2 * i], pl[2 * i + 1]});
}
__device__ __forceinline__ void mf_right(const long (&pl)[8], mf_v4i (&HT)[MF_NT]) {  // tuples {2p | 2p+1}
#pragma unroll
    for (int p = 0; p < MF_NT; p++) HT[p] = __builtin_bit_cast(mf_v4i, mf_v2l{pl[2 * p], pl[2 * p + 1]});
}
__device__ __forceinline__ void mf_right(const long (&pl)[8], mf_v4i (&HW)[MF_NW]) {  // windows {7-j | 6-j}
#pragma unroll
    for (int j = 0; j < MF_NW; j++) HW[j] = __builtin_bit_cast(mf_v4i, mf_v2l{pl[7 - j], pl[6 - j]});
}

// ac[s] += S_s of one 16 x 16 tile over one 32-row chunk, left windows x right tuples: 28
// paired products (a = 1..7, p = 0..3) and the pairs left over, (0, 2p) and (7, 2p+1), one
// 16x16x32 each.
__device__ __forceinline__ void mf_mac_tile(mf_v4i (&ac)[15], const mf_v4i (&AW)[MF_NW], const mf_v4i (&HT)[MF_NT]) {
#pragma unroll
    for (int a = 1; a < 8; a++)
#pragma unroll
        for (int p = 0; p < MF_NT; p++)
            ac[a + 2 * p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(AW[a - 1], HT[p], ac[a + 2 * p], 0, 0, 0);
    const long a0 = __builtin_bit_cast(mf_v2l, AW[0])[1], a7 = __builtin_bit_cast(mf_v2l, AW[MF_NW - 1])[0];
#pragma unroll
    for (int p = 0; p < MF_NT; p++) {
        const mf_v2l h = __builtin_bit_cast(mf_v2l, HT[p]);
        ac[2 * p] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a0, h[0], ac[2 * p], 0, 0, 0);
        ac[8 + 2 * p] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a7, h[1], ac[8 + 2 * p], 0, 0, 0);
    }
}
// Left tuples x right windows: AT[i] x HW[7 - b] adds (2i, b) and (2i+1, b-1) for b = 1..7 (28
// products); the planes left over (a = s for even s <= 6, b = 7 for even s >= 8) take one
// 16x16x32 each.
__device__ __forceinline__ void mf_mac_tile(mf_v4i (&ac)[15], const mf_v4i (&AT)[MF_NT], const mf_v4i (&HW)[MF_NW]) {
    auto plane_a = [&](int a) -> long { return __builtin_bit_cast(mf_v2l, AT[a / 2])[a % 2]; };
    auto hsing = [&](int bb) -> long {  // plane b inside HW: HW[7 - b] = {H_b, H_b-1}, HW[6] = {H_1, H_0}
        return bb > 0 ? __builtin_bit_cast(mf_v2l, HW[7 - bb])[0] : __builtin_bit_cast(mf_v2l, HW[6])[1];
    };
#pragma unroll
    for (int i = 0; i < MF_NT; i++)
#pragma unroll
        for (int sd = 0; sd < 15; sd++) {
            const int bb = sd - 2 * i;  // pair (2i, b), (2i+1, b-1)
            if (bb < 1 || bb > 7) continue;
            ac[sd] = __builtin_amdgcn_mfma_i32_16x16x64_i8(AT[i], HW[7 - bb], ac[sd], 0, 0, 0);
        }
#pragma unroll
    for (int sd = 0; sd < 15; sd += 2) {  // leftovers: a = s (b = 0) for s <= 6, a = s - 7 (b = 7) for s >= 8
        const int aa = sd <= 6 ? sd : sd - 7, bb = sd - aa;
        ac[sd] = __builtin_amdgcn_mfma_i32_16x16x32_i8(plane_a(aa), hsing(bb), ac[sd], 0, 0, 0);
    }
}


// Reduction constants of one modulus t (host::recomb_row): 256^(8+d) mod t split in
// 30-bit halves, 2^60 mod t with its Shoup quotient, t, and 8t - [2^91]_t.
struct MfRecomb {
    int32_t clo[7], chi[7];
    uint64_t r60, r60p, tq, kfix;
};
template <class Load>
__device__ __forceinline__ MfRecomb mf_recomb_consts(Load &&rc) {
    MfRecomb k;
#pragma unroll
    for (int d = 0; d < 7; d++) {
        const uint64_t c = rc(d);
        k.clo[d] = (int32_t)(uint32_t)c;
        k.chi[d] = (int32_t)(uint32_t)(c >> 32);
        // hides that the high halves are below 2^30: a product of a known non-negative value
        // with a signed sum is otherwise taken as a full 64 x 64-bit product (five instructions)
        // instead of one signed 32 x 32 + 64-bit multiply-add
        asm volatile("" : "+v"(k.chi[d]));
    }
    k.r60 = rc(7);
    k.r60p = rc(8);
    k.tq = rc(9);
    k.kfix = rc(10);
    return k;
}

// The powers of two of the recombination, kept in registers (w2 from mf_w2) so that each term
// is one 32 x 32 + 64-bit multiply-add.
struct MfW2 {
    int32_t w[7];
};
__device__ __forceinline__ MfW2 mf_w2() {
    MfW2 w{{1 << 8, 1 << 16, 1 << 24, 1 << 2, 1 << 10, 1 << 18, 1 << 26}};
#pragma unroll
    for (int d = 0; d < 7; d++) asm volatile("" : "+v"(w.w[d]));
    return w;
}

// sum_s 256^s acc[s][v] mod t, in [0, t), for |acc[s][v]| <= 2^28.
__device__ __forceinline__ uint64_t mf_recombine(const mf_v4i (&acc)[15], int v, const MfW2 &w2, const MfRecomb &k) {
    // value = lo + 2^30 hi: lo takes the weights 1 .. 2^24 and the low 30 bits
    // of 256^s mod t (s >= 8), hi the weights 2^2 .. 2^26 and the high 30 bits;
    // |S_s| <= 2^28 keeps both below 2^61 in magnitude
    int64_t lo_s = (int64_t)acc[0][v];
    lo_s += (int64_t)acc[1][v] * (int64_t)w2.w[0];
    lo_s += (int64_t)acc[2][v] * (int64_t)w2.w[1];
    lo_s += (int64_t)acc[3][v] * (int64_t)w2.w[2];
    int64_t hi_s = (int64_t)acc[4][v] * (int64_t)w2.w[3];
    hi_s += (int64_t)acc[5][v] * (int64_t)w2.w[4];
    hi_s += (int64_t)acc[6][v] * (int64_t)w2.w[5];
    hi_s += (int64_t)acc[7][v] * (int64_t)w2.w[6];
#pragma unroll
    for (int d = 0; d < 7; d++) {
        lo_s += (int64_t)acc[8 + d][v] * (int64_t)k.clo[d];
        hi_s += (int64_t)acc[8 + d][v] * (int64_t)k.chi[d];
    }
    // hi = 2^30 h1 + h0 (0 <= h0 < 2^30, |h1| < 2^31); 2^60 h1 = 2^60 (h1 + 2^31)
    // - 2^91, and kfix = 8t - [2^91]_t makes the sum positive:
    // 0 < x = lo + 2^30 h0 + [2^60 (h1 + 2^31)]_lazy + kfix < 2^63
    const uint64_t h0 = (uint64_t)hi_s & M30;
    const uint32_t h1b = (uint32_t)(hi_s >> 30) ^ 0x80000000u;
    const uint64_t x = (uint64_t)lo_s + (h0 << 30) + shoup_lazy(h1b, k.r60, k.r60p, k.tq) + k.kfix;
    // t in (2^59, 2^59 + 2^52) and x < 2^63: x >> 59 is floor(x / t) or one more
    const uint64_t qh = x >> 59;
    int64_t r = (int64_t)(x - qh * k.tq);
    r += (r >> 63) & (int64_t)k.tq;
    return (uint64_t)r;
}

// mf_recombine for contractions of at most 32 rows (one chunk): then |S_s| <= n_s 32 2^14, with
// n_s = min(s, 14 - s) + 1 digit pairs on diagonal s, so neighbouring diagonals merge exactly
// into int32 sums
//   P_j = S_2j + 256 S_2j+1 (|P_j| < 2^30 + 2^22),  value = sum_j 2^16j P_j + 2^112 S_14,
// which halves the 64-bit multiply-adds.
__device__ __forceinline__ uint64_t mf_recombine32(const mf_v4i (&acc)[15], int v, const MfW2 &w2, const MfRecomb &k) {
    int32_t p[7];
#pragma unroll
    for (int j = 0; j < 7; j++) p[j] = acc[2 * j][v] + acc[2 * j + 1][v] * 256;
    // lo: weights 1, 2^16 and the low 30 bits of 2^16j mod t (j = 4, 5, 6, and 2^112 for S_14);
    // hi: weights 2^2, 2^18 (2^32 = 2^30 2^2, 2^48 = 2^30 2^18) and the high bits (below 2^29.01,
    // as t < 2^59.01).  With |P_4|, |P_5|, |P_6| below 0.76, 0.51, 0.26 2^30: |lo| < 1.52 2^60
    // and |hi| < 0.77 2^60, so h1 below fits the 2^31 offset of mf_recombine
    int64_t lo = (int64_t)p[0] + (int64_t)p[1] * (int64_t)w2.w[1];
    int64_t hi = (int64_t)p[2] * (int64_t)w2.w[3] + (int64_t)p[3] * (int64_t)w2.w[5];
#pragma unroll
    for (int j = 4; j < 7; j++) {
        lo += (int64_t)p[j] * (int64_t)k.clo[2 * (j - 4)];
        hi += (int64_t)p[j] * (int64_t)k.chi[2 * (j - 4)];
    }
    lo += (int64_t)acc[14][v] * (int64_t)k.clo[6];
    hi += (int64_t)acc[14][v] * (int64_t)k.chi[6];
    // as in mf_recombine: 0 < x = lo + 2^30 h0 + [2^60 (h1 + 2^31)]_lazy + 8t - [2^91]_t < 8.6 2^60
    const uint64_t h0 = (uint64_t)hi & M30;
    const uint32_t h1b = (uint32_t)(hi >> 30) ^ 0x80000000u;
    const uint64_t x = (uint64_t)lo + (h0 << 30) + shoup_lazy(h1b, k.r60, k.r60p, k.tq) + k.kfix;
    // t in (2^59, 2^59 + 2^52) and x < 2^64: x / 2^59 exceeds x / t by less than 1/4, so
    // x >> 59 is floor(x / t) or one more
    const uint64_t qh = x >> 59;
    int64_t r = (int64_t)(x - qh * k.tq);
    r += (r >> 63) & (int64_t)k.tq;
    return (uint64_t)r;
}

}  // namespace ckks
