// butterfly.h -- radix-2 NTT butterflies shared by the one-workgroup (n = 2048)
// and the four-step (n = 65536) transforms.
//
// Harvey's lazy forms with a truncated Shoup quotient (shoup_lazy4): the twiddle
// product lands in [0, 4q).  Cooley-Tukey butterflies may leave their top input
// unreduced, so that outputs grow by 4q per stage until a stage reduces it;
// Gentleman-Sande butterflies keep both values below 4q.
#pragma once
#include "ckks_common.h"

namespace ckks {

// Per-prime constants of the butterflies.  The negated thresholds pass through an
// empty asm so that x - c stays one 64-bit add (v_lshl_add_u64) instead of being
// turned back into a subtract with borrow.
struct BfConsts {
    uint64_t q, q4, n4, n8, n16;
};
__device__ __forceinline__ BfConsts bf_consts(uint64_t q) {
    BfConsts c{q, 4 * q, 0 - 4 * q, 0 - 8 * q, 0 - 16 * q};
    asm volatile("" : "+v"(c.n4));
    asm volatile("" : "+v"(c.n8));
    asm volatile("" : "+v"(c.n16));
    return c;
}

// x - c if x >= c else x (nc = 2^64 - c): one add, one unsigned compare, a select.
__device__ __forceinline__ uint64_t csub_n(uint64_t x, uint64_t c, uint64_t nc) {
    const uint64_t m = x + nc;
    return x >= c ? m : x;
}

// Cooley-Tukey butterfly (x, y) -> (a + t, a + 4q - t), a = x reduced by RED (0: as is,
// else x - RED q when x >= RED q), t = y w in [0, 4q).  Without a reduction the bound of
// the outputs grows by 4q per stage, so the forward transform reduces only where its
// bounds require (see fwd).
template <int RED>
__device__ __forceinline__ void bf_ct(uint64_t &x, uint64_t &y, uint64_t w, uint64_t wp, const BfConsts &c) {
    uint64_t a = x;
    if (RED == 4) a = csub_n(x, c.q4, c.n4);
    if (RED == 8) a = csub_n(x, 2 * c.q4, c.n8);
    if (RED == 16) a = csub_n(x, 4 * c.q4, c.n16);
    const uint64_t t = shoup_lazy4(y, w, wp, 0 - c.q);  // [0, 4q)
    x = a + t;
    y = a + c.q4 - t;
}

__device__ __forceinline__ void bf_gs(uint64_t &x, uint64_t &y, uint64_t w, uint64_t wp, const BfConsts &c) {
    const uint64_t s = x + y;                         // [0, 8q)
    const uint64_t d = x + c.q4 - y;                  // (0, 8q)
    x = csub_n(s, c.q4, c.n4);                        // [0, 4q)
    y = shoup_lazy4(d, w, wp, 0 - c.q);               // [0, 4q)
}

// The forward transform's outputs ([0, 24q)) fully reduced.
__device__ __forceinline__ uint64_t reduce_out(uint64_t x, uint64_t q) { return reduce59(x, q, 0 - q); }

}  // namespace ckks
