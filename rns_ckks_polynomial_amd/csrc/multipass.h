// multipass.h -- NTT for ring degrees whose limb does not fit one workgroup's
// LDS (n = 65536: 512 KiB per limb).
//
// Four-step split n = n1 n2 (256 x 256), index i = n2 i1 + i2, j = j1 + n1 j2:
//   A_{j1 + n1 j2} = sum_{i2} psi2^{i2 (2 j2 + 1)} [ T[j1][i2] sum_{i1} a_{n2 i1 + i2} psi1^{i1 (2 j1 + 1)} ]
// with psi1 = psi^n2, psi2 = psi^n1 (primitive 2*256-th roots) and the cross
// twiddle T[j1][i2] = psi^{i2 (2 j1 + 1 - n1)}: a column pass of length-256
// negacyclic NTTs, the twiddle, then a row pass of length-256 transforms whose
// outputs land transposed in natural order.
//
// The cross twiddle is never stored whole.  With j1 = 16 k + t (t < 16) it
// factors as T = TA[i2][t] * gamma_k^{i2}, TA[i2][t] = psi^{i2 (2t + 1 - n1)},
// gamma_k = psi^{32 k}:
//  - the column pass multiplies by TA, one constant per thread (a thread holds
//    one column i2 and the rows t + 16 k);
//  - a row workgroup holds the 16 rows of one k, so gamma_k^{i2} goes into its
//    twiddles: the row pass evaluates its input at the points
//    psi^{n1 + 32 k} omega^{j2} (omega = psi^{2 n1}), a Cooley-Tukey transform whose
//    twiddle at heap index m = 2^s + b is psi^{(128 >> s)(256 + 32 k + 512 bitrev_s(b))}.
// Tables per prime: 2 x 4 KiB (column twiddles) + 2 x 64 KiB (TA and its inverse)
// + 2 x 64 KiB (row twiddles of the 16 k) instead of a 1 MiB twiddle matrix per
// direction.  The inverse runs the mirror image (row pass with the inverse row
// twiddles, then TA^-1 before the inverse column pass).  One pass is out of place,
// through a transpose buffer: the caller's (from an operation's workspace,
// MP_CHUNK limbs), or for the bare NTT calls the context's, whose users are
// ordered across streams by an event.
#pragma once
#include "ctx_internal.h"

namespace ckks {

constexpr uint32_t MP_N1 = 256, MP_LOG1 = 8;
constexpr uint32_t MP_CHUNK = 320;  // most limbs per transpose pass (320 x 512 KiB = 160 MiB)

// Limbs per pass for nblk limbs: the fewest passes of at most MP_CHUNK, evenly sized, so that
// no pass is a short tail that leaves most of the chip idle.
inline int mp_chunk(int nblk) {
    const int passes = (nblk + (int)MP_CHUNK - 1) / (int)MP_CHUNK;
    return passes > 1 ? (nblk + passes - 1) / passes : nblk;
}

struct MultipassPlan {
    uint64_t *d_tw256f = nullptr, *d_tw256i = nullptr;  // [ntot][256][2]  (psi^256)^(+-bitrev8(k)), Shoup
    uint64_t *d_taf = nullptr, *d_tai = nullptr;        // [ntot][256 i2][16 t][2]  TA, TA^-1, Shoup
    uint64_t *d_rowf = nullptr, *d_rowi = nullptr;      // [ntot][16 k][256 m][2]  row twiddles and inverses
    uint64_t *d_scratch = nullptr;                       // [MP_CHUNK][n]: the bare NTT calls' transpose buffer
    hipEvent_t scratch_done = nullptr;                   // recorded after the last use of d_scratch
    std::mutex scratch_mu;                               // orders the enqueues that use d_scratch
    std::vector<void *> owned;
};

// Words of an operation's transpose buffer (0 when the ring fits one LDS tile).
inline size_t mp_scratch_words(uint32_t n) { return n > 2048 ? (size_t)MP_CHUNK * n : 0; }

int multipass_init(ckks_ctx *ctx);
void multipass_free(ckks_ctx *ctx);

}  // namespace ckks
