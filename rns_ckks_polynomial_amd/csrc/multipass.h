// multipass.h -- NTT for ring degrees whose limb does not fit one workgroup's
// LDS (n = 65536: 512 KiB per limb).
//
// Four-step split n = n1 n2 (256 x 256), index i = n2 i1 + i2, j = j1 + n1 j2:
//   A_{j1 + n1 j2} = sum_{i2} psi2^{i2 (2 j2 + 1)} [ T[j1][i2] sum_{i1} a_{n2 i1 + i2} psi1^{i1 (2 j1 + 1)} ]
// with psi1 = psi^n2, psi2 = psi^n1 (primitive 2*256-th roots) and the cross
// twiddle T[j1][i2] = psi^{i2 (2 j1 + 1 - n1)}: a column pass of length-256
// negacyclic NTTs, the twiddle, then a row pass of length-256 negacyclic NTTs
// whose outputs land transposed in natural order.  The inverse runs the
// mirror image.  One pass is out of place, through a transpose buffer: the
// caller's (from an operation's workspace, MP_CHUNK limbs), or for the bare
// NTT calls the context's, whose users are ordered across streams by an event.
#pragma once
#include "ctx_internal.h"

namespace ckks {

constexpr uint32_t MP_N1 = 256, MP_LOG1 = 8;
constexpr uint32_t MP_CHUNK = 64;  // limbs per transpose pass (64 x 512 KiB = 32 MiB)

struct MultipassPlan {
    uint64_t *d_tw256f = nullptr, *d_tw256i = nullptr;  // [ntot][256][2]  (psi^256)^(+-bitrev8(k)), Shoup
    uint64_t *d_cross = nullptr;                         // [ntot][256 j1][256 i2][2]  T, Shoup
    uint64_t *d_crossinvT = nullptr;                     // [ntot][256 i2][256 j1][2]  T^-1 transposed, Shoup
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
