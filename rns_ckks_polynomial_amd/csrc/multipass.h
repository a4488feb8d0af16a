// multipass.h -- NTT for ring degrees whose limb does not fit one workgroup's
// LDS (n = 65536: 512 KiB per limb).  Four-step split n = n1 * n2: a first
// pass of n2 column transforms of length n1 (strided), a twiddle by the
// inner roots, then n1 row transforms of length n2; the last pass writes the
// result in natural order.
#pragma once
#include "ctx_internal.h"

namespace ckks {

struct MultipassPlan {
    uint32_t n1 = 0, n2 = 0, log1 = 0, log2 = 0;
    // Per prime: column-stage twiddles (length-n1 merged-psi table of the
    // 2*n1-th root psi^(n2)), the cross twiddles psi^((2 j1 + 1) i2) ... see multipass.hip
    uint64_t *d_tw1f = nullptr, *d_tw1i = nullptr;  // [ntot][n1][2]
    uint64_t *d_tw2f = nullptr, *d_tw2i = nullptr;  // [ntot][n2][2]
    uint64_t *d_twxf = nullptr, *d_twxi = nullptr;  // [ntot][n][2] cross twiddles
    std::vector<void *> owned;
};

int multipass_init(ckks_ctx *ctx);
void multipass_free(ckks_ctx *ctx);

}  // namespace ckks
