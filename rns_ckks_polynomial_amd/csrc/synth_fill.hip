// synth_fill.hip -- device-side SplitMix64 fill of synthetic inputs (see
// include/ckks_synth.h for the definition; no RNS-CKKS arithmetic here).
#include "../../include/ckks_synth.h"
#include "ctx_internal.h"
#include "ops.h"

namespace ckks {


__global__ void k_fill_uniform(uint64_t *__restrict__ dst, const PrimeConsts *__restrict__ pc, uint32_t n,
                               uint32_t nl, uint32_t first, uint64_t key, uint64_t stream0, size_t total) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
        const size_t limb = e / n;
        const uint64_t i = e % n;
        const uint64_t q = pc[first + limb % nl].q;
        const uint64_t st = sm_at(key, stream0 + limb);
        const uint64_t w = sm_at(st, i);
        uint64_t v = 0;
        bool ok = false;
        for (uint64_t r = 0; r < 64 && !ok; r++) {
            v = sm_at(w, r) & ((1ull << 60) - 1);
            ok = v < q;
        }
        dst[e] = ok ? v : v % q;
    }
}

int op_fill_uniform(const ckks_ctx *c, uint64_t *dst, int count, int first, int nlimbs, uint64_t seed, uint64_t tag,
                    uint64_t stream0, hipStream_t s) {
    const uint64_t key = sm_at(seed, tag);
    const size_t total = (size_t)count * nlimbs * c->n;
    if (!total) return CKKS_OK;
    size_t blocks = std::min<size_t>((total + 255) / 256, 1u << 20);
    hipLaunchKernelGGL(k_fill_uniform, dim3((unsigned)blocks), dim3(256), 0, s, dst, c->d_pc, c->n, (uint32_t)nlimbs,
                       (uint32_t)first, key, stream0, total);
    return hipGetLastError() == hipSuccess ? CKKS_OK : CKKS_EHIP;
}

}  // namespace ckks
