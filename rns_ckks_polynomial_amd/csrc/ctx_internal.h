// ctx_internal.h -- the library context: per-prime tables plus the tables of
// every prepared level, all resident in HBM; read-only once prepared.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ckks_gpu.h"
#include "ckks_common.h"

namespace ckks {

// Tables that depend on the level l (the last key-switching digit may be partial).
struct LevelTables {
    uint32_t l = 0, beta = 0;
    BasisDev *d_digits = nullptr;   // [beta] device copies of the digit bases at level l
    std::vector<BasisDev> h_digits; // host copies (pointers are device pointers)
    uint64_t *d_modup_scale = nullptr;  // [l][2] Shoup pair of n^-1 [Bhat_i^-1]_{q_i} (digit of i)
    uint64_t *d_rescale_inv = nullptr;  // [l-1][2] Shoup pair of q_{l-1}^-1 mod q_i
    std::vector<void *> owned;          // device allocations owned by this level
};

// ModRaise tables for a source level l0: the basis of primes [0, l0) with
// every chain prime as a target, and n^-1 [Bhat_i^-1]_{q_i} (Shoup pairs).
struct RaiseTables {
    BasisDev *d_basis = nullptr;
    uint64_t *d_scale = nullptr;  // [l0][2]
    std::vector<void *> owned;
};

struct MultipassPlan;  // large-n NTT tables (n > 2048)

// Optional per-launch timing with HIP events (enabled by ckks_profile_begin).
struct Profiler {
    bool on = false;
    std::vector<std::string> names;
    struct Rec {
        int name;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
    size_t used = 0;
    std::mutex mu;
    hipEvent_t take();
    int name_id(const char *n);
};

}  // namespace ckks

struct ckks_ctx {
    uint32_t n = 0, L = 0, K = 0, dnum = 0, alpha = 0, logn = 0;
    int device = 0;
    std::vector<uint64_t> primes, psi;  // [L+K]
    ckks::PrimeConsts *d_pc = nullptr;  // [L+K]
    uint64_t *d_tw_fwd = nullptr;       // [L+K][n][2]  psi^bitrev(k), Shoup
    uint64_t *d_tw_inv = nullptr;       // [L+K][n][2]  psi^-bitrev(k), Shoup
    uint64_t *d_iota = nullptr;         // [L+K]        psi^(n/2), the NTT of X^(n/2) is iota (-1)^k
    uint64_t *d_prc = nullptr;          // [L+K][MF_RC] matrix-core reduction constants of each prime
    // base of the special primes P (targets: every chain prime)
    ckks::BasisDev h_pbasis{};
    ckks::BasisDev *d_pbasis = nullptr;
    uint64_t *d_moddown_scale = nullptr;  // [K][2] Shoup pair of n^-1 [Phat_k^-1]_{p_k}
    uint64_t *d_pinv = nullptr;           // [L][2] Shoup pair of P^-1 mod q_i
    uint64_t *d_pmod = nullptr;           // [L]    P mod q_i
    // full-width digits at the top level (reused by every level where the digit is whole)
    std::vector<ckks::BasisDev> full_digits;
    std::vector<std::vector<uint64_t>> full_inv_hat;  // host Shoup pairs of each full digit's [Bhat_i^-1]
    std::vector<void *> owned;
    std::map<uint32_t, ckks::LevelTables *> levels;  // prepared levels
    std::map<uint32_t, ckks::RaiseTables *> raise;   // ModRaise tables by prepared source level
    ckks::MultipassPlan *mp = nullptr;
    ckks::Profiler *prof = nullptr;
};

namespace ckks {
// Records HIP events around the launches made in its scope when profiling is on.
struct ProfScope {
    const ckks_ctx *c;
    hipStream_t s;
    int name = -1;
    hipEvent_t b{};
    ProfScope(const ckks_ctx *ctx, const char *nm, hipStream_t st) : c(ctx), s(st) {
        if (c->prof && c->prof->on) {
            std::lock_guard<std::mutex> g(c->prof->mu);
            name = c->prof->name_id(nm);
            hipEvent_t a = c->prof->take();
            b = c->prof->take();
            (void)hipEventRecord(a, s);
            c->prof->recs.push_back({name, a, b});
        }
    }
    ~ProfScope() {
        if (name >= 0) (void)hipEventRecord(b, s);
    }
};
}  // namespace ckks

namespace ckks {
// host-side number theory (independent of any reference code)
uint64_t h_mulmod(uint64_t a, uint64_t b, uint64_t q);
uint64_t h_powmod(uint64_t a, uint64_t e, uint64_t q);
uint64_t h_invmod(uint64_t a, uint64_t q);
uint64_t h_shoup(uint64_t w, uint64_t q);

// Build (blocking, allocating) the tables of level l / of ModRaise source level l0;
// a level already built is kept.
int prepare_level(ckks_ctx *ctx, uint32_t l);
int prepare_raise(ckks_ctx *ctx, uint32_t l0);
// The prepared tables, or nullptr when the level was not prepared (lookups only).
const LevelTables *find_level(const ckks_ctx *ctx, uint32_t l);
const RaiseTables *find_raise(const ckks_ctx *ctx, uint32_t l0);
// Build a basis table for primes [first, first + m) with every chain prime as target.
// chain_targets: lay the conversion table over the chain primes [0, L) (as for
// the special primes) instead of specials-first-then-outside-the-digit.
// inv_hat_host (optional) receives the Shoup pairs of [Bhat_i^-1]_{b_i}.
int build_basis(ckks_ctx *ctx, uint32_t first, uint32_t m, BasisDev *out, std::vector<void *> &owned,
                bool chain_targets = false, std::vector<uint64_t> *inv_hat_host = nullptr);
}  // namespace ckks
