// host_tables.h -- host-side number theory and constant tables of the
// library (plain C++17: built into the library, and on its own with the
// host sanitizers by the test-suite).
//
// Everything here runs once per context or prepared level; the device
// headers take the table layouts from here.
#pragma once
#include <stdint.h>

#include <vector>

namespace ckks {

// Per-prime reduction constants (device arrays indexed by global prime index).
struct PrimeConsts {
    uint64_t q;      // the prime
    uint64_t mu;     // floor(2^122 / q)
    uint64_t r64;    // 2^64 mod q
    uint64_t r64p;   // Shoup companion of r64
    uint64_t m64;    // floor(2^64 / q)  (Shoup companion of 1)
    uint64_t ninv;   // n^-1 mod q
    uint64_t ninvp;  // Shoup companion of ninv
    uint64_t r60;    // 2^60 mod q
    uint64_t r60p;   // Shoup companion of r60
};

// Reduction constants of a modulus t for the matrix-core products (the base
// conversion's targets, the multiply-accumulate's chain primes): [0..6] 256^s
// mod t for s = 8..14 (low 30 bits | high 30 bits << 32), [7] 2^60 mod t, [8]
// its Shoup quotient, [9] t, [10] 8t - [2^91]_t.
constexpr uint32_t MF_RC = 11;

namespace host {

uint64_t mulmod(uint64_t a, uint64_t b, uint64_t q);
uint64_t powmod(uint64_t a, uint64_t e, uint64_t q);
uint64_t invmod(uint64_t a, uint64_t q);  // a invertible modulo q
uint64_t shoup(uint64_t w, uint64_t q);    // floor(w 2^64 / q), w < q
bool is_prime(uint64_t x);
// The `count` smallest primes in (2^59, 2^60) that are 1 mod 2n, ascending.
bool chain(uint32_t n, uint32_t count, std::vector<uint64_t> &out);
// The smallest primitive 2n-th root of unity modulo q.
uint64_t min_root(uint32_t n, uint64_t q);
uint32_t bitrev(uint32_t x, uint32_t bits);
// The MF_RC reduction constants of modulus q (row[0 .. MF_RC)).
void recomb_row(uint64_t q, uint64_t *row);
// Signed base-256 digits of v < 2^63: byte a of the result, read as an int8,
// is d_a with v = sum_a d_a 256^a, -128 <= d_a <= 127.
inline uint64_t digit_form(uint64_t v) { return (v + 0x8080808080808080ull) ^ 0x8080808080808080ull; }

// One prime's constants and twiddles: tw_fwd / tw_inv [n][2] hold the Shoup
// pairs of psi^bitrev(k) and psi^-bitrev(k); iota = psi^(n/2).
void prime_tables(uint32_t n, uint64_t q, uint64_t psi, PrimeConsts &pc, uint64_t *tw_fwd, uint64_t *tw_inv,
                  uint64_t &iota);

// Entry order of the n = 2048 tables read by the one-workgroup transform.  In the
// register pass next to the natural-order side (forward stages s = 9, 10; inverse
// stages s = 8, 9, 10) thread t runs the bit-reversed indices 8 brev8(t) + k, so the
// heap entry 2^s + c brev8(t) + h (c = 2^(s-8), h < c) is stored at 2^s + c t + h: each
// thread's twiddles stay a contiguous run.  The other stages keep the heap order.
void ntt2048_twiddle_order(uint64_t *tw_fwd, uint64_t *tw_inv);

// Exact base conversion from the primes [first, first + m) of the chain
// (L main primes, then K special primes) to other chain primes.
struct BasisTables {
    uint32_t m = 0, first = 0, mk = 0, npos = 0;
    std::vector<uint64_t> inv_hat;  // [m][2] Shoup pair of [Bhat_i^-1]_{b_i}
    std::vector<uint64_t> hat_mod;  // [m][2] Shoup pair of [Bhat_i]_{b_i}
    std::vector<uint64_t> R;        // [m] floor(2^123 / b_i)
    std::vector<uint64_t> garner;   // [m][m][2] Shoup pair of b_k^-1 mod b_i (k < i)
    std::vector<uint64_t> half;     // [m] mixed-radix digits of (B - 1) / 2
    std::vector<uint32_t> pos;      // target position -> chain prime index
    std::vector<int8_t> HD;         // [npad][8][mk] signed base-256 digits of the conversion rows
    std::vector<uint64_t> RC;       // [npad][MF_RC]
};
// chain_targets: targets are the main primes [0, L) in order (the special
// basis, ModRaise); otherwise the special primes, then the main primes
// outside the basis.
void basis_tables(const std::vector<uint64_t> &primes, uint32_t L, uint32_t K, uint32_t first, uint32_t m,
                  bool chain_targets, BasisTables &out);

}  // namespace host
}  // namespace ckks
