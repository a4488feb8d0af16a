// ntt2048.h -- one n = 2048 negacyclic NTT per 256-thread workgroup, limb in LDS.
//
// Transform (natural order in and out): A_j = sum_i a_i psi^(i(2j+1)) mod q,
// the "NTT/INTT" polynomial-multiply accelerator of the Kestrel article's
// technique table; the EncryptedLLM GPU blog (section 3.4) keeps one
// polynomial's butterfly region in shared memory per block.
//
// Schedule (gfx950, wave64): each of the 256 threads owns 8 coefficients whose
// indices differ in 3 consecutive bits, so three radix-2 stages run in
// registers between LDS exchanges:
//   forward  (merged-psi Cooley-Tukey, bits high -> low): [10 9 8] [7 6 5] [4 3 2] [1 0]
//   inverse  (merged-psi Gentleman-Sande, bits low -> high): [0 1 2] [3 4 5] [6 7 8] [9 10]
// The merged-psi forward leaves the result in bit-reversed order; the final
// LDS exchange writes it back in natural order (and the inverse reads its
// input through the same permutation), so no separate reorder pass exists.
// Twiddles are Shoup pairs (w, floor(w 2^64/q)) of psi^bitrev(k) (forward) and
// psi^-bitrev(k) (inverse), interleaved [k][2].  Butterflies are Harvey's lazy
// forms with a truncated Shoup quotient (see shoup_lazy4): the twiddle product
// lands in [0, 4q), so values stay in [0, 8q) (forward) or [0, 4q) (inverse),
// all below 2^63 for q < 2^60.
#pragma once
#include "ckks_common.h"

namespace ckks {
namespace n2048 {

constexpr int LOGN = 11;
constexpr int N = 1 << LOGN;
constexpr int NT = 256;  // threads per workgroup
constexpr int E = 8;     // coefficients per thread
constexpr int LDS_WORDS = N + N / 32;

// LDS slot of coefficient index i (one pad word per 32 breaks power-of-two strides).
__device__ __forceinline__ int slot(int i) { return i + (i >> 5); }

// Index of the k-th coefficient owned by thread t in a pass that owns bits [C, C+3).
template <int C>
__device__ __forceinline__ int own(int t, int k) {
    return (t & ((1 << C) - 1)) | (k << C) | ((t >> C) << (C + 3));
}

__device__ __forceinline__ int brev(int i) { return (int)(__builtin_bitreverse32((uint32_t)i) >> (32 - LOGN)); }

// Per-prime constants of the butterflies.  -4q passes through an empty asm so
// that x - 4q stays one 64-bit add (v_lshl_add_u64) instead of being turned
// back into a subtract with borrow.
struct BfConsts {
    uint64_t q, q4, nq4;
};
__device__ __forceinline__ BfConsts bf_consts(uint64_t q) {
    BfConsts c{q, 4 * q, 0 - 4 * q};
    asm volatile("" : "+v"(c.nq4));
    return c;
}

__device__ __forceinline__ void bf_ct(uint64_t &x, uint64_t &y, uint64_t w, uint64_t wp, const BfConsts &c) {
    const uint64_t a = csub_sign(x, c.nq4);           // [0, 4q)
    const uint64_t t = shoup_lazy4(y, w, wp, 0 - c.q); // [0, 4q)
    x = a + t;                                        // [0, 8q)
    y = a + c.q4 - t;                                 // (0, 8q)
}

__device__ __forceinline__ void bf_gs(uint64_t &x, uint64_t &y, uint64_t w, uint64_t wp, const BfConsts &c) {
    const uint64_t s = x + y;                         // [0, 8q)
    const uint64_t d = x + c.q4 - y;                  // (0, 8q)
    x = csub_sign(s, c.nq4);                          // [0, 4q)
    y = shoup_lazy4(d, w, wp, 0 - c.q);               // [0, 4q)
}

// [0, 8q) -> [0, q): the forward transform's outputs fully reduced.
__device__ __forceinline__ uint64_t reduce8(uint64_t x, uint64_t q) {
    x = x >= 4 * q ? x - 4 * q : x;
    x = x >= 2 * q ? x - 2 * q : x;
    return x >= q ? x - q : x;
}

// One radix-2 stage (bit BIT of the index) on the 8 registers of a pass owning bits [C, C+3).
template <int C, int BIT, bool INV>
__device__ __forceinline__ void stage(uint64_t (&v)[E], int t, const uint64_t *__restrict__ tw, const BfConsts &q) {
    constexpr int s = LOGN - 1 - BIT;  // stage number in the Cooley-Tukey order
    constexpr int kb = 1 << (BIT - C);
#pragma unroll
    for (int k = 0; k < E; k++) {
        if (k & kb) continue;
        const int j = own<C>(t, k);
        const int ti = (1 << s) + (j >> (LOGN - s));
        const uint64_t w = tw[2 * ti], wp = tw[2 * ti + 1];
        if (INV) bf_gs(v[k], v[k | kb], w, wp, q);
        else bf_ct(v[k], v[k | kb], w, wp, q);
    }
}

template <int C>
__device__ __forceinline__ void to_lds(uint64_t *lds, const uint64_t (&v)[E], int t) {
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(own<C>(t, k))] = v[k];
}
template <int C>
__device__ __forceinline__ void from_lds(const uint64_t *lds, uint64_t (&v)[E], int t) {
#pragma unroll
    for (int k = 0; k < E; k++) v[k] = lds[slot(own<C>(t, k))];
}

// Forward NTT.  On entry v[k] = a[t + 256 k] (natural order, values < 8q);
// on exit v[k] = A[t + 256 k] in [0, 8q) (reduce8 finishes).  Uses lds[LDS_WORDS]; ends with a barrier.
__device__ __forceinline__ void fwd(uint64_t (&v)[E], uint64_t *lds, const uint64_t *__restrict__ tw, uint64_t qv) {
    const int t = threadIdx.x;
    const BfConsts q = bf_consts(qv);
    stage<8, 10, false>(v, t, tw, q);
    stage<8, 9, false>(v, t, tw, q);
    stage<8, 8, false>(v, t, tw, q);
    to_lds<8>(lds, v, t);
    __syncthreads();
    from_lds<5>(lds, v, t);
    stage<5, 7, false>(v, t, tw, q);
    stage<5, 6, false>(v, t, tw, q);
    stage<5, 5, false>(v, t, tw, q);
    __syncthreads();
    to_lds<5>(lds, v, t);
    __syncthreads();
    from_lds<2>(lds, v, t);
    stage<2, 4, false>(v, t, tw, q);
    stage<2, 3, false>(v, t, tw, q);
    stage<2, 2, false>(v, t, tw, q);
    __syncthreads();
    to_lds<2>(lds, v, t);
    __syncthreads();
    from_lds<0>(lds, v, t);
    stage<0, 1, false>(v, t, tw, q);
    stage<0, 0, false>(v, t, tw, q);
    __syncthreads();
    // coefficient own<0>(t,k) = 8t + k now holds A_{brev(8t+k)}: write back in natural order
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(brev(8 * t + k))] = v[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < E; k++) v[k] = lds[slot(t + NT * k)];
    __syncthreads();
}

// Inverse NTT without the final n^-1 scaling.  On entry v[k] = A[t + 256 k]
// (values < 4q); on exit v[k] = n a[t + 256 k] in [0, 4q).
__device__ __forceinline__ void inv(uint64_t (&v)[E], uint64_t *lds, const uint64_t *__restrict__ tw, uint64_t qv) {
    const int t = threadIdx.x;
    const BfConsts q = bf_consts(qv);
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(brev(t + NT * k))] = v[k];
    __syncthreads();
    from_lds<0>(lds, v, t);
    stage<0, 0, true>(v, t, tw, q);
    stage<0, 1, true>(v, t, tw, q);
    stage<0, 2, true>(v, t, tw, q);
    __syncthreads();
    to_lds<0>(lds, v, t);
    __syncthreads();
    from_lds<3>(lds, v, t);
    stage<3, 3, true>(v, t, tw, q);
    stage<3, 4, true>(v, t, tw, q);
    stage<3, 5, true>(v, t, tw, q);
    __syncthreads();
    to_lds<3>(lds, v, t);
    __syncthreads();
    from_lds<6>(lds, v, t);
    stage<6, 6, true>(v, t, tw, q);
    stage<6, 7, true>(v, t, tw, q);
    stage<6, 8, true>(v, t, tw, q);
    __syncthreads();
    to_lds<6>(lds, v, t);
    __syncthreads();
    from_lds<8>(lds, v, t);
    stage<8, 9, true>(v, t, tw, q);
    stage<8, 10, true>(v, t, tw, q);
    __syncthreads();
}

}  // namespace n2048
}  // namespace ckks
