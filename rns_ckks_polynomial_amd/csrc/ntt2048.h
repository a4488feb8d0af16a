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
// The merged-psi forward works in bit-reversed order.  In the register pass
// next to the natural-order side (the forward's last, the inverse's first)
// thread t takes the bit-reversed indices 8 brev8(t) + k, which sit at the
// natural positions t + 256 brev3(k): the order change is a renaming of
// registers, with no LDS exchange of its own.  The twiddles of those passes'
// stages are stored permuted to match (host::ntt2048_twiddle_order), so their
// twiddle reads stay the same contiguous runs.
// Twiddles are Shoup pairs (w, floor(w 2^64/q)) of psi^bitrev(k) (forward) and
// psi^-bitrev(k) (inverse), interleaved [k][2].  Butterflies are Harvey's lazy
// forms with a truncated Shoup quotient (see shoup_lazy4): the twiddle product
// lands in [0, 4q); the forward transform (inputs below 4q) reduces its top
// inputs at two of its eleven stages (values below 28q < 2^64), the inverse
// keeps them below 4q.
#pragma once
#include "butterfly.h"

namespace ckks {
namespace n2048 {

constexpr int LOGN = 11;
constexpr int N = 1 << LOGN;
constexpr int NT = 256;  // threads per workgroup
constexpr int E = 8;     // coefficients per thread
constexpr int LDS_WORDS = N + N / 32;

// LDS slot of coefficient index i (one pad word per 32 breaks power-of-two strides).
// slot(a | b) = slot(a) + slot(b) when a and b have no bit in common, so every
// exchange below is a per-thread base plus a compile-time offset per register
// (one address computation per exchange instead of one per access).
__device__ __forceinline__ constexpr int slot(int i) { return i + (i >> 5); }

// Index of the k-th coefficient owned by thread t in a pass that owns bits [C, C+3).
template <int C>
__device__ __forceinline__ int own(int t, int k) {
    return (t & ((1 << C) - 1)) | (k << C) | ((t >> C) << (C + 3));
}

__device__ __forceinline__ constexpr int brev8(int i) { return (int)(__builtin_bitreverse32((uint32_t)i) >> 24); }
__device__ __forceinline__ constexpr int brev3(int k) { return ((k & 1) << 2) | (k & 2) | ((k >> 2) & 1); }

// v[k] <- v[brev3(k)] (an involution): a compile-time renaming of registers.
__device__ __forceinline__ void swap_brev3(uint64_t (&v)[E]) {
    const uint64_t t1 = v[1], t3 = v[3];
    v[1] = v[4];
    v[4] = t1;
    v[3] = v[6];
    v[6] = t3;
}

// One radix-2 stage (bit BIT of the index) on the 8 registers of a pass owning bits [C, C+3).
template <int C, int BIT, bool INV, int RED = 4>
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
        else bf_ct<RED>(v[k], v[k | kb], w, wp, q);
    }
}

// own<C>(t, k) = own<C>(t, 0) | (k << C), two disjoint bit fields
template <int C>
__device__ __forceinline__ void to_lds(uint64_t *lds, const uint64_t (&v)[E], int t) {
    uint64_t *b = lds + slot(own<C>(t, 0));
#pragma unroll
    for (int k = 0; k < E; k++) b[slot(k << C)] = v[k];
}
template <int C>
__device__ __forceinline__ void from_lds(const uint64_t *lds, uint64_t (&v)[E], int t) {
    const uint64_t *b = lds + slot(own<C>(t, 0));
#pragma unroll
    for (int k = 0; k < E; k++) v[k] = b[slot(k << C)];
}

// Forward NTT.  On entry v[k] = a[t + 256 k] (natural order, values < 4q);
// on exit v[k] = A[t + 256 k] in [0, 24q) (reduce_out finishes).  Uses lds[LDS_WORDS]; ends with a barrier.
// tw: the prime's forward table in the order of host::ntt2048_twiddle_order.
// Bounds: a stage without reduction maps inputs below B q to outputs below (B + 4) q.
// From below 4q, six stages run unreduced (below 28q); the first stage of each of the
// last two register passes reduces its top input below 16q, so no value reaches 28q
// and a + 4q stays below 2^64 (28 q < 2^64 for every chain prime).
__device__ __forceinline__ void fwd(uint64_t (&v)[E], uint64_t *lds, const uint64_t *__restrict__ tw, uint64_t qv) {
    const int t = threadIdx.x;
    const BfConsts q = bf_consts(qv);
    stage<8, 10, false, 0>(v, t, tw, q);   // outputs < 8q
    stage<8, 9, false, 0>(v, t, tw, q);    //         < 12q
    stage<8, 8, false, 0>(v, t, tw, q);    //         < 16q
    to_lds<8>(lds, v, t);
    __syncthreads();
    from_lds<5>(lds, v, t);
    stage<5, 7, false, 0>(v, t, tw, q);    //          < 20q
    stage<5, 6, false, 0>(v, t, tw, q);    //          < 24q
    stage<5, 5, false, 0>(v, t, tw, q);    //          < 28q
    __syncthreads();
    to_lds<5>(lds, v, t);
    __syncthreads();
    from_lds<2>(lds, v, t);
    stage<2, 4, false, 16>(v, t, tw, q);   // a < 16q, < 20q
    stage<2, 3, false, 0>(v, t, tw, q);    //          < 24q
    stage<2, 2, false, 0>(v, t, tw, q);    //          < 28q (a + 4q < 28q)
    __syncthreads();
    to_lds<2>(lds, v, t);
    __syncthreads();
    // thread t takes the indices 8 brev8(t) + k (the stages' twiddle index uses t: the
    // table's stage-9 and stage-10 entries are stored in that order)
    from_lds<0>(lds, v, brev8(t));
    stage<0, 1, false, 16>(v, t, tw, q);   // a < 16q, < 20q
    stage<0, 0, false, 0>(v, t, tw, q);    //          < 24q
    // v[k] holds A_{brev11(8 brev8(t) + k)} = A_{t + 256 brev3(k)}
    swap_brev3(v);
    __syncthreads();
}

// Inverse NTT without the final n^-1 scaling.  On entry v[k] = A[t + 256 k]
// (values < 4q); on exit v[k] = n a[t + 256 k] in [0, 4q).  lds must be free on entry
// (its first access is a write); ends with a barrier.  tw: the prime's inverse table in
// the order of host::ntt2048_twiddle_order.
__device__ __forceinline__ void inv(uint64_t (&v)[E], uint64_t *lds, const uint64_t *__restrict__ tw, uint64_t qv) {
    const int t = threadIdx.x;
    const BfConsts q = bf_consts(qv);
    // thread t takes the bit-reversed indices 8 brev8(t) + k, at the natural positions
    // t + 256 brev3(k): v[brev3(k)] (the stages' twiddle index uses t: the table's stage-8, -9
    // and -10 entries are stored in that order)
    swap_brev3(v);
    stage<0, 0, true>(v, t, tw, q);
    stage<0, 1, true>(v, t, tw, q);
    stage<0, 2, true>(v, t, tw, q);
    to_lds<0>(lds, v, brev8(t));
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
