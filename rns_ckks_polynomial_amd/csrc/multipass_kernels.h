// multipass_kernels.h -- kernels of the four-step NTT (see multipass.h).
//
// A workgroup of 256 threads transforms 16 length-256 vectors held in LDS;
// each thread owns 16 elements of one vector, so a vector is two 4-stage
// register passes with one LDS exchange (forward: bits 7..4 then 3..0,
// merged-psi Cooley-Tukey; inverse: Gentleman-Sande in the mirror order).
// The thread -> (vector, lane) assignment is chosen per kernel so that every
// global access is a run of at least 16 consecutive uint64 (128 bytes).  The
// transpose buffer is blocked by V columns (sidx), so the column kernels move one
// contiguous block and the row kernels 2 KiB runs.
// Butterflies are the lazy forms of butterfly.h.
#pragma once
#include "butterfly.h"
#include "multipass.h"

namespace ckks {
namespace mp {

constexpr int LOG = 8, E = 16, V = 16;
constexpr int NT = 16 * V;  // threads per workgroup: 16 per vector
// LDS words per vector: 256 + one pad word per 16.  The column kernels put consecutive
// vectors in consecutive lanes, the row kernels consecutive elements of one vector; with
// this stride and padding every exchange pattern of both (own<4>, own<0> and their bit
// reversals) spreads a half-wave's 64-bit accesses evenly over the banks (264 with a pad
// per 32, the stride for the row layout alone, put 8 to 16 lanes of a column kernel on one
// bank).
constexpr int VSTRIDE = 273;

// Word of element (row j1, column i2) of a limb in the transpose buffer: blocks of V columns.
__device__ __forceinline__ uint32_t sidx(uint32_t j1, uint32_t i2) {
    return (i2 / V) * (MP_N1 * V) + j1 * V + i2 % V;
}

// islot(a | b) = islot(a) + islot(b) for a and b without common bits, so the exchanges
// are a per-thread base plus a compile-time offset per register.
__device__ __forceinline__ constexpr int islot(int i) { return i + (i >> 4); }
__device__ __forceinline__ int slot(int v, int i) { return v * VSTRIDE + islot(i); }
template <int C>
__device__ __forceinline__ int own(int t, int k) {  // element k of lane t in a pass owning bits [C, C+4)
    return (t & ((1 << C) - 1)) | (k << C) | ((t >> C) << (C + 4));
}
__device__ __forceinline__ constexpr int brev8(int i) { return (int)(__builtin_bitreverse32((uint32_t)i) >> 24); }

// One radix-2 stage (bit BIT) on the 16 registers of a pass owning bits [C, C+4);
// tw holds the heap-ordered twiddles (index 2^s + b at stage s).
template <int C, int BIT, bool INV, int RED = 0>
__device__ __forceinline__ void stage(uint64_t (&x)[E], int t, const uint64_t *__restrict__ tw, const BfConsts &c) {
    constexpr int s = LOG - 1 - BIT;
    constexpr int kb = 1 << (BIT - C);
#pragma unroll
    for (int k = 0; k < E; k++) {
        if (k & kb) continue;
        const int j = own<C>(t, k);
        const int ti = (1 << s) + (j >> (LOG - s));
        if (INV) bf_gs(x[k], x[k | kb], tw[2 * ti], tw[2 * ti + 1], c);
        else bf_ct<RED>(x[k], x[k | kb], tw[2 * ti], tw[2 * ti + 1], c);
    }
}

// Forward: x[k] = element t + 16k (natural, < 4q) of vector v on entry; on
// exit the transform sits in lds in natural order, values < 24q.
// Bounds: a stage without reduction maps inputs below B q to outputs below (B + 4) q;
// the top input is reduced below 16q at stages 3 and 1, so no value reaches 24q.
__device__ __forceinline__ void fwd(uint64_t (&x)[E], uint64_t *lds, int v, int t, const uint64_t *__restrict__ tw,
                                    const BfConsts &c) {
    stage<4, 7, false>(x, t, tw, c);      // < 8q
    stage<4, 6, false>(x, t, tw, c);      // < 12q
    stage<4, 5, false>(x, t, tw, c);      // < 16q
    stage<4, 4, false>(x, t, tw, c);      // < 20q
    {  // own<4>(t, k) = t | 16k, own<0>(t, k) = 16t | k (t < 16)
        uint64_t *b = lds + slot(v, t);
#pragma unroll
        for (int k = 0; k < E; k++) b[islot(16 * k)] = x[k];
    }
    __syncthreads();
    {
        const uint64_t *b = lds + slot(v, 16 * t);
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = b[islot(k)];
    }
    stage<0, 3, false, 16>(x, t, tw, c);  // < 20q
    stage<0, 2, false>(x, t, tw, c);      // < 24q
    stage<0, 1, false, 16>(x, t, tw, c);  // < 20q
    stage<0, 0, false>(x, t, tw, c);      // < 24q
    __syncthreads();
    {  // brev8(16t | k) = brev8(16t) | brev8(k)
        uint64_t *b = lds + slot(v, brev8(16 * t));
#pragma unroll
        for (int k = 0; k < E; k++) b[islot(brev8(k))] = x[k];
    }
    __syncthreads();
}

// Inverse (without 1/256): x[k] = element t + 16k (natural, < 4q) on entry
// and on exit (values < 4q).  Ends with a barrier.
__device__ __forceinline__ void inv(uint64_t (&x)[E], uint64_t *lds, int v, int t, const uint64_t *__restrict__ tw,
                                    const BfConsts &c) {
    {  // brev8(t | 16k) = brev8(t) | brev8(16k)
        uint64_t *b = lds + slot(v, brev8(t));
#pragma unroll
        for (int k = 0; k < E; k++) b[islot(brev8(16 * k))] = x[k];
    }
    __syncthreads();
    {
        const uint64_t *b = lds + slot(v, 16 * t);
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = b[islot(k)];
    }
    stage<0, 0, true>(x, t, tw, c);
    stage<0, 1, true>(x, t, tw, c);
    stage<0, 2, true>(x, t, tw, c);
    stage<0, 3, true>(x, t, tw, c);
    __syncthreads();
    {
        uint64_t *b = lds + slot(v, 16 * t);
#pragma unroll
        for (int k = 0; k < E; k++) b[islot(k)] = x[k];
    }
    __syncthreads();
    {
        const uint64_t *b = lds + slot(v, t);
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = b[islot(16 * k)];
    }
    stage<4, 4, true>(x, t, tw, c);
    stage<4, 5, true>(x, t, tw, c);
    stage<4, 6, true>(x, t, tw, c);
    stage<4, 7, true>(x, t, tw, c);
    __syncthreads();
}

// ---- forward pass 1: columns i2 in [16 bx, +16) of limb; times TA -> scratch (< 4q)
template <class Map>
__global__ __launch_bounds__(NT) void k_fwd_cols(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ tw, const uint64_t *__restrict__ taf,
                                                   uint64_t *__restrict__ scratch) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const BfConsts c = bf_consts(pc[prime].q);
    const int v = threadIdx.x % V, t = threadIdx.x / V;
    const int c0 = blockIdx.x * V;
    // this thread's factor TA[i2][t] of the cross twiddle (rows t + 16 k of column i2)
    const uint64_t *ta = taf + (((size_t)prime * MP_N1 + c0 + v) * 16 + t) * 2;
    const uint64_t w = ta[0], wp = ta[1];
    uint64_t x[E];
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = src[(size_t)(t + 16 * k) * MP_N1 + c0 + v];
    fwd(x, lds, v, t, tw + (size_t)prime * MP_N1 * 2, c);
    uint64_t *o = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
    const uint64_t *lb = lds + slot(v, t);
#pragma unroll
    for (int k = 0; k < E; k++) {
        const int j1 = t + 16 * k;
        o[sidx(j1, c0 + v)] = shoup_lazy4(lb[islot(16 * k)], w, wp, 0 - c.q);  // [0, 4q)
    }
}

// ---- forward pass 2: rows j1 in [16 bx, +16) of scratch (k = bx); outputs A[j1 + 256 j2] -> dst.
// GAL: the outputs come out permuted by the automorphism X -> X^g (odd g < 2n), out[j] = A[g j + (g-1)/2
// mod n].  With j = j1 + 256 j2 the source index splits as j1' = (g j1 + (g-1)/2) mod 256 and
// j2' = (g j2 + floor((g j1 + (g-1)/2) / 256)) mod 256, so output row j1 is the transform of row j1'
// read in a permuted order: the workgroup transforms the rows j1' of its 16 output rows (each with the
// twiddles of its own group j1' / 16) and gathers from LDS.
template <class Map, bool GAL>
__global__ __launch_bounds__(NT) void k_fwd_rows(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ rowf,
                                                   const uint64_t *__restrict__ scratch, uint32_t g) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const uint64_t q = pc[prime].q;
    const BfConsts c = bf_consts(q);
    const int r0 = blockIdx.x * V;
    const uint64_t *in = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
    {
        const int t = threadIdx.x % 16, v = threadIdx.x / 16;  // lanes along a row
        const uint32_t row = GAL ? ((g * (uint32_t)(r0 + v) + (g >> 1)) & (MP_N1 - 1)) : (uint32_t)(r0 + v);
        uint64_t x[E];
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = in[sidx(row, t + 16 * k)];
        fwd(x, lds, v, t, rowf + ((size_t)prime * 16 + (row >> 4)) * MP_N1 * 2, c);
    }
    const int v = threadIdx.x % V, t = threadIdx.x / V;  // lanes across rows for the transposed store
    const uint32_t carry = GAL ? (g * (uint32_t)(r0 + v) + (g >> 1)) >> MP_LOG1 : 0;
    const uint64_t *lb = lds + slot(v, t);
#pragma unroll
    for (int k = 0; k < E; k++) {
        const uint32_t j2 = t + 16 * k;
        const uint64_t y = GAL ? lds[slot(v, (g * j2 + carry) & (MP_N1 - 1))] : lb[islot(16 * k)];
        dst[(size_t)(r0 + v) + (size_t)MP_N1 * j2] = reduce_out(y, q);
    }
}

// ---- inverse pass 1: rows j1 = 16 bx + v: gather A[j1 + 256 j2], inverse row transform -> scratch[j1][i2]
template <class Map>
__global__ __launch_bounds__(NT) void k_inv_rows(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ rowi, uint64_t *__restrict__ scratch) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const BfConsts c = bf_consts(pc[prime].q);
    const int r0 = blockIdx.x * V;
    {
        const int v = threadIdx.x % V, t = threadIdx.x / V;
        uint64_t x[E];
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = src[(size_t)(r0 + v) + (size_t)MP_N1 * (t + 16 * k)];
        inv(x, lds, v, t, rowi + ((size_t)prime * 16 + ((r0 + v) >> 4)) * MP_N1 * 2, c);
        uint64_t *lb = lds + slot(v, t);
#pragma unroll
        for (int k = 0; k < E; k++) lb[islot(16 * k)] = x[k];
    }
    __syncthreads();
    const int t = threadIdx.x % 16, v = threadIdx.x / 16;
    uint64_t *o = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
    const uint64_t *lb = lds + slot(v, t);
#pragma unroll
    for (int k = 0; k < E; k++) o[sidx(r0 + v, t + 16 * k)] = lb[islot(16 * k)];
}

// ---- inverse pass 2: columns i2 = 16 bx + v of scratch; times TA^-1, inverse; scale -> dst[256 i1 + i2]
template <class Map>
__global__ __launch_bounds__(NT) void k_inv_cols(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ tw, const uint64_t *__restrict__ tai,
                                                   const uint64_t *__restrict__ scratch) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const PrimeConsts &P = pc[prime];
    const BfConsts c = bf_consts(P.q);
    const int v = threadIdx.x % V, t = threadIdx.x / V;
    const int c0 = blockIdx.x * V;
    const uint64_t *ta = tai + (((size_t)prime * MP_N1 + c0 + v) * 16 + t) * 2;
    const uint64_t wa = ta[0], wap = ta[1];
    const uint64_t *in = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
    uint64_t x[E];
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = shoup_lazy4(in[sidx(t + 16 * k, c0 + v)], wa, wap, 0 - c.q);
    inv(x, lds, v, t, tw + (size_t)prime * MP_N1 * 2, c);
    const uint64_t w = sc ? sc[0] : P.ninv, wp = sc ? sc[1] : P.ninvp;
#pragma unroll
    for (int k = 0; k < E; k++) {
        const uint64_t r = shoup(x[k], w, wp, P.q);
        dst[(size_t)(t + 16 * k) * MP_N1 + c0 + v] = Map::digit_out ? digit_form(r) : r;
    }
}

}  // namespace mp

template <class Map>
static int multipass_launch(const ckks_ctx *c, const Map &map, int nblk, bool inverse, hipStream_t s,
                            uint64_t *scratch, uint32_t gal) {
    const MultipassPlan *p = c->mp;
    const dim3 blk(mp::NT);
    for (int l0 = 0, ch = mp_chunk(nblk); l0 < nblk; l0 += ch) {
        const dim3 grid(MP_N1 / mp::V, (unsigned)std::min<int>(ch, nblk - l0));
        if (!inverse) {
            hipLaunchKernelGGL(mp::k_fwd_cols<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_tw256f,
                               p->d_taf, scratch);
            if (gal == 1)
                hipLaunchKernelGGL((mp::k_fwd_rows<Map, false>), grid, blk, 0, s, map, (uint32_t)l0, c->d_pc,
                                   p->d_rowf, (const uint64_t *)scratch, 1u);
            else
                hipLaunchKernelGGL((mp::k_fwd_rows<Map, true>), grid, blk, 0, s, map, (uint32_t)l0, c->d_pc,
                                   p->d_rowf, (const uint64_t *)scratch, gal);
        } else {
            hipLaunchKernelGGL(mp::k_inv_rows<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_rowi,
                               scratch);
            hipLaunchKernelGGL(mp::k_inv_cols<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_tw256i,
                               p->d_tai, (const uint64_t *)scratch);
        }
        if (hipGetLastError() != hipSuccess) return CKKS_EHIP;
    }
    return CKKS_OK;
}

// scratch: the caller's transpose buffer of mp_scratch_words(n) words, or null for
// the context's, whose users wait for the previous user's event on their stream.
// gal: an odd Galois element whose automorphism permutes the forward outputs
// (1: natural order; ignored by the inverse).
template <class Map>
int multipass_ntt(const ckks_ctx *c, const Map &map, int nblk, bool inverse, hipStream_t s, uint64_t *scratch,
                  uint32_t gal = 1) {
    MultipassPlan *p = c->mp;
    if (!p) return CKKS_EUNSUPPORTED;
    if (scratch) return multipass_launch(c, map, nblk, inverse, s, scratch, gal);
    std::lock_guard<std::mutex> lk(p->scratch_mu);
    if (hipStreamWaitEvent(s, p->scratch_done, 0) != hipSuccess) return CKKS_EHIP;
    const int e = multipass_launch(c, map, nblk, inverse, s, p->d_scratch, gal);
    if (hipEventRecord(p->scratch_done, s) != hipSuccess) return CKKS_EHIP;
    return e;
}

}  // namespace ckks
