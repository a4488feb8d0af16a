// multipass_kernels.h -- kernels of the four-step NTT (see multipass.h).
//
// A workgroup of 256 threads transforms 16 length-256 vectors held in LDS;
// each thread owns 16 elements of one vector, so a vector is two 4-stage
// register passes with one LDS exchange (forward: bits 7..4 then 3..0,
// merged-psi Cooley-Tukey; inverse: Gentleman-Sande in the mirror order).
// The thread -> (vector, lane) assignment is chosen per kernel so that every
// global access is a run of 16 consecutive uint64 (128 bytes).
#pragma once
#include "ckks_common.h"
#include "multipass.h"

namespace ckks {
namespace mp {

constexpr int LOG = 8, E = 16, V = 16;
constexpr int VSTRIDE = 264;  // LDS words per vector (256 + padding)

__device__ __forceinline__ int slot(int v, int i) { return v * VSTRIDE + i + (i >> 5); }
template <int C>
__device__ __forceinline__ int own(int t, int k) {  // element k of lane t in a pass owning bits [C, C+4)
    return (t & ((1 << C) - 1)) | (k << C) | ((t >> C) << (C + 4));
}
__device__ __forceinline__ int brev8(int i) { return (int)(__builtin_bitreverse32((uint32_t)i) >> 24); }

__device__ __forceinline__ void bf_ct(uint64_t &x, uint64_t &y, uint64_t w, uint64_t wp, uint64_t q) {
    const uint64_t q2 = 2 * q;
    const uint64_t a = x >= q2 ? x - q2 : x;
    const uint64_t t = shoup_lazy(y, w, wp, q);
    x = a + t;
    y = a - t + q2;
}
__device__ __forceinline__ void bf_gs(uint64_t &x, uint64_t &y, uint64_t w, uint64_t wp, uint64_t q) {
    const uint64_t q2 = 2 * q;
    const uint64_t s = x + y, d = x - y + q2;
    x = s >= q2 ? s - q2 : s;
    y = shoup_lazy(d, w, wp, q);
}

template <int C, int BIT, bool INV>
__device__ __forceinline__ void stage(uint64_t (&x)[E], int t, const uint64_t *__restrict__ tw, uint64_t q) {
    constexpr int s = LOG - 1 - BIT;
    constexpr int kb = 1 << (BIT - C);
#pragma unroll
    for (int k = 0; k < E; k++) {
        if (k & kb) continue;
        const int j = own<C>(t, k);
        const int ti = (1 << s) + (j >> (LOG - s));
        if (INV) bf_gs(x[k], x[k | kb], tw[2 * ti], tw[2 * ti + 1], q);
        else bf_ct(x[k], x[k | kb], tw[2 * ti], tw[2 * ti + 1], q);
    }
}

// Forward: x[k] = element t + 16k (natural, < 4q) of vector v on entry; on
// exit the transform sits in lds in natural order (values < 4q).
__device__ __forceinline__ void fwd(uint64_t (&x)[E], uint64_t *lds, int v, int t, const uint64_t *__restrict__ tw,
                                    uint64_t q) {
    stage<4, 7, false>(x, t, tw, q);
    stage<4, 6, false>(x, t, tw, q);
    stage<4, 5, false>(x, t, tw, q);
    stage<4, 4, false>(x, t, tw, q);
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(v, own<4>(t, k))] = x[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = lds[slot(v, own<0>(t, k))];
    stage<0, 3, false>(x, t, tw, q);
    stage<0, 2, false>(x, t, tw, q);
    stage<0, 1, false>(x, t, tw, q);
    stage<0, 0, false>(x, t, tw, q);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(v, brev8(own<0>(t, k)))] = x[k];
    __syncthreads();
}

// Inverse (without 1/256): x[k] = element t + 16k (natural, < 2q) on entry
// and on exit (values < 2q).  Ends with a barrier.
__device__ __forceinline__ void inv(uint64_t (&x)[E], uint64_t *lds, int v, int t, const uint64_t *__restrict__ tw,
                                    uint64_t q) {
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(v, brev8(own<4>(t, k)))] = x[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = lds[slot(v, own<0>(t, k))];
    stage<0, 0, true>(x, t, tw, q);
    stage<0, 1, true>(x, t, tw, q);
    stage<0, 2, true>(x, t, tw, q);
    stage<0, 3, true>(x, t, tw, q);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < E; k++) lds[slot(v, own<0>(t, k))] = x[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = lds[slot(v, own<4>(t, k))];
    stage<4, 4, true>(x, t, tw, q);
    stage<4, 5, true>(x, t, tw, q);
    stage<4, 6, true>(x, t, tw, q);
    stage<4, 7, true>(x, t, tw, q);
    __syncthreads();
}

// ---- forward pass 1: columns i2 in [16 bx, +16) of limb; T applied; -> scratch
template <class Map>
__global__ __launch_bounds__(256) void k_fwd_cols(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ tw, const uint64_t *__restrict__ cross,
                                                   uint64_t *__restrict__ scratch) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const uint64_t q = pc[prime].q;
    const int v = threadIdx.x % V, t = threadIdx.x / V;
    const int c0 = blockIdx.x * V;
    uint64_t x[E];
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = src[(size_t)(t + 16 * k) * MP_N1 + c0 + v];
    fwd(x, lds, v, t, tw + (size_t)prime * MP_N1 * 2, q);
    const uint64_t *T = cross + (size_t)prime * MP_N1 * MP_N1 * 2;
    uint64_t *o = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
#pragma unroll
    for (int k = 0; k < E; k++) {
        const int j1 = t + 16 * k;
        const size_t e = (size_t)j1 * MP_N1 + c0 + v;
        o[e] = shoup_lazy(lds[slot(v, j1)], T[2 * e], T[2 * e + 1], q);  // [0, 2q)
    }
}

// ---- forward pass 2: rows j1 in [16 bx, +16) of scratch; outputs A[j1 + 256 j2] -> dst
template <class Map>
__global__ __launch_bounds__(256) void k_fwd_rows(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ tw,
                                                   const uint64_t *__restrict__ scratch) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const uint64_t q = pc[prime].q;
    const int r0 = blockIdx.x * V;
    const uint64_t *in = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
    {
        const int t = threadIdx.x % 16, v = threadIdx.x / 16;  // lanes along a row
        uint64_t x[E];
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = in[(size_t)(r0 + v) * MP_N1 + t + 16 * k];
        fwd(x, lds, v, t, tw + (size_t)prime * MP_N1 * 2, q);
    }
    const int v = threadIdx.x % V, t = threadIdx.x / V;  // lanes across rows for the transposed store
#pragma unroll
    for (int k = 0; k < E; k++) {
        const int j2 = t + 16 * k;
        uint64_t y = lds[slot(v, j2)];
        y = y >= 2 * q ? y - 2 * q : y;
        dst[(size_t)(r0 + v) + (size_t)MP_N1 * j2] = csub(y, q);
    }
}

// ---- inverse pass 1: rows j1 = 16 bx + v: gather A[j1 + 256 j2], inverse, T^-1 -> scratch[j1][i2]
template <class Map>
__global__ __launch_bounds__(256) void k_inv_rows(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ tw,
                                                   const uint64_t *__restrict__ crossinvT,
                                                   uint64_t *__restrict__ scratch) {
    __shared__ uint64_t lds[V * VSTRIDE];
    const uint64_t *src;
    uint64_t *dst;
    int prime;
    const uint64_t *sc;
    const uint32_t limb = limb0 + blockIdx.y;
    map.get(limb, src, dst, prime, sc);
    if (!src) return;
    const uint64_t q = pc[prime].q;
    const int r0 = blockIdx.x * V;
    const uint64_t *Ti = crossinvT + (size_t)prime * MP_N1 * MP_N1 * 2;
    {
        const int v = threadIdx.x % V, t = threadIdx.x / V;
        uint64_t x[E];
#pragma unroll
        for (int k = 0; k < E; k++) x[k] = src[(size_t)(r0 + v) + (size_t)MP_N1 * (t + 16 * k)];
        inv(x, lds, v, t, tw + (size_t)prime * MP_N1 * 2, q);
#pragma unroll
        for (int k = 0; k < E; k++) {
            const size_t e = (size_t)(t + 16 * k) * MP_N1 + r0 + v;  // transposed table: [i2][j1]
            lds[slot(v, t + 16 * k)] = shoup_lazy(x[k], Ti[2 * e], Ti[2 * e + 1], q);
        }
    }
    __syncthreads();
    const int t = threadIdx.x % 16, v = threadIdx.x / 16;
    uint64_t *o = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
#pragma unroll
    for (int k = 0; k < E; k++) o[(size_t)(r0 + v) * MP_N1 + t + 16 * k] = lds[slot(v, t + 16 * k)];
}

// ---- inverse pass 2: columns i2 = 16 bx + v of scratch; inverse; scale -> dst[256 i1 + i2]
template <class Map>
__global__ __launch_bounds__(256) void k_inv_cols(Map map, uint32_t limb0, const PrimeConsts *__restrict__ pc,
                                                   const uint64_t *__restrict__ tw,
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
    const uint64_t q = P.q;
    const int v = threadIdx.x % V, t = threadIdx.x / V;
    const int c0 = blockIdx.x * V;
    const uint64_t *in = scratch + (size_t)blockIdx.y * MP_N1 * MP_N1;
    uint64_t x[E];
#pragma unroll
    for (int k = 0; k < E; k++) x[k] = in[(size_t)(t + 16 * k) * MP_N1 + c0 + v];
    inv(x, lds, v, t, tw + (size_t)prime * MP_N1 * 2, q);
    const uint64_t w = sc ? sc[0] : P.ninv, wp = sc ? sc[1] : P.ninvp;
#pragma unroll
    for (int k = 0; k < E; k++) {
        const uint64_t r = shoup(x[k], w, wp, q);
        dst[(size_t)(t + 16 * k) * MP_N1 + c0 + v] = Map::split_out ? split30(r) : r;
    }
}

}  // namespace mp

template <class Map>
int multipass_ntt(const ckks_ctx *c, const Map &map, int nblk, bool inverse, hipStream_t s) {
    const MultipassPlan *p = c->mp;
    if (!p) return CKKS_EUNSUPPORTED;
    const dim3 blk(256);
    for (int l0 = 0; l0 < nblk; l0 += MP_CHUNK) {
        const dim3 grid(MP_N1 / mp::V, (unsigned)std::min<int>(MP_CHUNK, nblk - l0));
        if (!inverse) {
            hipLaunchKernelGGL(mp::k_fwd_cols<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_tw256f,
                               p->d_cross, p->d_scratch);
            hipLaunchKernelGGL(mp::k_fwd_rows<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_tw256f,
                               (const uint64_t *)p->d_scratch);
        } else {
            hipLaunchKernelGGL(mp::k_inv_rows<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_tw256i,
                               p->d_crossinvT, p->d_scratch);
            hipLaunchKernelGGL(mp::k_inv_cols<Map>, grid, blk, 0, s, map, (uint32_t)l0, c->d_pc, p->d_tw256i,
                               (const uint64_t *)p->d_scratch);
        }
        if (hipGetLastError() != hipSuccess) return CKKS_EHIP;
    }
    return CKKS_OK;
}

}  // namespace ckks
