/*
 * ckks_synth.h -- seeded synthetic inputs generated directly in HBM.
 *
 * Not part of the arithmetic: a device-side implementation of the SplitMix64
 * counter-based generator (Steele, Lea, Flood, OOPSLA 2014) used to fill
 * large benchmark / test inputs without a host round trip.
 *
 * Definition (identical to the CPU-side generator module):
 *   splitmix(s, i)   = mix64(s + (i + 1) * 0x9e3779b97f4a7c15)
 *   mix64(z)         = z ^= z >> 30, z *= 0xbf58476d1ce4e5b9,
 *                      z ^= z >> 27, z *= 0x94d049bb133111eb, z ^ (z >> 31)
 *   stream(seed,tag,j) = splitmix(splitmix(seed, tag), j)
 *   element i of stream j modulo q: first value v = splitmix(w, r) & (2^60-1),
 *     r = 0, 1, ..., 63, with v < q, where w = splitmix(stream(seed,tag,j), i);
 *     after 64 misses, the last v mod q.
 */
#ifndef CKKS_SYNTH_H
#define CKKS_SYNTH_H
#include <stdint.h>

#include "ckks_gpu.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Fill dst ([count][nlimbs][n], device) with uniform residues: limb r of
 * polynomial c is modulo prime first_prime + r and uses stream
 * stream0 + c * nlimbs + r. */
int ckks_fill_uniform(const ckks_ctx *ctx, uint64_t *dst, int count, int first_prime, int nlimbs, uint64_t seed,
                      uint64_t tag, uint64_t stream0, void *stream);

#ifdef __cplusplus
}
#endif
#endif
