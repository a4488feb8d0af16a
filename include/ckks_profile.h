/*
 * ckks_profile.h -- optional per-launch timing of the library's kernels.
 *
 * Between ckks_profile_begin and ckks_profile_end every kernel launch made by
 * the context is bracketed by two HIP events recorded on the launch's own
 * stream.  ckks_profile_end waits for those events and returns, per kernel
 * name, the launch count and the summed / min / max event-to-event times.
 * Intended for measurement (it adds two event records per launch); calls on
 * one context from several host threads while profiling is on are serialised
 * by an internal lock.
 */
#ifndef CKKS_PROFILE_H
#define CKKS_PROFILE_H
#include "ckks_gpu.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    char name[48];
    int launches;
    double total_ms, min_ms, max_ms;
} ckks_kernel_stat;

/* Start recording (clears earlier records). */
int ckks_profile_begin(ckks_ctx *ctx);
/* Stop recording, synchronise, and copy up to max_entries aggregated rows to
 * out (host array); *n_entries receives the number of distinct names. */
int ckks_profile_end(ckks_ctx *ctx, ckks_kernel_stat *out, int max_entries, int *n_entries);

#ifdef __cplusplus
}
#endif
#endif
