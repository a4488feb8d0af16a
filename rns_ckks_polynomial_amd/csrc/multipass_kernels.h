// multipass_kernels.h -- launch templates of the large-n NTT (see multipass.h).
#pragma once
#include "multipass.h"

namespace ckks {

template <class Map>
int multipass_ntt(const ckks_ctx *c, const Map &map, int nblk, bool inverse, hipStream_t s) {
    (void)c; (void)map; (void)nblk; (void)inverse; (void)s;
    return CKKS_EUNSUPPORTED;
}

}  // namespace ckks
