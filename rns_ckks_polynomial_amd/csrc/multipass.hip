// multipass.hip -- tables of the large-n NTT.
#include "multipass.h"

namespace ckks {
int multipass_init(ckks_ctx *ctx) { (void)ctx; return CKKS_EUNSUPPORTED; }
void multipass_free(ckks_ctx *ctx) { (void)ctx; }
}  // namespace ckks
