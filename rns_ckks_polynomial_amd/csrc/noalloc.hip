// noalloc.hip -- rotation whose key-switching workspace is a file-scope device
// array, for callers that cannot allocate device memory (code under stream
// capture, serving loops, harnesses that forbid hipMalloc).
//
// The array lives in the library's code object: each GPU the library runs on
// holds one copy for the life of the process.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): its
// device address is looked up once per device with hipGetSymbolAddress, at
// context creation with that device current, and that address is what the
// launches receive.  Every call on a device shares its copy, so calls that
// overlap on one GPU race; the key switch writes every word of the workspace
// it later reads, so nothing needs clearing between calls.
#include <mutex>

#include "../../include/ckks_gpu.h"
#include "ctx_internal.h"
#include "ops.h"

namespace {

constexpr size_t NOALLOC_WORDS = CKKS_NOALLOC_SCRATCH_BYTES / 8;
static __device__ __align__(256) uint64_t scratch[NOALLOC_WORDS];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES] = {};  // device address of `scratch` on each device

}  // namespace

namespace ckks {

// Called with `device` current (context creation).
int noalloc_init(int device) {
    if (device < 0 || device >= MAX_DEVICES) return CKKS_EUNSUPPORTED;
    std::lock_guard<std::mutex> g(g_mu);
    if (g_ptr[device]) return CKKS_OK;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CKKS_EHIP;
    g_ptr[device] = p;
    return CKKS_OK;
}

}  // namespace ckks

using namespace ckks;

extern "C" int ckks_rotate_noalloc(const ckks_ctx *c, const uint64_t *in, uint64_t *out, int batch, int level,
                                   uint32_t galois_elt, const ckks_swk *key, void *stream) {
    if (!c || !c->K || batch < 1) return CKKS_EINVAL;
    if (level < 1 || (uint32_t)level > c->L) return CKKS_ELEVEL;
    if (c->device < 0 || c->device >= MAX_DEVICES) return CKKS_EUNSUPPORTED;
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> g(g_mu);
        ws = g_ptr[c->device];
    }
    if (!ws) return CKKS_EHIP;
    const size_t need = ws_bytes_rotate(c, batch, level);
    if (need > CKKS_NOALLOC_SCRATCH_BYTES) return CKKS_EWORKSPACE;
    // the same validation and launches as ckks_rotate, with the device array as its workspace
    return ckks_rotate(c, in, out, batch, level, galois_elt, key, ws, need, stream);
}
