// profile.hip -- per-launch event timing (see include/ckks_profile.h).
#include <string.h>

#include <algorithm>

#include "../../include/ckks_profile.h"
#include "ctx_internal.h"

namespace ckks {

hipEvent_t Profiler::take() {
    if (used == pool.size()) {
        hipEvent_t e{};
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        pool.push_back(e);
    }
    return pool[used++];
}

int Profiler::name_id(const char *n) {
    for (size_t i = 0; i < names.size(); i++)
        if (names[i] == n) return (int)i;
    names.emplace_back(n);
    return (int)names.size() - 1;
}

}  // namespace ckks

using namespace ckks;

extern "C" int ckks_profile_begin(ckks_ctx *c) {
    if (!c) return CKKS_EINVAL;
    if (!c->prof) c->prof = new Profiler();
    std::lock_guard<std::mutex> g(c->prof->mu);
    c->prof->recs.clear();
    c->prof->used = 0;
    c->prof->on = true;
    return CKKS_OK;
}

extern "C" int ckks_profile_end(ckks_ctx *c, ckks_kernel_stat *out, int max_entries, int *n_entries) {
    if (!c || !c->prof) return CKKS_EINVAL;
    Profiler *p = c->prof;
    std::lock_guard<std::mutex> g(p->mu);
    p->on = false;
    const size_t nn = p->names.size();
    std::vector<ckks_kernel_stat> agg(nn);
    for (size_t i = 0; i < nn; i++) {
        memset(&agg[i], 0, sizeof(ckks_kernel_stat));
        strncpy(agg[i].name, p->names[i].c_str(), sizeof(agg[i].name) - 1);
        agg[i].min_ms = 1e30;
    }
    int err = CKKS_OK;
    for (const auto &r : p->recs) {
        float ms = 0;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            err = CKKS_EHIP;
            continue;
        }
        ckks_kernel_stat &a = agg[r.name];
        a.launches++;
        a.total_ms += ms;
        a.min_ms = std::min(a.min_ms, (double)ms);
        a.max_ms = std::max(a.max_ms, (double)ms);
    }
    int k = 0;
    for (size_t i = 0; i < nn; i++) {
        if (!agg[i].launches) continue;
        if (out && k < max_entries) out[k] = agg[i];
        k++;
    }
    if (n_entries) *n_entries = k;
    p->recs.clear();
    p->used = 0;
    return err;
}
