// Opt-in per-kernel timing: HIP event pairs around every kernel the library
// launches, on the stream it launches on. Off by default; host-side state is
// process-global and not thread-safe (instrumentation for benchmarks).
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <string.h>

#include <vector>

namespace gdn {
namespace prof {

struct Rec {
    const char* name;
    hipEvent_t start, stop;
};

static bool g_on = false;
static std::vector<Rec> g_pool;
static size_t g_used = 0;
static bool g_failed = false;

void begin(hipStream_t s, const char* name) {
    if (!g_on) return;
    if (g_used == g_pool.size()) {
        Rec r{name, nullptr, nullptr};
        if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
            g_failed = true;
            return;
        }
        g_pool.push_back(r);
    }
    g_pool[g_used].name = name;
    if (hipEventRecord(g_pool[g_used].start, s) != hipSuccess) g_failed = true;
}

void end(hipStream_t s) {
    if (!g_on || g_used >= g_pool.size()) return;
    if (hipEventRecord(g_pool[g_used].stop, s) != hipSuccess) g_failed = true;
    ++g_used;
}

}  // namespace prof
}  // namespace gdn

extern "C" {

gdn_status_t gdn_profile_start(void) {
    gdn::prof::g_on = true;
    gdn::prof::g_used = 0;
    gdn::prof::g_failed = false;
    return GDN_OK;
}

int32_t gdn_profile_stop(int32_t max_kernels, char* names, int32_t* counts, double* total_ms) {
    using namespace gdn::prof;
    g_on = false;
    if (g_failed) return -1;
    int32_t nk = 0;
    for (size_t i = 0; i < g_used; ++i) {
        if (hipEventSynchronize(g_pool[i].stop) != hipSuccess) return -1;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_pool[i].start, g_pool[i].stop) != hipSuccess) return -1;
        int32_t j = 0;
        while (j < nk && strncmp(names + 64 * j, g_pool[i].name, 63) != 0) ++j;
        if (j == nk) {
            if (nk == max_kernels) continue;
            strncpy(names + 64 * j, g_pool[i].name, 63);
            names[64 * j + 63] = '\0';
            counts[j] = 0;
            total_ms[j] = 0.0;
            ++nk;
        }
        counts[j] += 1;
        total_ms[j] += ms;
    }
    g_used = 0;
    return nk;
}

}  // extern "C"
