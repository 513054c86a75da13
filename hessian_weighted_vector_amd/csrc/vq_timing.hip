// Optional per-step GPU timing: when enabled, each step launcher brackets its
// kernels with HIP events recorded on the stream the kernels run on.  The
// events are read (and the durations summed per (step name, K)) only when
// the caller asks, after the work has completed.  Disabled by default; the
// only cost when disabled is one flag test per launch.
#include "vq_internal.h"

#include <cstdio>
#include <iterator>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

namespace vq {
namespace {

struct Pending {
    std::string name;
    int K;
    hipEvent_t a, b;
};

struct Stat {
    int64_t launches = 0;
    double total_ms = 0.0, min_ms = 1e300, max_ms = 0.0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::map<std::pair<std::string, int>, Stat> g_stats;

hipEvent_t take_event()
{
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void drain_locked()
{
    for (auto& p : g_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            Stat& s = g_stats[{p.name, p.K}];
            s.launches += 1;
            s.total_ms += ms;
            s.min_ms = ms < s.min_ms ? ms : s.min_ms;
            s.max_ms = ms > s.max_ms ? ms : s.max_ms;
        }
        g_free.push_back(p.a);
        g_free.push_back(p.b);
    }
    g_pending.clear();
}

}  // namespace

TimedRegion::TimedRegion(const char* name, int K, hipStream_t st) : name_(name), K_(K), st_(st)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    a_ = take_event();
    if (a_ && hipEventRecord(static_cast<hipEvent_t>(a_), st_) != hipSuccess) a_ = nullptr;
}

TimedRegion::~TimedRegion()
{
    if (!a_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t b = take_event();
    if (!b) return;
    if (hipEventRecord(b, st_) != hipSuccess) return;
    g_pending.push_back({name_, K_, static_cast<hipEvent_t>(a_), b});
}

bool timing_on()
{
    std::lock_guard<std::mutex> lk(g_mu);
    return g_on;
}

void timing_count(const char* name, int K, int64_t n)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    Stat& s = g_stats[{name, K}];
    s.launches += n;
    s.min_ms = 0.0;
}

}  // namespace vq

using namespace vq;

extern "C" {

void vq_timing_enable(int on)
{
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    g_stats.clear();
    g_on = on != 0;
}

int vq_timing_count(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    return (int)g_stats.size();
}

int vq_timing_get(int i, char* name, int name_len, int* K, int64_t* launches, double* total_ms,
                  double* min_ms, double* max_ms)
{
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    if (i < 0 || i >= (int)g_stats.size()) return 1;
    auto it = g_stats.begin();
    std::advance(it, i);
    if (name && name_len > 0) {
        std::snprintf(name, (size_t)name_len, "%s", it->first.first.c_str());
    }
    if (K) *K = it->first.second;
    if (launches) *launches = it->second.launches;
    if (total_ms) *total_ms = it->second.total_ms;
    if (min_ms) *min_ms = it->second.min_ms;
    if (max_ms) *max_ms = it->second.max_ms;
    return 0;
}

}  // extern "C"
