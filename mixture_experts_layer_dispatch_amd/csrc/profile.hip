// Opt-in kernel timing: HIP events around each launch on its stream.
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "profile.h"

namespace moe {
namespace {

struct Pending {
    const char* name;
    hipEvent_t a, b;
};

struct State {
    std::mutex mu;
    std::atomic<bool> on{false};
    std::vector<hipEvent_t> pool;
    std::vector<Pending> pending;
    std::map<std::string, std::pair<int64_t, double>> stats;
};

State& st() {
    static State s;
    return s;
}

hipEvent_t take_event(State& s) {
    if (!s.pool.empty()) {
        hipEvent_t e = s.pool.back();
        s.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

ProfScope::ProfScope(hipStream_t stream, const char* name) : stream_(stream), name_(name) {
    State& s = st();
    if (!s.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(s.mu);
    a_ = take_event(s);
    b_ = take_event(s);
    if (a_ && b_) (void)hipEventRecord(a_, stream_);
}

ProfScope::~ProfScope() {
    if (!a_ || !b_) return;
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    (void)hipEventRecord(b_, stream_);
    s.pending.push_back({name_, a_, b_});
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_profile_enable(int on) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    s.on = on != 0;
    return MOE_OK;
}

moe_status moe_profile_collect(void) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    moe_status rc = MOE_OK;
    for (Pending& p : s.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
            rc = MOE_ERR_HIP;
        } else {
            auto& v = s.stats[p.name];
            v.first += 1;
            v.second += ms;
        }
        s.pool.push_back(p.a);
        s.pool.push_back(p.b);
    }
    s.pending.clear();
    return rc;
}

moe_status moe_profile_query(const char* name, int64_t* launches, double* total_ms) {
    if (!name || !launches || !total_ms) return MOE_ERR_INVALID_ARG;
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    auto it = s.stats.find(name);
    *launches = it == s.stats.end() ? 0 : it->second.first;
    *total_ms = it == s.stats.end() ? 0.0 : it->second.second;
    return MOE_OK;
}

moe_status moe_profile_names(char* buf, size_t cap) {
    if (!buf || cap == 0) return MOE_ERR_INVALID_ARG;
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    std::string out;
    for (auto& kv : s.stats) out += kv.first + "\n";
    size_t n = out.size() < cap - 1 ? out.size() : cap - 1;
    out.copy(buf, n);
    buf[n] = 0;
    return MOE_OK;
}

moe_status moe_profile_reset(void) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    s.stats.clear();
    return MOE_OK;
}

}  // extern "C"
