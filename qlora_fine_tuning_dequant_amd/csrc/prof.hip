// Optional per-kernel timing with HIP events, recorded on the stream each
// kernel is launched on. Off unless qlx_profile_begin() is called; then every
// launcher (or only those whose row name starts with a given prefix)
// brackets its kernel with an event pair and notes the kernel's algorithmic
// flops and HBM bytes, and qlx_profile_end() sums them per kernel.
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "qlx_internal.h"

namespace qlx {

namespace {
struct Rec {
    const char* name;
    double flops, bytes;
    hipEvent_t b, e;
};
std::mutex g_mu;
bool g_on = false;
std::string g_prefix;  // only rows whose name starts with it (empty: all)
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
size_t g_used = 0;

hipEvent_t take_event() {
    if (g_used == g_pool.size()) {
        // timing only: no system-scope fence (a cache writeback and invalidate
        // that would inflate the measured window and slow the next kernel)
        hipEvent_t e;
        QLX_CHECK_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
        g_pool.push_back(e);
    }
    return g_pool[g_used++];
}
}  // namespace

ProfScope::ProfScope(const char* name, double flops, double bytes, hipStream_t s, bool ext) : s_(s), ext_(ext) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    if (!g_prefix.empty() && std::strncmp(name, g_prefix.c_str(), g_prefix.size()) != 0) return;
    idx_ = int64_t(g_recs.size());
    Rec r{name, flops, bytes, take_event(), take_event()};
    if (!ext_) QLX_CHECK_HIP(hipEventRecord(r.b, s));
    g_recs.push_back(r);
}

ProfScope::~ProfScope() {
    if (idx_ < 0 || ext_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (idx_ < int64_t(g_recs.size())) (void)hipEventRecord(g_recs[idx_].e, s_);
}

hipEvent_t ProfScope::start() const {
    std::lock_guard<std::mutex> lk(g_mu);
    return (idx_ >= 0 && idx_ < int64_t(g_recs.size())) ? g_recs[idx_].b : nullptr;
}
hipEvent_t ProfScope::stop() const {
    std::lock_guard<std::mutex> lk(g_mu);
    return (idx_ >= 0 && idx_ < int64_t(g_recs.size())) ? g_recs[idx_].e : nullptr;
}

}  // namespace qlx

using namespace qlx;

extern "C" int qlx_profile_begin_prefix(const char* name_prefix) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.clear();
    g_used = 0;
    g_prefix = name_prefix ? name_prefix : "";
    g_on = true;
    return QLX_OK;
}

extern "C" int qlx_profile_begin(void) { return qlx_profile_begin_prefix(nullptr); }

extern "C" int qlx_profile_end(qlx_kernel_prof* out, int max_out, int* count) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = false;
    try {
        struct Agg {
            int64_t n = 0;
            double ms = 0, flops = 0, bytes = 0;
        };
        std::map<std::string, Agg> agg;
        for (const Rec& r : g_recs) {
            QLX_CHECK_HIP(hipEventSynchronize(r.e));
            float ms = 0.f;
            QLX_CHECK_HIP(hipEventElapsedTime(&ms, r.b, r.e));
            Agg& a = agg[r.name];
            a.n += 1;
            a.ms += ms;
            a.flops += r.flops;
            a.bytes += r.bytes;
        }
        int i = 0;
        for (const auto& kv : agg) {
            if (out && i < max_out) {
                std::memset(&out[i], 0, sizeof(qlx_kernel_prof));
                std::strncpy(out[i].name, kv.first.c_str(), sizeof(out[i].name) - 1);
                out[i].launches = kv.second.n;
                out[i].ms = kv.second.ms;
                out[i].flops = kv.second.flops;
                out[i].bytes = kv.second.bytes;
            }
            ++i;
        }
        if (count) *count = i;
        g_recs.clear();
        g_used = 0;
        return QLX_OK;
    } catch (const Error& e) {
        set_error(e.msg);
        return e.code;
    }
}
