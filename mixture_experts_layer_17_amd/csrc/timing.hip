// Optional per-kernel timing: when enabled, every kernel the library launches
// is bracketed by two HIP events recorded on the caller's stream.  Events come
// from a pool that grows on first use and is reused afterwards, so after one
// warm-up pass the timed passes create nothing.  Reading the report waits for
// the recorded events and sums elapsed time per kernel name.  Off by default.
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace moe {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<hipEvent_t> g_pool;
size_t g_used = 0;
std::vector<Rec> g_recs;

hipEvent_t take_event() {
  if (g_used == g_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_used++];
}

}  // namespace

bool timing_on() { return g_on; }

void timing_mark(const char* name, hipStream_t s, bool begin) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  hipEvent_t e = take_event();
  if (!e) return;
  hipEventRecord(e, s);
  if (begin) {
    g_recs.push_back(Rec{name, e, nullptr});
  } else if (!g_recs.empty()) {
    g_recs.back().b = e;
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  g_recs.clear();
  g_used = 0;
  return MOE_OK;
}

extern "C" int moe_timing_report(char* buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!buf || len == 0) return MOE_EINVAL;
  std::map<std::string, std::pair<long, double>> acc;
  for (const Rec& r : g_recs) {
    if (!r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return MOE_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return MOE_EHIP;
    auto& v = acc[r.name];
    v.first += 1;
    v.second += ms;
  }
  std::string out;
  for (const auto& kv : acc)
    out += kv.first + " " + std::to_string(kv.second.first) + " " + std::to_string(kv.second.second) + "\n";
  g_recs.clear();
  g_used = 0;
  if (out.size() + 1 > len) return MOE_EINVAL;
  for (size_t i = 0; i < out.size(); ++i) buf[i] = out[i];
  buf[out.size()] = 0;
  return MOE_OK;
}
