// Per-kernel timing with HIP events, recorded on the stream each kernel is
// launched on.  Off by default; when on, every launcher's ProfScope records an
// event pair, and hstu_profile_read() waits for them and reports
// "name count total_ms" per kernel name.
#include <stdio.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "hstu_attn.h"

namespace hstu {

namespace {

struct Pending {
  std::string name;
  hipEvent_t start, stop;
};

struct Totals {
  long count = 0;
  double ms = 0.0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::map<std::string, Totals> g_totals;

void drain_locked() {
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      Totals& t = g_totals[p.name];
      t.count += 1;
      t.ms += ms;
    }
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
}

}  // namespace

ProfScope::ProfScope(hipStream_t stream, const char* name) : stream_(stream), name_(name) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on) return;
  if (hipEventCreate(&start_) != hipSuccess) {
    start_ = nullptr;
    return;
  }
  if (hipEventRecord(start_, stream_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    start_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t stop = nullptr;
  if (hipEventCreate(&stop) == hipSuccess && hipEventRecord(stop, stream_) == hipSuccess) {
    g_pending.push_back(Pending{name_, start_, stop});
  } else {
    (void)hipEventDestroy(start_);
    if (stop) (void)hipEventDestroy(stop);
  }
}

}  // namespace hstu

using namespace hstu;

extern "C" int hstu_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_mu);
  const int prev = g_on ? 1 : 0;
  g_on = on != 0;
  return prev;
}

extern "C" void hstu_profile_reset(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  drain_locked();
  g_totals.clear();
}

extern "C" size_t hstu_profile_read(char* buf, size_t len) {
  std::lock_guard<std::mutex> lock(g_mu);
  drain_locked();
  std::string out;
  char line[256];
  for (const auto& kv : g_totals) {
    snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.count,
             kv.second.ms);
    out += line;
  }
  if (buf && len > 0) {
    const size_t n = out.size() < len - 1 ? out.size() : len - 1;
    out.copy(buf, n);
    buf[n] = '\0';
  }
  return out.size() + 1;
}
