// Per-kernel timing with HIP events attached to each kernel's dispatch (see
// trace.h).  The only mutable global
// state of the library; it is touched only while tracing is enabled.
#include "trace.h"

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace ds4 {
namespace {

struct Pending {
  int id;
  hipEvent_t a, b;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<std::string> g_names;
std::vector<double> g_ms;
std::vector<long long> g_count;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;

hipEvent_t get_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int name_id(const char* name) {
  for (size_t i = 0; i < g_names.size(); ++i)
    if (g_names[i] == name) return (int)i;
  g_names.emplace_back(name);
  g_ms.push_back(0.0);
  g_count.push_back(0);
  return (int)g_names.size() - 1;
}

// kernel names arrive as written in the launch macro: "k_x", "(k_x<16, true>)"
std::string clean(const char* raw) {
  std::string s(raw);
  while (!s.empty() && (s.front() == '(' || s.front() == ' ')) s.erase(s.begin());
  while (!s.empty() && (s.back() == ')' || s.back() == ' ')) s.pop_back();
  return s;
}

}  // namespace

TraceScope::TraceScope(const char* name, hipStream_t s) : st(s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a = get_event();
  b = get_event();
  if (!a || !b) {
    if (a) g_free.push_back(a);
    if (b) g_free.push_back(b);
    a = b = nullptr;
    return;
  }
  id = name_id(clean(name).c_str());
}

TraceScope::~TraceScope() {
  if (id < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back(Pending{id, a, b});
}

}  // namespace ds4

using namespace ds4;

extern "C" {

int ds4moe_trace_enable(int on) {
  g_on.store(on ? 1 : 0);
  return DS4MOE_OK;
}

int ds4moe_trace_read(char* names, size_t names_cap, double* ms, long long* counts, int cap, int reset) {
  std::lock_guard<std::mutex> lk(g_mu);
  // entries are taken off the list as they are counted, so an error midway
  // leaves only the uncounted ones pending
  size_t done = 0;
  int rc = DS4MOE_OK;
  for (; done < g_pending.size(); ++done) {
    const Pending& p = g_pending[done];
    float t = 0.0f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&t, p.a, p.b) != hipSuccess) {
      rc = DS4MOE_EHIP;
      break;
    }
    g_ms[p.id] += t;
    g_count[p.id] += 1;
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.erase(g_pending.begin(), g_pending.begin() + (std::ptrdiff_t)done);
  if (rc != DS4MOE_OK) return rc;
  const int n = (int)g_names.size();
  std::string joined;
  for (int i = 0; i < n && i < cap; ++i) {
    if (ms) ms[i] = g_ms[i];
    if (counts) counts[i] = g_count[i];
    joined += g_names[i];
    joined += '\n';
  }
  if (names && names_cap) {
    size_t m = std::min(names_cap - 1, joined.size());
    std::memcpy(names, joined.data(), m);
    names[m] = '\0';
  }
  if (reset) {
    for (int i = 0; i < n; ++i) {
      g_ms[i] = 0.0;
      g_count[i] = 0;
    }
  }
  return n;
}

}  // extern "C"
