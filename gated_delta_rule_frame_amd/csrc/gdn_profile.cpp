// Per-kernel timing with HIP events on the launch stream (diagnostics only).
#include <atomic>
#include <mutex>
#include <vector>

#include "gdn_internal.h"

namespace gdn {
namespace {

struct Pending {
  int kernel;
  hipEvent_t start, stop;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;          // reusable events
std::vector<Pending> g_pending;          // recorded, not yet read
Pending g_open[GDN_KERNEL_COUNT];        // started, not yet ended
long long g_launches[GDN_KERNEL_COUNT] = {};
double g_ms[GDN_KERNEL_COUNT] = {};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Waits for every pending pair and folds it into the totals.
void drain_locked() {
  for (Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      g_launches[p.kernel] += 1;
      g_ms[p.kernel] += ms;
    }
    g_pool.push_back(p.start);
    g_pool.push_back(p.stop);
  }
  g_pending.clear();
}

}  // namespace

void prof_begin(hipStream_t stream, int kernel) {
  if (!g_enabled.load(std::memory_order_relaxed) || kernel < 0 || kernel >= GDN_KERNEL_COUNT) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Pending p{kernel, take_event(), take_event()};
  if (!p.start || !p.stop) return;
  (void)hipEventRecord(p.start, stream);
  g_open[kernel] = p;
}

void prof_end(hipStream_t stream, int kernel) {
  if (!g_enabled.load(std::memory_order_relaxed) || kernel < 0 || kernel >= GDN_KERNEL_COUNT) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Pending p = g_open[kernel];
  if (!p.start || !p.stop) return;
  (void)hipEventRecord(p.stop, stream);
  g_pending.push_back(p);
  g_open[kernel] = Pending{kernel, nullptr, nullptr};
}

}  // namespace gdn

extern "C" {

gdn_status gdn_profile_enable(int32_t on) {
  gdn::g_enabled.store(on != 0);
  return GDN_OK;
}

gdn_status gdn_profile_reset(void) {
  std::lock_guard<std::mutex> lk(gdn::g_mu);
  gdn::drain_locked();
  for (int k = 0; k < GDN_KERNEL_COUNT; ++k) {
    gdn::g_launches[k] = 0;
    gdn::g_ms[k] = 0.0;
  }
  return GDN_OK;
}

gdn_status gdn_profile_read(int32_t kernel, int64_t* launches, double* total_ms) {
  if (kernel < 0 || kernel >= GDN_KERNEL_COUNT || !launches || !total_ms) return GDN_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(gdn::g_mu);
  gdn::drain_locked();
  *launches = gdn::g_launches[kernel];
  *total_ms = gdn::g_ms[kernel];
  return GDN_OK;
}

const char* gdn_kernel_name(int32_t kernel) {
  switch (kernel) {
    case GDN_KERNEL_SEG_MAP: return "seg_map_kernel";
    case GDN_KERNEL_SEG_CHAIN: return "seg_chain_kernel";
    case GDN_KERNEL_SEG_OUT: return "seg_out_kernel";
    case GDN_KERNEL_RECURRENT: return "recurrent_kernel";
    case GDN_KERNEL_JAC_MAP: return "jac_map_kernel";
    case GDN_KERNEL_JAC_OUT: return "jac_out_kernel";
    case GDN_KERNEL_PROLOGUE: return "prologue_kernel";
    case GDN_KERNEL_SCAN_PREP: return "scan_prep_kernel";
    case GDN_KERNEL_SCAN: return "scan_kernel";
    default: return "";
  }
}

}  // extern "C"
