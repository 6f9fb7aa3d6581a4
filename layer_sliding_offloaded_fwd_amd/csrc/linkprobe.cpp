// Host-link diagnostic: the time of one copy between pinned host memory and HBM on each of the
// GPU's copy engines, in both directions. The slot ring's copies (SlideFormer summary, section
// 2A: layers and gradients cross the host link asynchronously) run on whichever engine the HIP
// runtime picks, and the engines differ several-fold on this link; this call measures that.
#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>
#include <string.h>

#include <chrono>

#include "../../include/slide.h"

namespace slide {
int fail(int code, const char* fmt, ...);
}
using slide::fail;

namespace {
int agent_of(const void* p, size_t n, bool host, hsa_agent_t* agent) {
  hsa_amd_pointer_info_t info;
  memset(&info, 0, sizeof info);
  info.size = sizeof info;
  if (hsa_amd_pointer_info(p, &info, nullptr, nullptr, nullptr) != HSA_STATUS_SUCCESS)
    return fail(SLIDE_E_HIP, "host_link_engine_rates: hsa_amd_pointer_info failed");
  const bool ok = host ? (info.type == HSA_EXT_POINTER_TYPE_HSA ||
                          info.type == HSA_EXT_POINTER_TYPE_LOCKED)
                       : info.type == HSA_EXT_POINTER_TYPE_HSA;
  const char* base = (const char*)(host ? info.hostBaseAddress : info.agentBaseAddress);
  if (!ok || (const char*)p < base || (const char*)p + n > base + info.sizeInBytes)
    return fail(SLIDE_E_ARG, "host_link_engine_rates: %s buffer is not %s memory of %zu bytes",
                host ? "host" : "device", host ? "pinned" : "device", n);
  *agent = info.agentOwner;
  return SLIDE_OK;
}
}  // namespace

extern "C" int slide_host_link_engine_rates(void* dev, void* host, size_t nbytes, int reps,
                                            double* d2h_ms, double* h2d_ms, uint32_t* info4) {
  if (!dev || !host || !d2h_ms || !h2d_ms || !info4 || nbytes == 0 || reps < 1)
    return fail(SLIDE_E_ARG, "host_link_engine_rates: bad arguments");
  for (int e = 0; e < 32; ++e) d2h_ms[e] = h2d_ms[e] = -1.0;
  if (hipDeviceSynchronize() != hipSuccess)
    return fail(SLIDE_E_HIP, "host_link_engine_rates: hipDeviceSynchronize failed");
  if (hsa_init() != HSA_STATUS_SUCCESS) return fail(SLIDE_E_HIP, "host_link_engine_rates: hsa_init failed");
  int rc = SLIDE_OK;
  hsa_agent_t gpu{}, cpu{};
  hsa_signal_t sig{};
  if ((rc = agent_of(dev, nbytes, false, &gpu)) == SLIDE_OK &&
      (rc = agent_of(host, nbytes, true, &cpu)) == SLIDE_OK) {
    uint32_t ne = 0, nx = 0, pref_d2h = 0, pref_h2d = 0, avail_d2h = 0, avail_h2d = 0;
    hsa_agent_get_info(gpu, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_ENG, &ne);
    hsa_agent_get_info(gpu, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_XGMI_ENG, &nx);
    hsa_amd_memory_get_preferred_copy_engine(cpu, gpu, &pref_d2h);
    hsa_amd_memory_get_preferred_copy_engine(gpu, cpu, &pref_h2d);
    hsa_amd_memory_copy_engine_status(cpu, gpu, &avail_d2h);
    hsa_amd_memory_copy_engine_status(gpu, cpu, &avail_h2d);
    info4[0] = ne;
    info4[1] = nx;
    info4[2] = pref_d2h;
    info4[3] = pref_h2d;
    if (hsa_signal_create(1, 0, nullptr, &sig) != HSA_STATUS_SUCCESS)
      rc = fail(SLIDE_E_HIP, "host_link_engine_rates: hsa_signal_create failed");
    for (int dir = 0; rc == SLIDE_OK && dir < 2; ++dir) {
      const uint32_t avail = dir == 0 ? avail_d2h : avail_h2d;
      for (int e = 0; rc == SLIDE_OK && e < 32; ++e) {
        if (!(avail & (1u << e))) continue;
        double best = 1e30;
        for (int k = 0; k < reps; ++k) {
          hsa_signal_store_relaxed(sig, 1);
          const auto t0 = std::chrono::steady_clock::now();
          const hsa_status_t st =
              dir == 0 ? hsa_amd_memory_async_copy_on_engine(host, cpu, dev, gpu, nbytes, 0,
                                                             nullptr, sig,
                                                             (hsa_amd_sdma_engine_id_t)(1u << e),
                                                             true)
                       : hsa_amd_memory_async_copy_on_engine(dev, gpu, host, cpu, nbytes, 0,
                                                             nullptr, sig,
                                                             (hsa_amd_sdma_engine_id_t)(1u << e),
                                                             true);
          if (st != HSA_STATUS_SUCCESS) break;   // engine refused: left at -1
          // bounded: a copy of this size takes milliseconds
          bool done = false;
          for (int w = 0; w < 200 && !done; ++w)
            done = hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_LT, 1, 100000000,
                                             HSA_WAIT_STATE_BLOCKED) < 1;
          if (!done) {
            rc = fail(SLIDE_E_TIMEOUT, "host_link_engine_rates: engine %d did not finish", e);
            break;
          }
          const double ms =
              std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0)
                  .count();
          if (ms < best) best = ms;
        }
        if (best < 1e30) (dir == 0 ? d2h_ms : h2d_ms)[e] = best;
      }
    }
  }
  // a copy that did not finish in time may still write its signal: leave that signal (and the
  // runtime reference) alive rather than free them under it
  if (rc == SLIDE_E_TIMEOUT) return rc;
  if (sig.handle) hsa_signal_destroy(sig);
  hsa_shut_down();
  return rc;
}
