// Slot ring: the pre-allocated GPU cache queue of the layer-sliding method (SlideFormer
// summary, section 2B: a fixed set of identical buffers holding only the active layers'
// parameters and gradients, each reused as soon as it is free, so nothing is allocated while
// training; section 2A: gradients leave asynchronously while the next layer computes and the
// layer after that is prefetched, on transfer streams separate from the compute stream).
//
// All ordering is expressed with events so that the host never blocks on the GPU except in
// slide_slot_ring_wait_flush (the CPU optimizer needs the gradients in host memory):
//   load     copy stream waits for the slot's last release event, then copies the weights
//   acquire  compute stream waits for the load and for any flush still reading the slot
//   flush    copy stream waits for the compute stream, then copies the gradients out
//   release  records an event on the compute stream (the next load into the slot waits on it)
// The host engine runs the same state machine on host memory with a copy thread, so the
// bookkeeping and its failure paths can be exercised without a GPU.
//
// The HSA engine moves the same bytes on chosen copy engines. hipMemcpyAsync lets the runtime
// pick the engine, and on this GPU the engines built for copies between GPUs run the host link
// at a quarter of the host-optimised ones' rate or less; whole steps' gradient copies have landed
// there. Here a host thread per direction runs the copies in order with
// hsa_amd_memory_async_copy_on_engine: before a copy it waits on the host for the HIP events
// the HIP engine would make the copy stream wait for (the slot's release for a load, the
// compute stream's work for a flush), and it waits on the host for the copy's completion
// signal. No GPU queue ever waits on a host-written value; instead acquire blocks the calling
// thread until the slot's load (and any flush still reading it) has completed, as the host
// engine's acquire does. Every host wait is bounded.
#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/slide.h"

namespace slide {
int fail(int code, const char* fmt, ...);
}
using slide::fail;

namespace {

constexpr int kTicketPool = 1024;
// Copy engines of the HSA engine: two of the host-optimised ones (engines 0-3 run the host link
// at ~57 GB/s in both directions on this GPU, the others at 7-13 GB/s device to host), one per
// direction so that uploads and gradient copies run side by side, and neither of them engine 0,
// which also carries the runtime's own copies (with gradient copies on engine 0 the batch-32
// step's copies took 357 ms per step against 284-300 ms on engines 1, 2 or 3).
constexpr int kHsaEngineH2D = 3, kHsaEngineD2H = 1;

// ------------------------------------------------------------------ host engine pieces
struct HostEvent {
  std::atomic<int> st{1};  // 0 pending, 1 done, 2 failed
  double t_done = 0;       // CLOCK_MONOTONIC seconds at completion (HSA engine)
};

double mono_now() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

struct HostCopyQueue {
  struct Job {
    std::vector<std::shared_ptr<HostEvent>> waits;
    void* dst;
    const void* src;
    size_t n;
    std::shared_ptr<HostEvent> done;
    int fault;  // 0 none, 1 fail, 2 never complete
  };
  std::mutex mu;
  std::condition_variable cv;
  std::deque<Job> q;
  bool stop = false;
  std::thread th;

  HostCopyQueue() { th = std::thread([this] { run(); }); }
  ~HostCopyQueue() {
    {
      std::lock_guard<std::mutex> lk(mu);
      stop = true;
    }
    cv.notify_all();
    th.join();
  }
  void push(Job j) {
    {
      std::lock_guard<std::mutex> lk(mu);
      q.push_back(std::move(j));
    }
    cv.notify_all();
  }
  void run() {
    for (;;) {
      Job j;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || !q.empty(); });
        if (stop && q.empty()) return;
        j = std::move(q.front());
        q.pop_front();
      }
      bool dep_failed = false;
      for (auto& w : j.waits) {
        // a dependency that never completes stalls this queue, as a GPU stream would
        while (w->st.load() == 0) {
          {
            std::lock_guard<std::mutex> lk(mu);
            if (stop) return;
          }
          std::this_thread::sleep_for(std::chrono::microseconds(100));
        }
        if (w->st.load() == 2) dep_failed = true;
      }
      if (j.fault == 2) continue;  // never completes
      if (j.fault == 1 || dep_failed) {
        j.done->st.store(2);
        continue;
      }
      memcpy(j.dst, j.src, j.n);
      j.done->t_done = mono_now();
      j.done->st.store(1);
    }
  }
};

// ------------------------------------------------------------------ HSA engine pieces
constexpr int kHsaWaitMs = 60000;   // bound of every host wait of the HSA engine's threads

// The HSA agent that owns a pointer (the GPU for device memory, the CPU for pinned host memory).
bool agent_of(const void* p, hsa_agent_t* agent) {
  hsa_amd_pointer_info_t info;
  memset(&info, 0, sizeof info);
  info.size = sizeof info;
  if (hsa_amd_pointer_info(p, &info, nullptr, nullptr, nullptr) != HSA_STATUS_SUCCESS)
    return false;
  if (info.type != HSA_EXT_POINTER_TYPE_HSA && info.type != HSA_EXT_POINTER_TYPE_LOCKED)
    return false;
  *agent = info.agentOwner;
  return true;
}

struct HsaCopyQueue {
  struct Job {
    hipEvent_t gpu_wait = nullptr;   // GPU work to finish first (HIP event)
    bool own_gpu_wait = false;       // destroy the event once waited for
    void* dst;
    const void* src;
    size_t n;
    bool to_device;
    std::shared_ptr<HostEvent> done;
  };
  hsa_agent_t gpu{};
  uint32_t engine = 0;               // hsa_amd_sdma_engine_id_t bit
  hsa_signal_t sig{};
  std::mutex mu;
  std::condition_variable cv;
  std::deque<Job> q;
  bool stop = false;
  // A copy that ran out of time may still be in flight and would signal sig later: no further
  // copy is issued on this queue (every later job fails), and sig is never destroyed under it.
  bool broken = false;
  std::thread th;

  HsaCopyQueue(hsa_agent_t g, uint32_t eng) : gpu(g), engine(eng) {
    hsa_signal_create(1, 0, nullptr, &sig);
    th = std::thread([this] { run(); });
  }
  ~HsaCopyQueue() {
    {
      std::lock_guard<std::mutex> lk(mu);
      stop = true;
    }
    cv.notify_all();
    th.join();
    if (sig.handle && !broken) hsa_signal_destroy(sig);
  }
  void push(Job j) {
    {
      std::lock_guard<std::mutex> lk(mu);
      q.push_back(std::move(j));
    }
    cv.notify_all();
  }
  // 0 done, 1 failed, 2 ran out of time
  int wait_gpu(hipEvent_t e) {
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
      const hipError_t r = hipEventQuery(e);
      if (r == hipSuccess) return 0;
      if (r != hipErrorNotReady) return 1;
      if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(kHsaWaitMs)) return 2;
      // a copy takes milliseconds: polling every 200 us starts it at most that late, and leaves
      // the cores to the CPU optimizer
      std::this_thread::sleep_for(std::chrono::microseconds(200));
    }
  }
  int copy(const Job& j) {
    hsa_agent_t host_agent;
    if (!agent_of(j.to_device ? j.src : j.dst, &host_agent)) return 1;
    hsa_signal_store_relaxed(sig, 1);
    const hsa_status_t st =
        j.to_device
            ? hsa_amd_memory_async_copy_on_engine(j.dst, gpu, j.src, host_agent, j.n, 0, nullptr,
                                                  sig, (hsa_amd_sdma_engine_id_t)engine, true)
            : hsa_amd_memory_async_copy_on_engine(j.dst, host_agent, j.src, gpu, j.n, 0, nullptr,
                                                  sig, (hsa_amd_sdma_engine_id_t)engine, true);
    if (st != HSA_STATUS_SUCCESS) return 1;
    for (int w = 0; w < kHsaWaitMs / 100; ++w)   // 100 ms per wait
      if (hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_LT, 1, 100000000,
                                    HSA_WAIT_STATE_BLOCKED) < 1)
        return 0;
    return 2;
  }
  void run() {
    for (;;) {
      Job j;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || !q.empty(); });
        if (stop && q.empty()) return;
        j = std::move(q.front());
        q.pop_front();
      }
      int rc = broken ? 1 : 0;
      if (j.gpu_wait) {
        if (rc == 0) rc = wait_gpu(j.gpu_wait);
        if (j.own_gpu_wait) hipEventDestroy(j.gpu_wait);
      }
      if (rc == 0) {
        rc = copy(j);
        if (rc == 2) broken = true;
      }
      j.done->t_done = mono_now();
      j.done->st.store(rc == 0 ? 1 : 2);
    }
  }
};

// ------------------------------------------------------------------ slot
struct Ev {
  hipEvent_t hip = nullptr;
  std::shared_ptr<HostEvent> host;
  bool valid = false;
};

struct Slot {
  int state = SLIDE_SLOT_FREE;
  int layer = -1;
  bool content_valid = false;
  uint64_t released_at = 0;
  Ev load_ev, free_ev, flush_ev;
};

}  // namespace

struct slide_ring {
  int n = 0;
  size_t wb = 0, gb = 0;
  char* base = nullptr;
  hipStream_t h2d = nullptr, d2h = nullptr;
  int engine = SLIDE_ENGINE_HIP;
  std::vector<Slot> slots;
  uint64_t clock = 1;
  std::mutex mu;
  // flush tickets
  uint64_t next_ticket = 1;
  std::vector<Ev> ticket_ev;
  std::vector<uint64_t> ticket_id;
  // host engine
  std::unique_ptr<HostCopyQueue> hq_h2d, hq_d2h;
  // HSA engine
  std::unique_ptr<HsaCopyQueue> sq_h2d, sq_d2h;
  bool hsa_up = false;
  int fault_mode = 0, fault_count = 0;

  char* w_ptr(int s) { return base + (size_t)s * (wb + gb); }
  char* g_ptr(int s) { return base + (size_t)s * (wb + gb) + wb; }

  int take_fault() {
    if (fault_count <= 0) return 0;
    --fault_count;
    return fault_mode;
  }

  bool host_events() const { return engine != SLIDE_ENGINE_HIP; }

  // record an event "now" on a compute stream (host engine: host compute is synchronous)
  int record_compute(Ev& e, void* stream) {
    if (engine == SLIDE_ENGINE_HOST) {
      e.host = std::make_shared<HostEvent>();
      e.valid = true;
      return SLIDE_OK;
    }
    if (!e.hip && hipEventCreateWithFlags(&e.hip, hipEventDisableTiming) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring: hipEventCreate failed");
    if (hipEventRecord(e.hip, (hipStream_t)stream) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring: hipEventRecord failed");
    e.valid = true;
    return SLIDE_OK;
  }

  // host wait for an event with a deadline (ms < 0: no limit)
  int host_wait(const Ev& e, int timeout_ms, const char* what) {
    if (!e.valid) return SLIDE_OK;
    auto t0 = std::chrono::steady_clock::now();
    for (;;) {
      int st;
      if (host_events()) {
        st = e.host->st.load();
        if (st == 2) return fail(SLIDE_E_HIP, "slot ring: %s: copy failed", what);
        if (st == 1) return SLIDE_OK;
      } else {
        hipError_t q = hipEventQuery(e.hip);
        if (q == hipSuccess) return SLIDE_OK;
        if (q != hipErrorNotReady)
          return fail(SLIDE_E_HIP, "slot ring: %s: %s", what, hipGetErrorString(q));
      }
      if (timeout_ms >= 0) {
        auto el = std::chrono::duration_cast<std::chrono::milliseconds>(
                      std::chrono::steady_clock::now() - t0).count();
        if (el >= timeout_ms)
          return fail(SLIDE_E_TIMEOUT, "slot ring: %s: no completion after %d ms", what,
                      timeout_ms);
      }
      std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
  }
};

namespace {
int check_ring(slide_ring* r, int slot) {
  if (!r) return fail(SLIDE_E_ARG, "slot ring: null handle");
  if (slot < 0 || slot >= r->n) return fail(SLIDE_E_ARG, "slot ring: slot %d out of range", slot);
  return SLIDE_OK;
}
const char* state_name(int s) {
  switch (s) {
    case SLIDE_SLOT_FREE: return "FREE";
    case SLIDE_SLOT_LOADING: return "LOADING";
    case SLIDE_SLOT_IN_USE: return "IN_USE";
    case SLIDE_SLOT_FLUSHING: return "FLUSHING";
  }
  return "?";
}
}  // namespace

extern "C" int slide_slot_ring_create(slide_ring** out, int n_slots, size_t w_bytes,
                                      size_t g_bytes, void* dev_base, void* h2d_stream,
                                      void* d2h_stream, int engine) {
  if (!out || !dev_base) return fail(SLIDE_E_ARG, "slot ring create: null pointer");
  if (n_slots < 1 || n_slots > 4096) return fail(SLIDE_E_ARG, "slot ring create: n_slots %d", n_slots);
  if (w_bytes == 0) return fail(SLIDE_E_ARG, "slot ring create: w_bytes must be > 0");
  if ((w_bytes % 256) || (g_bytes % 256))
    return fail(SLIDE_E_ARG, "slot ring create: w_bytes and g_bytes must be multiples of 256");
  if (engine != SLIDE_ENGINE_HIP && engine != SLIDE_ENGINE_HOST && engine != SLIDE_ENGINE_HSA)
    return fail(SLIDE_E_ARG, "slot ring create: unknown engine %d", engine);
  hsa_agent_t gpu{};
  if (engine == SLIDE_ENGINE_HSA) {
    if (hsa_init() != HSA_STATUS_SUCCESS) return fail(SLIDE_E_HIP, "slot ring create: hsa_init failed");
    if (!agent_of(dev_base, &gpu)) {
      hsa_shut_down();
      return fail(SLIDE_E_ARG, "slot ring create: dev_base is not device memory known to HSA");
    }
  }
  auto* r = new slide_ring();
  r->n = n_slots;
  r->wb = w_bytes;
  r->gb = g_bytes;
  r->base = (char*)dev_base;
  r->h2d = (hipStream_t)h2d_stream;
  r->d2h = (hipStream_t)d2h_stream;
  r->engine = engine;
  r->slots.resize(n_slots);
  r->ticket_ev.resize(kTicketPool);
  r->ticket_id.assign(kTicketPool, 0);
  if (engine == SLIDE_ENGINE_HOST) {
    r->hq_h2d.reset(new HostCopyQueue());
    r->hq_d2h.reset(new HostCopyQueue());
  }
  if (engine == SLIDE_ENGINE_HSA) {
    r->hsa_up = true;
    r->sq_h2d.reset(new HsaCopyQueue(gpu, 1u << kHsaEngineH2D));
    r->sq_d2h.reset(new HsaCopyQueue(gpu, 1u << kHsaEngineD2H));
  }
  *out = r;
  return SLIDE_OK;
}

namespace {
// Start (slot < 0: on the next FREE slot, which becomes LOADING) or continue (slot LOADING with
// this layer) the copy of weight bytes [off, off + n) from host_w + off into the slot. The
// slot's load event is re-recorded after every part; the copy stream runs the parts in order,
// so the last event covers them all.
int load_part(slide_ring* r, int layer, const void* host_w, size_t off, size_t n, int* slot_io,
              const char* what) {
  if (!r || !host_w || !slot_io) return fail(SLIDE_E_ARG, "slot ring %s: null pointer", what);
  if (n == 0 || off > r->wb || n > r->wb - off)
    return fail(SLIDE_E_ARG, "slot ring %s(layer %d): bytes [%zu, +%zu) outside the %zu-byte slot",
                what, layer, off, n, r->wb);
  std::lock_guard<std::mutex> lk(r->mu);
  int s = *slot_io;
  const bool first = s < 0;
  if (first) {
    for (int k = 0; k < r->n; ++k)
      if (r->slots[k].state == SLIDE_SLOT_FREE &&
          (s < 0 || r->slots[k].released_at < r->slots[s].released_at))
        s = k;
    if (s < 0) return fail(SLIDE_E_STATE, "slot ring %s(layer %d): no FREE slot", what, layer);
  } else {
    if (s >= r->n) return fail(SLIDE_E_ARG, "slot ring %s: slot %d out of range", what, s);
    if (r->slots[s].state != SLIDE_SLOT_LOADING || r->slots[s].layer != layer)
      return fail(SLIDE_E_STATE, "slot ring %s: slot %d is not LOADING layer %d", what, s,
                  layer);
  }
  Slot& sl = r->slots[s];
  char* dst = r->w_ptr(s) + off;
  const char* src = (const char*)host_w + off;
  if (r->engine == SLIDE_ENGINE_HOST) {
    HostCopyQueue::Job j;
    if (first && sl.free_ev.valid) j.waits.push_back(sl.free_ev.host);
    j.dst = dst;
    j.src = src;
    j.n = n;
    j.done = std::make_shared<HostEvent>();
    j.done->st.store(0);
    j.fault = r->take_fault();
    sl.load_ev.host = j.done;
    sl.load_ev.valid = true;
    r->hq_h2d->push(std::move(j));
  } else if (r->engine == SLIDE_ENGINE_HSA) {
    HsaCopyQueue::Job j;
    // the slot's release event stays valid until the slot is released again, which needs
    // this load to complete first (acquire waits for it)
    if (first && sl.free_ev.valid) j.gpu_wait = sl.free_ev.hip;
    j.dst = dst;
    j.src = src;
    j.n = n;
    j.to_device = true;
    j.done = std::make_shared<HostEvent>();
    j.done->st.store(0);
    sl.load_ev.host = j.done;
    sl.load_ev.valid = true;
    r->sq_h2d->push(std::move(j));
  } else {
    if (first && sl.free_ev.valid && hipStreamWaitEvent(r->h2d, sl.free_ev.hip, 0) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring %s: hipStreamWaitEvent failed", what);
    hipError_t e = hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, r->h2d);
    if (e != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring %s: hipMemcpyAsync: %s", what, hipGetErrorString(e));
    if (!sl.load_ev.hip &&
        hipEventCreateWithFlags(&sl.load_ev.hip, hipEventDisableTiming) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring %s: hipEventCreate failed", what);
    if (hipEventRecord(sl.load_ev.hip, r->h2d) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring %s: hipEventRecord failed", what);
    sl.load_ev.valid = true;
  }
  if (first) {
    sl.state = SLIDE_SLOT_LOADING;
    sl.layer = layer;
    sl.content_valid = true;
  }
  *slot_io = s;
  return SLIDE_OK;
}
}  // namespace

extern "C" int slide_slot_ring_load(slide_ring* r, int layer, const void* host_w, int* slot_out) {
  if (!slot_out) return fail(SLIDE_E_ARG, "slot ring load: null pointer");
  int s = -1;
  int rc = load_part(r, layer, host_w, 0, r ? r->wb : 0, &s, "load");
  if (rc == SLIDE_OK) *slot_out = s;
  return rc;
}

extern "C" int slide_slot_ring_load_range(slide_ring* r, int layer, const void* host_w,
                                          size_t offset, size_t nbytes, int* slot_inout) {
  return load_part(r, layer, host_w, offset, nbytes, slot_inout, "load_range");
}

// Re-claim a FREE slot whose weights still hold `layer` (nothing was loaded over them since),
// without copying. SLIDE_E_STATE if there is none.
extern "C" int slide_slot_ring_reuse(slide_ring* r, int layer, int* slot_out) {
  if (!r || !slot_out) return fail(SLIDE_E_ARG, "slot ring reuse: null pointer");
  std::lock_guard<std::mutex> lk(r->mu);
  for (int s = 0; s < r->n; ++s) {
    Slot& sl = r->slots[s];
    if (sl.state == SLIDE_SLOT_FREE && sl.content_valid && sl.layer == layer) {
      sl.state = SLIDE_SLOT_LOADING;  // its load event (already complete) still orders it
      *slot_out = s;
      return SLIDE_OK;
    }
  }
  return fail(SLIDE_E_STATE, "slot ring reuse: no FREE slot holds layer %d", layer);
}

extern "C" int slide_slot_ring_acquire(slide_ring* r, int slot, void* compute_stream,
                                       void** w_dev, void** g_dev) {
  int rc = check_ring(r, slot);
  if (rc) return rc;
  std::unique_lock<std::mutex> lk(r->mu);
  Slot& sl = r->slots[slot];
  if (sl.state != SLIDE_SLOT_LOADING)
    return fail(SLIDE_E_STATE, "slot ring acquire: slot %d is %s, expected LOADING", slot,
                state_name(sl.state));
  if (r->host_events()) {
    Ev le = sl.load_ev, fe = sl.flush_ev;
    lk.unlock();
    // host compute runs synchronously (host engine), and no GPU queue waits on a host-signalled
    // copy (HSA engine): the stream-side wait becomes a bounded host wait
    const int limit = r->engine == SLIDE_ENGINE_HSA ? kHsaWaitMs : 10000;
    rc = r->host_wait(le, limit, "acquire (load)");
    if (rc == SLIDE_OK) rc = r->host_wait(fe, limit, "acquire (pending flush)");
    if (rc) return rc;
    lk.lock();
  } else {
    if (sl.load_ev.valid &&
        hipStreamWaitEvent((hipStream_t)compute_stream, sl.load_ev.hip, 0) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring acquire: hipStreamWaitEvent failed");
    if (sl.flush_ev.valid &&
        hipStreamWaitEvent((hipStream_t)compute_stream, sl.flush_ev.hip, 0) != hipSuccess)
      return fail(SLIDE_E_HIP, "slot ring acquire: hipStreamWaitEvent failed");
  }
  sl.state = SLIDE_SLOT_IN_USE;
  if (w_dev) *w_dev = r->w_ptr(slot);
  if (g_dev) *g_dev = r->gb ? r->g_ptr(slot) : nullptr;
  return SLIDE_OK;
}

namespace {
// After the work queued so far on compute_stream: copy gradient bytes [off, off + n) of the
// slot to host_g + off on the d2h stream. The first part takes the slot from IN_USE to
// FLUSHING; further parts of the same flush are accepted while it is FLUSHING.
int flush_part(slide_ring* r, int slot, void* host_g, size_t off, size_t n,
               void* compute_stream, uint64_t* ticket, const char* what) {
  int rc = check_ring(r, slot);
  if (rc) return rc;
  if (!host_g || !ticket) return fail(SLIDE_E_ARG, "slot ring %s: null pointer", what);
  std::lock_guard<std::mutex> lk(r->mu);
  Slot& sl = r->slots[slot];
  if (r->gb == 0) return fail(SLIDE_E_STATE, "slot ring %s: ring has no gradient region", what);
  if (n == 0 || off > r->gb || n > r->gb - off)
    return fail(SLIDE_E_ARG, "slot ring %s: bytes [%zu, +%zu) outside the %zu-byte gradient",
                what, off, n, r->gb);
  if (sl.state != SLIDE_SLOT_IN_USE && sl.state != SLIDE_SLOT_FLUSHING)
    return fail(SLIDE_E_STATE, "slot ring %s: slot %d is %s, expected IN_USE or FLUSHING",
                what, slot, state_name(sl.state));
  uint64_t t = r->next_ticket++;
  Ev& te = r->ticket_ev[t % kTicketPool];
  char* dst = (char*)host_g + off;
  const char* src = r->g_ptr(slot) + off;
  if (r->engine == SLIDE_ENGINE_HOST) {
    HostCopyQueue::Job j;
    j.dst = dst;
    j.src = src;
    j.n = n;
    j.done = std::make_shared<HostEvent>();
    j.done->st.store(0);
    j.fault = r->take_fault();
    te.host = j.done;
    te.valid = true;
    r->hq_d2h->push(std::move(j));
  } else if (r->engine == SLIDE_ENGINE_HSA) {
    Ev cdone;
    if ((rc = r->record_compute(cdone, compute_stream))) return rc;
    HsaCopyQueue::Job j;
    j.gpu_wait = cdone.hip;
    j.own_gpu_wait = true;
    j.dst = dst;
    j.src = src;
    j.n = n;
    j.to_device = false;
    j.done = std::make_shared<HostEvent>();
    j.done->st.store(0);
    te.host = j.done;
    te.valid = true;
    r->sq_d2h->push(std::move(j));
  } else {
    Ev cdone;
    if ((rc = r->record_compute(cdone, compute_stream))) return rc;
    hipError_t e = hipStreamWaitEvent(r->d2h, cdone.hip, 0);
    if (e == hipSuccess) e = hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToHost, r->d2h);
    if (e == hipSuccess && !te.hip)
      e = hipEventCreateWithFlags(&te.hip, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(te.hip, r->d2h);
    hipEventDestroy(cdone.hip);  // destruction is deferred by HIP until the event completes
    if (e != hipSuccess) return fail(SLIDE_E_HIP, "slot ring %s: %s", what, hipGetErrorString(e));
    te.valid = true;
  }
  r->ticket_id[t % kTicketPool] = t;
  sl.flush_ev = te;
  sl.state = SLIDE_SLOT_FLUSHING;
  *ticket = t;
  return SLIDE_OK;
}
}  // namespace

extern "C" int slide_slot_ring_flush(slide_ring* r, int slot, void* host_g, void* compute_stream,
                                     uint64_t* ticket) {
  if (r && slot >= 0 && slot < r->n) {
    std::lock_guard<std::mutex> lk(r->mu);
    if (r->slots[slot].state != SLIDE_SLOT_IN_USE)
      return fail(SLIDE_E_STATE, "slot ring flush: slot %d is %s, expected IN_USE", slot,
                  state_name(r->slots[slot].state));
  }
  return flush_part(r, slot, host_g, 0, r ? r->gb : 0, compute_stream, ticket, "flush");
}

extern "C" int slide_slot_ring_flush_range(slide_ring* r, int slot, void* host_g, size_t offset,
                                           size_t nbytes, void* compute_stream,
                                           uint64_t* ticket) {
  return flush_part(r, slot, host_g, offset, nbytes, compute_stream, ticket, "flush_range");
}

extern "C" int slide_slot_ring_wait_flush(slide_ring* r, uint64_t ticket, int timeout_ms) {
  if (!r) return fail(SLIDE_E_ARG, "slot ring wait_flush: null handle");
  Ev e;
  {
    std::lock_guard<std::mutex> lk(r->mu);
    if (ticket == 0 || ticket >= r->next_ticket)
      return fail(SLIDE_E_ARG, "slot ring wait_flush: unknown ticket %llu",
                  (unsigned long long)ticket);
    // If the pool entry was reused by a later flush, waiting on the later one is a safe
    // over-wait: copies on the d2h queue complete in order.
    e = r->ticket_ev[ticket % kTicketPool];
  }
  return r->host_wait(e, timeout_ms, "wait_flush");
}

extern "C" int slide_slot_ring_release(slide_ring* r, int slot, void* compute_stream) {
  int rc = check_ring(r, slot);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(r->mu);
  Slot& sl = r->slots[slot];
  if (sl.state != SLIDE_SLOT_IN_USE && sl.state != SLIDE_SLOT_FLUSHING)
    return fail(SLIDE_E_STATE, "slot ring release: slot %d is %s, expected IN_USE or FLUSHING",
                slot, state_name(sl.state));
  if ((rc = r->record_compute(sl.free_ev, compute_stream))) return rc;
  sl.state = SLIDE_SLOT_FREE;
  sl.released_at = r->clock++;
  return SLIDE_OK;
}

extern "C" int slide_slot_ring_state(slide_ring* r, int slot, int* state, int* layer) {
  int rc = check_ring(r, slot);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(r->mu);
  if (state) *state = r->slots[slot].state;
  if (layer) *layer = r->slots[slot].layer;
  return SLIDE_OK;
}

extern "C" int slide_slot_ring_find(slide_ring* r, int layer, int* slot_out) {
  if (!r || !slot_out) return fail(SLIDE_E_ARG, "slot ring find: null pointer");
  std::lock_guard<std::mutex> lk(r->mu);
  *slot_out = -1;
  for (int s = 0; s < r->n; ++s)
    if (r->slots[s].state != SLIDE_SLOT_FREE && r->slots[s].layer == layer) *slot_out = s;
  return SLIDE_OK;
}

extern "C" int slide_slot_ring_inject_fault(slide_ring* r, int fail_mode, int count) {
  if (!r) return fail(SLIDE_E_ARG, "slot ring inject_fault: null handle");
  if (r->engine != SLIDE_ENGINE_HOST)
    return fail(SLIDE_E_UNSUPPORTED, "slot ring inject_fault: host engine only");
  if (fail_mode < 0 || fail_mode > 2 || count < 0)
    return fail(SLIDE_E_ARG, "slot ring inject_fault: bad mode %d / count %d", fail_mode, count);
  std::lock_guard<std::mutex> lk(r->mu);
  r->fault_mode = fail_mode;
  r->fault_count = count;
  return SLIDE_OK;
}

extern "C" int slide_slot_ring_ticket_time(slide_ring* r, uint64_t ticket, double* t_done) {
  if (!r || !t_done) return fail(SLIDE_E_ARG, "slot ring ticket_time: null pointer");
  if (r->engine == SLIDE_ENGINE_HIP)
    return fail(SLIDE_E_UNSUPPORTED, "slot ring ticket_time: host-timed engines only");
  std::lock_guard<std::mutex> lk(r->mu);
  if (ticket == 0 || ticket >= r->next_ticket || r->ticket_id[ticket % kTicketPool] != ticket)
    return fail(SLIDE_E_ARG, "slot ring ticket_time: unknown or recycled ticket %llu",
                (unsigned long long)ticket);
  const Ev& e = r->ticket_ev[ticket % kTicketPool];
  if (!e.host || e.host->st.load() != 1)
    return fail(SLIDE_E_STATE, "slot ring ticket_time: ticket %llu has not landed",
                (unsigned long long)ticket);
  *t_done = e.host->t_done;
  return SLIDE_OK;
}

extern "C" int slide_slot_ring_destroy(slide_ring* r) {
  if (!r) return fail(SLIDE_E_ARG, "slot ring destroy: null handle");
  if (r->engine == SLIDE_ENGINE_HSA) {
    // the copy threads finish their queued copies (each bounded) and exit
    r->sq_h2d.reset();
    r->sq_d2h.reset();
    for (auto& s : r->slots)
      if (s.free_ev.hip) hipEventDestroy(s.free_ev.hip);
    if (r->hsa_up) hsa_shut_down();
    delete r;
    return SLIDE_OK;
  }
  if (r->engine == SLIDE_ENGINE_HIP) {
    auto drop = [](Ev& e) {
      if (e.hip) hipEventDestroy(e.hip);
      e.hip = nullptr;
    };
    for (auto& s : r->slots) {
      drop(s.load_ev);
      drop(s.free_ev);
    }
    for (auto& e : r->ticket_ev) drop(e);
  } else {
    // copies that can never complete (injected faults) would stall the copy threads forever;
    // mark every pending event failed so the threads can drain and exit
    for (auto& s : r->slots) {
      for (Ev* e : {&s.load_ev, &s.free_ev, &s.flush_ev})
        if (e->host && e->host->st.load() == 0) e->host->st.store(2);
    }
    for (auto& e : r->ticket_ev)
      if (e.host && e.host->st.load() == 0) e.host->st.store(2);
  }
  delete r;
  return SLIDE_OK;
}
