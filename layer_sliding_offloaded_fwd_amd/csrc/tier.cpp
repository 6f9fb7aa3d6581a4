// Disk tier of the CPU optimizer's state. The method keeps the optimizer state of its per-layer
// CPU optimizer in host memory and can move it to NVMe (SlideFormer summary, section 2B,
// "Layer-Adam"); for models larger than host memory the optimizer state is the first thing to
// go to NVMe (summary, section 3; the paper page's "Analysis of NVMe Offloading").
//
// A tier is one file holding fp32 arrays (master weights, first and second moments) at
// caller-chosen offsets that are multiples of 4096 bytes. All file traffic goes through the
// tier's own page-aligned bounce buffers and is opened with O_DIRECT where the file system
// allows it, so the bytes really travel to the device instead of stopping in the page cache;
// where it does not (tmpfs, some overlays) the file is opened buffered and the tier says so.
// Transfers are split into 1 MiB requests served by a pool of I/O threads, which keeps several
// requests in flight at the device.
//
// slide_tier_adamw streams one parameter block through the CPU AdamW in chunks with three
// bounce sets: while chunk k is updated in memory, chunk k+1's state is being read and chunk
// k-1's written back. The update of each element is slide_cpu_adamw's, so the results are the
// same bits as with the state in host memory.
#include <errno.h>
#include <fcntl.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/slide.h"

namespace slide {
int fail(int code, const char* fmt, ...);
}
using slide::fail;

namespace {

constexpr size_t kPage = 4096;
constexpr size_t kReq = size_t(1) << 20;            // bytes per I/O request
constexpr size_t kDefaultChunk = size_t(1) << 22;   // elements per chunk (16 MiB per array)

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

// A set of requests that is waited for as a whole.
struct Group {
  std::mutex mu;
  std::condition_variable cv;
  int pending = 0;
  int err = 0;
};

struct Req {
  bool write;
  char* buf;
  size_t len;
  uint64_t off;
  Group* grp;
};

}  // namespace

struct slide_tier {
  int fd = -1;
  bool direct = false;
  uint64_t capacity = 0;
  size_t chunk = 0;                  // elements per chunk (multiple of 1024)
  char* bounce = nullptr;            // 3 sets x 3 arrays x chunk floats, page aligned
  std::vector<std::thread> io;
  std::mutex qmu;
  std::condition_variable qcv;
  std::deque<Req> q;
  bool stop = false;
  Group rd[3], wr[3];
  std::mutex call_mu;                // one transfer or update at a time (shared bounce sets)
  uint64_t bytes_read = 0, bytes_written = 0;
  double busy_s = 0, stall_s = 0;

  float* set_array(int set, int a) {
    return (float*)(bounce + ((size_t)set * 3 + a) * chunk * sizeof(float));
  }
  char* set_base(int set) { return bounce + (size_t)set * 3 * chunk * sizeof(float); }
  size_t set_bytes() const { return 3 * chunk * sizeof(float); }
};

namespace {

void io_loop(slide_tier* t) {
  for (;;) {
    Req r;
    {
      std::unique_lock<std::mutex> lk(t->qmu);
      t->qcv.wait(lk, [&] { return t->stop || !t->q.empty(); });
      if (t->q.empty()) return;
      r = t->q.front();
      t->q.pop_front();
    }
    int err = 0;
    size_t done = 0;
    while (done < r.len) {
      ssize_t n = r.write ? pwrite(t->fd, r.buf + done, r.len - done, (off_t)(r.off + done))
                          : pread(t->fd, r.buf + done, r.len - done, (off_t)(r.off + done));
      if (n < 0) {
        if (errno == EINTR) continue;
        err = errno;
        break;
      }
      if (n == 0) {
        if (r.write) {
          err = EIO;
        } else {  // past the end of the file: the file reads as zeros there
          memset(r.buf + done, 0, r.len - done);
          done = r.len;
        }
        break;
      }
      done += (size_t)n;
    }
    std::lock_guard<std::mutex> lk(r.grp->mu);
    if (err && !r.grp->err) r.grp->err = err;
    if (--r.grp->pending == 0) r.grp->cv.notify_all();
  }
}

// Queue a transfer of len bytes (a multiple of the page size) as 1 MiB requests.
void submit(slide_tier* t, Group* g, bool write, char* buf, size_t len, uint64_t off) {
  size_t nreq = (len + kReq - 1) / kReq;
  if (nreq == 0) return;
  {
    std::lock_guard<std::mutex> lk(g->mu);
    g->pending += (int)nreq;
  }
  {
    std::lock_guard<std::mutex> lk(t->qmu);
    for (size_t i = 0; i < nreq; ++i) {
      size_t o = i * kReq;
      t->q.push_back(Req{write, buf + o, std::min(kReq, len - o), off + o, g});
    }
  }
  t->qcv.notify_all();
}

// Wait for every request of the group; returns the first errno seen (0 if none) and clears it.
int wait_group(slide_tier* t, Group* g) {
  double t0 = now_s();
  std::unique_lock<std::mutex> lk(g->mu);
  g->cv.wait(lk, [&] { return g->pending == 0; });
  t->stall_s += now_s() - t0;
  int e = g->err;
  g->err = 0;
  return e;
}

int check_range(slide_tier* t, uint64_t off, size_t bytes, const char* what) {
  if (off % kPage)
    return fail(SLIDE_E_ARG, "%s: offset %llu is not a multiple of %zu", what,
                (unsigned long long)off, kPage);
  if (off > t->capacity || round_up(bytes, kPage) > t->capacity - off)
    return fail(SLIDE_E_ARG, "%s: [%llu, +%zu) reaches past the tier's %llu bytes", what,
                (unsigned long long)off, round_up(bytes, kPage),
                (unsigned long long)t->capacity);
  return SLIDE_OK;
}

}  // namespace

extern "C" size_t slide_tier_region_bytes(size_t n_floats) {
  return round_up(n_floats * sizeof(float), kPage);
}

extern "C" int slide_tier_create(slide_tier** out, const char* path, uint64_t capacity_bytes,
                                 size_t chunk_elems, int n_io_threads, int flags) {
  if (!out || !path) return fail(SLIDE_E_ARG, "slide_tier_create: null argument");
  *out = nullptr;
  if (flags & ~(SLIDE_TIER_DIRECT | SLIDE_TIER_UNLINK))
    return fail(SLIDE_E_ARG, "slide_tier_create: unknown flags 0x%x", flags);
  if (capacity_bytes % kPage)
    return fail(SLIDE_E_ARG, "slide_tier_create: capacity must be a multiple of %zu", kPage);
  size_t chunk = chunk_elems ? round_up(chunk_elems, kPage / sizeof(float)) : kDefaultChunk;
  int nio = n_io_threads > 0 ? std::min(n_io_threads, 64) : 8;
  int fd = -1;
  bool direct = false;
  if (flags & SLIDE_TIER_DIRECT) {
    fd = open(path, O_RDWR | O_CREAT | O_TRUNC | O_DIRECT, 0600);
    direct = fd >= 0;
    if (fd < 0 && errno != EINVAL)
      return fail(SLIDE_E_IO, "slide_tier_create: open(%s): %s", path, strerror(errno));
  }
  if (fd < 0) {
    fd = open(path, O_RDWR | O_CREAT | O_TRUNC, 0600);
    if (fd < 0) return fail(SLIDE_E_IO, "slide_tier_create: open(%s): %s", path, strerror(errno));
  }
  if (ftruncate(fd, (off_t)capacity_bytes) != 0) {
    int e = errno;
    close(fd);
    if (flags & SLIDE_TIER_UNLINK) unlink(path);
    return fail(SLIDE_E_IO, "slide_tier_create: ftruncate(%s, %llu): %s", path,
                (unsigned long long)capacity_bytes, strerror(e));
  }
  if (flags & SLIDE_TIER_UNLINK) unlink(path);  // the space is freed when the tier closes
  auto* t = new slide_tier;
  t->fd = fd;
  t->direct = direct;
  t->capacity = capacity_bytes;
  t->chunk = chunk;
  void* mem = nullptr;
  if (posix_memalign(&mem, kPage, 3 * t->set_bytes()) != 0) {
    close(fd);
    delete t;
    return fail(SLIDE_E_ARG, "slide_tier_create: cannot allocate %zu bytes of bounce buffers",
                3 * 3 * chunk * sizeof(float));
  }
  memset(mem, 0, 3 * t->set_bytes());
  t->bounce = (char*)mem;
  for (int i = 0; i < nio; ++i) t->io.emplace_back(io_loop, t);
  *out = t;
  return SLIDE_OK;
}

extern "C" int slide_tier_destroy(slide_tier* t) {
  if (!t) return SLIDE_OK;
  {
    std::lock_guard<std::mutex> lk(t->qmu);
    t->stop = true;
  }
  t->qcv.notify_all();
  for (auto& th : t->io) th.join();
  if (t->fd >= 0) close(t->fd);
  free(t->bounce);
  delete t;
  return SLIDE_OK;
}

extern "C" int slide_tier_info(slide_tier* t, int* direct, uint64_t* capacity_bytes,
                               size_t* chunk_elems) {
  if (!t) return fail(SLIDE_E_ARG, "slide_tier_info: null tier");
  if (direct) *direct = t->direct ? 1 : 0;
  if (capacity_bytes) *capacity_bytes = t->capacity;
  if (chunk_elems) *chunk_elems = t->chunk;
  return SLIDE_OK;
}

extern "C" int slide_tier_stats(slide_tier* t, uint64_t* bytes_read, uint64_t* bytes_written,
                                double* busy_s, double* stall_s) {
  if (!t) return fail(SLIDE_E_ARG, "slide_tier_stats: null tier");
  std::lock_guard<std::mutex> lk(t->call_mu);
  if (bytes_read) *bytes_read = t->bytes_read;
  if (bytes_written) *bytes_written = t->bytes_written;
  if (busy_s) *busy_s = t->busy_s;
  if (stall_s) *stall_s = t->stall_s;
  return SLIDE_OK;
}

// Copy host bytes into the tier (src == nullptr writes zeros). Whole pages are written: the
// bytes from off + bytes up to the next page boundary become zero.
extern "C" int slide_tier_write(slide_tier* t, uint64_t off, const void* src, size_t bytes) {
  if (!t) return fail(SLIDE_E_ARG, "slide_tier_write: null tier");
  int rc = check_range(t, off, bytes, "slide_tier_write");
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(t->call_mu);
  double t0 = now_s();
  const size_t piece = t->set_bytes();
  int err = 0;
  size_t k = 0;
  for (size_t done = 0; done < bytes; done += piece, ++k) {
    int s = (int)(k % 2);
    err = err ? err : wait_group(t, &t->wr[s]);   // the set's previous piece has been written
    if (err) break;
    size_t len = std::min(piece, bytes - done);
    char* b = t->set_base(s);
    if (src)
      memcpy(b, (const char*)src + done, len);
    else
      memset(b, 0, len);
    size_t plen = round_up(len, kPage);
    memset(b + len, 0, plen - len);
    submit(t, &t->wr[s], true, b, plen, off + done);
    t->bytes_written += plen;
  }
  for (int s = 0; s < 2; ++s) {
    int e = wait_group(t, &t->wr[s]);
    err = err ? err : e;
  }
  t->busy_s += now_s() - t0;
  if (err) return fail(SLIDE_E_IO, "slide_tier_write: %s", strerror(err));
  return SLIDE_OK;
}

// Copy bytes of the tier into host memory.
extern "C" int slide_tier_read(slide_tier* t, uint64_t off, void* dst, size_t bytes) {
  if (!t || (!dst && bytes)) return fail(SLIDE_E_ARG, "slide_tier_read: null argument");
  int rc = check_range(t, off, bytes, "slide_tier_read");
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(t->call_mu);
  double t0 = now_s();
  const size_t piece = t->set_bytes();
  const size_t npieces = (bytes + piece - 1) / piece;
  auto issue = [&](size_t k) {
    size_t len = std::min(piece, bytes - k * piece);
    submit(t, &t->rd[k % 2], false, t->set_base((int)(k % 2)), round_up(len, kPage),
           off + k * piece);
    t->bytes_read += round_up(len, kPage);
  };
  int err = 0;
  if (npieces) issue(0);
  for (size_t k = 0; k < npieces; ++k) {
    if (k + 1 < npieces && !err) issue(k + 1);
    int e = wait_group(t, &t->rd[k % 2]);
    err = err ? err : e;
    if (!err) {
      size_t len = std::min(piece, bytes - k * piece);
      memcpy((char*)dst + k * piece, t->set_base((int)(k % 2)), len);
    }
  }
  for (int s = 0; s < 2; ++s) {
    int e = wait_group(t, &t->rd[s]);
    err = err ? err : e;
  }
  t->busy_s += now_s() - t0;
  if (err) return fail(SLIDE_E_IO, "slide_tier_read: %s", strerror(err));
  return SLIDE_OK;
}

extern "C" int slide_tier_adamw(slide_tier* t, float* p, uint64_t p_off, float* m,
                                uint64_t m_off, float* v, uint64_t v_off, const void* g,
                                int g_dtype, uint16_t* p_bf16_out, size_t n, int64_t step,
                                const slide_adamw_hp* hp, int n_threads) {
  if (!t || !g || !hp) return fail(SLIDE_E_ARG, "slide_tier_adamw: null argument");
  if (g_dtype != SLIDE_BF16 && g_dtype != SLIDE_F32)
    return fail(SLIDE_E_ARG, "slide_tier_adamw: g_dtype must be SLIDE_BF16 or SLIDE_F32");
  if (step < 1) return fail(SLIDE_E_ARG, "slide_tier_adamw: step must be >= 1");
  if (n == 0) return SLIDE_OK;
  float* host[3] = {p, m, v};
  const uint64_t off[3] = {p_off, m_off, v_off};
  const size_t region = slide_tier_region_bytes(n);
  for (int a = 0; a < 3; ++a) {
    if (host[a]) continue;
    int rc = check_range(t, off[a], region, "slide_tier_adamw");
    if (rc) return rc;
    for (int b = 0; b < a; ++b)
      if (!host[b] && off[b] < off[a] + region && off[a] < off[b] + region)
        return fail(SLIDE_E_ARG, "slide_tier_adamw: the tier regions of p, m and v overlap");
  }
  std::lock_guard<std::mutex> lk(t->call_mu);
  double t0 = now_s();
  const size_t C = t->chunk;
  const size_t nch = (n + C - 1) / C;
  const size_t gsz = g_dtype == SLIDE_BF16 ? 2 : 4;
  auto len_of = [&](size_t k) { return std::min(C, n - k * C); };
  auto issue_read = [&](size_t k) {
    int s = (int)(k % 3);
    size_t bytes = round_up(len_of(k) * sizeof(float), kPage);
    for (int a = 0; a < 3; ++a) {
      if (host[a]) continue;
      submit(t, &t->rd[s], false, (char*)t->set_array(s, a), bytes,
             off[a] + k * C * sizeof(float));
      t->bytes_read += bytes;
    }
  };
  int err = 0, rc = SLIDE_OK;
  issue_read(0);
  for (size_t k = 0; k < nch; ++k) {
    const int s = (int)(k % 3);
    if (k + 1 < nch) {
      // chunk k+1 uses the set of chunk k-2, whose write-back must have finished
      int e = wait_group(t, &t->wr[(k + 1) % 3]);
      err = err ? err : e;
      if (!err) issue_read(k + 1);
    }
    int e = wait_group(t, &t->rd[s]);
    err = err ? err : e;
    if (err) break;
    const size_t len = len_of(k);
    float* arr[3];
    for (int a = 0; a < 3; ++a) arr[a] = host[a] ? host[a] + k * C : t->set_array(s, a);
    rc = slide_cpu_adamw(arr[0], (const char*)g + k * C * gsz, g_dtype, arr[1], arr[2],
                         p_bf16_out ? p_bf16_out + k * C : nullptr, len, step, hp, n_threads);
    if (rc != SLIDE_OK) break;
    const size_t bytes = round_up(len * sizeof(float), kPage);
    for (int a = 0; a < 3; ++a) {
      if (host[a]) continue;
      submit(t, &t->wr[s], true, (char*)arr[a], bytes, off[a] + k * C * sizeof(float));
      t->bytes_written += bytes;
    }
  }
  for (int s = 0; s < 3; ++s) {  // drain everything still in flight, also after an error
    int e1 = wait_group(t, &t->rd[s]);
    int e2 = wait_group(t, &t->wr[s]);
    err = err ? err : (e1 ? e1 : e2);
  }
  t->busy_s += now_s() - t0;
  if (rc != SLIDE_OK) return rc;  // slide_cpu_adamw's own message stands
  if (err) return fail(SLIDE_E_IO, "slide_tier_adamw: %s", strerror(err));
  return SLIDE_OK;
}
