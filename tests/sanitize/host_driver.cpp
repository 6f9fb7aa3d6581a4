// Host-side driver of the CPU optimizer and the disk tier for sanitizer builds (AddressSanitizer
// + UndefinedBehaviorSanitizer, or ThreadSanitizer): multi-threaded AdamW calls, tier writes and
// reads across chunk and page boundaries, a streamed tier update checked element by element
// against the in-memory update, and the tier's argument errors. Exit status 0 means every
// check held; the sanitizers report any memory error or data race on stderr and fail the run.
#include <stdio.h>
#include <stdarg.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <vector>

#include "../../include/slide.h"

namespace slide {
// the library's error reporter, reduced to a message on stderr
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfprintf(stderr, fmt, ap);
  va_end(ap);
  fputc('\n', stderr);
  return code;
}
}  // namespace slide

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                   \
    }                                                             \
  } while (0)

static float frand(unsigned& s) {
  s = s * 1664525u + 1013904223u;
  return ((s >> 8) & 0xffff) / 65536.0f - 0.5f;
}

int main(int argc, char** argv) {
  const char* dir = argc > 1 ? argv[1] : "/tmp";
  const size_t n = 3 * 4096 + 777;           // three chunks of 4096 plus a ragged one
  unsigned seed = 7;
  std::vector<float> p(n), m(n, 0.f), v(n, 0.f), g(n);
  for (size_t i = 0; i < n; ++i) {
    p[i] = frand(seed);
    g[i] = frand(seed) * 1e-2f;
  }
  std::vector<float> p2 = p, m2 = m, v2 = v;
  slide_adamw_hp hp = {1e-3, 0.9, 0.999, 1e-8, 0.01};
  std::vector<uint16_t> out(n), out2(n);

  char path[512];
  snprintf(path, sizeof path, "%s/slide-sanitize-%d.bin", dir, (int)getpid());
  slide_tier* t = nullptr;
  const size_t reg = slide_tier_region_bytes(n);
  CHECK(slide_tier_create(&t, path, 4 * reg, 4096, 4, SLIDE_TIER_DIRECT | SLIDE_TIER_UNLINK) ==
        SLIDE_OK);
  CHECK(slide_tier_write(t, 0, p2.data(), n * 4) == SLIDE_OK);
  CHECK(slide_tier_write(t, reg, nullptr, n * 4) == SLIDE_OK);
  CHECK(slide_tier_write(t, 2 * reg, nullptr, n * 4) == SLIDE_OK);
  for (int step = 1; step <= 3; ++step) {
    CHECK(slide_cpu_adamw(p.data(), g.data(), SLIDE_F32, m.data(), v.data(), out.data(), n, step,
                          &hp, 5) == SLIDE_OK);
    CHECK(slide_tier_adamw(t, nullptr, 0, nullptr, reg, nullptr, 2 * reg, g.data(), SLIDE_F32,
                           out2.data(), n, step, &hp, 3) == SLIDE_OK);
  }
  std::vector<float> back(n);
  CHECK(slide_tier_read(t, 0, back.data(), n * 4) == SLIDE_OK);
  CHECK(memcmp(back.data(), p.data(), n * 4) == 0);
  CHECK(slide_tier_read(t, reg, back.data(), n * 4) == SLIDE_OK);
  CHECK(memcmp(back.data(), m.data(), n * 4) == 0);
  CHECK(slide_tier_read(t, 2 * reg, back.data(), n * 4) == SLIDE_OK);
  CHECK(memcmp(back.data(), v.data(), n * 4) == 0);
  CHECK(memcmp(out.data(), out2.data(), n * 2) == 0);
  // errors: unaligned offset, past the capacity, overlapping regions
  CHECK(slide_tier_write(t, 100, p.data(), 16) == SLIDE_E_ARG);
  CHECK(slide_tier_read(t, 4 * reg, back.data(), 4) == SLIDE_E_ARG);
  CHECK(slide_tier_adamw(t, nullptr, 0, nullptr, 4096, v.data(), 0, g.data(), SLIDE_F32, nullptr,
                         n, 1, &hp, 2) == SLIDE_E_ARG);
  uint64_t rd = 0, wr = 0;
  double busy = 0, stall = 0;
  CHECK(slide_tier_stats(t, &rd, &wr, &busy, &stall) == SLIDE_OK);
  CHECK(rd > 0 && wr > 0);
  CHECK(slide_tier_destroy(t) == SLIDE_OK);
  CHECK(access(path, F_OK) != 0);            // unlinked at creation
  printf("host driver: ok\n");
  return 0;
}
