// Multi-threaded exercise of the library's host code, built with g++ under
// ThreadSanitizer by tests/test_sanitizers.py (CPU only):
//  * the launch code's caches (host_cache.h): per-device ints, the
//    occupancy table and the dynamic-LDS grant, hammered from 16 threads
//    with stand-in queries; the grant's attribute must never shrink and
//    must always cover what a caller was granted;
//  * independent block managers driven from 8 threads at once (the
//    manager itself is documented single-threaded per handle), with the
//    thread-local last-error strings checked per thread.
// Exit status 0 when every check holds; TSan reports make it nonzero.
// `--planted-race` runs an unsynchronised counter instead, so the test can
// show that TSan is active.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "host_cache.h"
#include "libpagedattn.h"

namespace {

int planted_race() {
  int counter = 0;
  std::thread a([&] {
    for (int i = 0; i < 100000; ++i) ++counter;
  });
  std::thread b([&] {
    for (int i = 0; i < 100000; ++i) ++counter;
  });
  a.join();
  b.join();
  std::printf("counter %d\n", counter);
  return 0;
}

int caches() {
  constexpr int kDev = 4;
  pa::DeviceIntCache cus;
  pa::IntTable<9, 41> occupancy;
  pa::LdsGrant grant(64 * 1024);
  std::atomic<int> attr[kDev] = {};  // stand-in for the runtime's per-device attribute
  std::atomic<int> bad{0};
  std::vector<std::thread> threads;
  for (int t = 0; t < 16; ++t) {
    threads.emplace_back([&, t] {
      std::mt19937 rng(1234 + t);
      for (int i = 0; i < 20000; ++i) {
        const int dev = static_cast<int>(rng() % kDev);
        if (cus.get(dev, [dev] { return 256 - dev; }) != 256 - dev) ++bad;
        const int a = static_cast<int>(rng() % 9), b = static_cast<int>(rng() % 41);
        if (occupancy.get(a, b, [a, b] { return 1 + (a * 41 + b) % 3; }) != 1 + (a * 41 + b) % 3) ++bad;
        const int want = 60 * 1024 + static_cast<int>(rng() % 26) * 4096;
        const bool ok = grant.ensure(dev, want, [&](int bytes) {
          if (bytes < attr[dev].load()) ++bad;  // a raise never lowers the attribute
          attr[dev].store(bytes);
          return true;
        });
        if (!ok || (want > 64 * 1024 && attr[dev].load() < want)) ++bad;
      }
    });
  }
  for (auto& th : threads) th.join();
  std::printf("caches: %d bad\n", bad.load());
  return bad.load();
}

int managers() {
  std::atomic<int> bad{0};
  std::vector<std::thread> threads;
  for (int t = 0; t < 8; ++t) {
    threads.emplace_back([&, t] {
      pa_bm* bm = nullptr;
      if (pa_bm_create(64, 16, nullptr, &bm) != PA_OK) {
        ++bad;
        return;
      }
      std::mt19937 rng(99 + t);
      std::vector<int64_t> slots(512);
      for (int i = 0; i < 3000; ++i) {
        const int64_t seq = static_cast<int64_t>(rng() % 6);
        int32_t src = 0, dst = 0, ncow = 0;
        switch (rng() % 4) {
          case 0:
          case 1:
            pa_alloc(bm, seq, static_cast<int32_t>(rng() % 40), slots.data(), &src, &dst, &ncow);
            break;
          case 2: pa_free(bm, seq); break;
          default: pa_fork(bm, seq, static_cast<int64_t>(rng() % 6)); break;
        }
        // an error names this thread's own request
        const int64_t missing = 1000 + t;
        if (pa_free(bm, missing) != PA_ERR_UNKNOWN_SEQ) ++bad;
        char want[32];
        std::snprintf(want, sizeof(want), "%lld", static_cast<long long>(missing));
        if (std::strstr(pa_last_error(), want) == nullptr) ++bad;
        pa_bm_stats_t st{};
        if (pa_bm_stats(bm, &st) != PA_OK || st.num_free + st.num_used != st.num_blocks) ++bad;
      }
      pa_bm_destroy(bm);
    });
  }
  for (auto& th : threads) th.join();
  std::printf("managers: %d bad\n", bad.load());
  return bad.load();
}

}  // namespace

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--planted-race") == 0) return planted_race();
  const int bad = caches() + managers();
  return bad == 0 ? 0 : 1;
}
