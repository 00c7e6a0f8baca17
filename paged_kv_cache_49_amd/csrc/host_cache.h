// Thread-safe host-side caches of the launch code: values read once from
// the HIP runtime per device (CU count, LDS per workgroup, occupancy) and
// the one-way raise of a kernel's dynamic-LDS limit. Several host threads
// may launch at once (the device entry points are documented thread-safe),
// so every shared value is an atomic, and raising a limit is serialised so
// that the attribute the runtime holds is never below the recorded one.
// Plain C++ (no HIP types), so a CPU build can test it under ThreadSanitizer.
#pragma once

#include <atomic>
#include <mutex>

namespace pa {

constexpr int kMaxDevices = 64;

// One positive int per device, filled on first use; 0 = not known yet.
// Racing first users each run `query` and store the same value.
class DeviceIntCache {
 public:
  // query() -> int; a value <= 0 (failure) is returned but not kept
  template <typename Query>
  int get(int dev, Query&& query) {
    if (dev < 0 || dev >= kMaxDevices) return query();
    const int v = value_[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    const int q = query();
    if (q > 0) value_[dev].store(q, std::memory_order_relaxed);
    return q;
  }

 private:
  std::atomic<int> value_[kMaxDevices] = {};
};

// A small table of positive ints keyed by (a, b), a < NA, b < NB, filled on
// first use (the occupancy of one kernel build per (heads, LDS size)).
template <int NA, int NB>
class IntTable {
 public:
  template <typename Query>
  int get(int a, int b, Query&& query) {
    if (a < 0 || a >= NA || b < 0 || b >= NB) return query();
    const int v = value_[a][b].load(std::memory_order_relaxed);
    if (v > 0) return v;
    const int q = query();
    if (q > 0) value_[a][b].store(q, std::memory_order_relaxed);
    return q;
  }

 private:
  std::atomic<int> value_[NA][NB] = {};
};

// The dynamic-LDS bytes one kernel may use on each device. ensure(dev,
// bytes, set) calls set(bytes) (which raises the runtime attribute and
// returns true on success) only when `bytes` exceeds what was granted
// before, one caller at a time, so the attribute only grows and always
// covers the recorded grant.
class LdsGrant {
 public:
  explicit constexpr LdsGrant(int initial) : initial_(initial) {}

  template <typename Set>
  bool ensure(int dev, int bytes, Set&& set) {
    if (bytes <= initial_) return true;
    if (dev < 0 || dev >= kMaxDevices) return set(bytes);
    if (bytes <= granted_[dev].load(std::memory_order_acquire)) return true;
    std::lock_guard<std::mutex> lock(mu_);
    if (bytes <= granted_[dev].load(std::memory_order_relaxed)) return true;
    if (!set(bytes)) return false;
    granted_[dev].store(bytes, std::memory_order_release);
    return true;
  }

 private:
  const int initial_;
  std::mutex mu_;
  std::atomic<int> granted_[kMaxDevices] = {};
};

}  // namespace pa
