// Launch-shape knobs of the streaming kernels, the sum-of-squares workspace
// bound and the per-device residency lookup. Host code only.
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "zs_launch.hpp"

namespace zs {

const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning x{0, 0, 0, 0, 0, 0, 0, 0, 0};
    // the overrides below are read only when ZS_TUNING=1 opts in, so that a
    // stray variable cannot change launch shapes unnoticed
    const char* on = std::getenv("ZS_TUNING");
    const bool use_env = on && on[0] == '1' && on[1] == '\0';
    auto env = [use_env](const char* name) -> const char* { return use_env ? std::getenv(name) : nullptr; };
    const char* e;
    x.adamw_v = (e = env("ZS_ADAMW_V")) ? std::atoi(e) : 1;
    if (x.adamw_v != 1 && x.adamw_v != 2 && x.adamw_v != 4) x.adamw_v = 1;
    // a 16 KiB reservation (10 one-wave workgroups per CU) measured best for AdamW
    x.adamw_lds = (e = env("ZS_ADAMW_LDS")) ? std::atoll(e) : 16384;
    if (x.adamw_lds < 0 || x.adamw_lds > 65536) x.adamw_lds = 16384;
    x.rank_chunk = (e = env("ZS_RANK_CHUNK")) ? std::atoi(e) : 8;
    if (x.rank_chunk != 4 && x.rank_chunk != 8) x.rank_chunk = 8;
    x.fused_g = (e = env("ZS_FUSED_G")) ? std::atoi(e) : 0;
    if (x.fused_g != 1 && x.fused_g != 2 && x.fused_g != 4 && x.fused_g != 8 && x.fused_g != 16) x.fused_g = 0;
    x.fused_lds = (e = env("ZS_FUSED_LDS")) ? std::atoll(e) : 0;
    if (x.fused_lds < 0 || x.fused_lds > 163840) x.fused_lds = 0;
    x.fused_bs = (e = env("ZS_FUSED_BS")) ? std::atoi(e) : 0;
    if (x.fused_bs != 64 && x.fused_bs != 256 && x.fused_bs != 512) x.fused_bs = 0;
    x.accum_shape = (e = env("ZS_ACCUM_SHAPE")) ? std::atoi(e) : 0;
    if (x.accum_shape != 1) x.accum_shape = 0;
    x.reduce_g = (e = env("ZS_REDUCE_G")) ? std::atoi(e) : 0;
    if (x.reduce_g != 1 && x.reduce_g != 4 && x.reduce_g != 16) x.reduce_g = 0;
    // an optional cap on workgroups per launch (grid-stride loops cover the
    // rest); launches also stay within the 32-bit work-item count of a dispatch
    x.grid_cap = (e = env("ZS_GRID_CAP")) ? std::atoll(e) : 0;
    if (x.grid_cap <= 0) x.grid_cap = INT64_MAX;
    return x;
  }();
  return t;
}

int64_t max_partials(int64_t n) {
  // every sum-of-squares launch uses at most one workgroup per 256 elements
  // (the smallest tile: one wave, one group per lane), up to a cap beyond
  // which launches grid-stride
  const int64_t b = (n + 255) / 256;
  const int64_t kMax = (int64_t(1) << 24) - 1;  // x 256 lanes stays a 32-bit dispatch
  return b < 1 ? 1 : (b > kMax ? kMax : b);
}

int64_t device_slots(hipStream_t s, const void* kernel, int bs, size_t lds) {
  struct Entry {
    const void* kernel;
    int dev;
    int bs;
    size_t lds;
    int64_t slots;
  };
  static std::mutex mu;
  static std::vector<Entry> known;
  int dev = 0;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : known)
    if (e.kernel == kernel && e.dev == dev && e.bs == bs && e.lds == lds) return e.slots;
  int cus = 0, per_cu = 0, cur = 0;
  int64_t slots = 0;
  // the occupancy query answers for the current device
  if (hipGetDevice(&cur) == hipSuccess && (cur == dev || hipSetDevice(dev) == hipSuccess)) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, bs, lds) == hipSuccess &&
        cus > 0 && per_cu > 0)
      slots = (int64_t)cus * per_cu;
    if (cur != dev) (void)hipSetDevice(cur);
  }
  // the entry points return before launching while an error is pending, so
  // an error left here is this lookup's own: clear it (the launch then uses
  // plain tiles)
  if (slots == 0) (void)hipGetLastError();
  known.push_back(Entry{kernel, dev, bs, lds, slots});
  return slots;
}

}  // namespace zs
