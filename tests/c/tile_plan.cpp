// Host check of the tile plans of the streaming kernels (zs_launch.hpp): for
// every (ngroups, span, slots) of a sweep, plain_tiles and balanced_tiles must
// cover the groups [0, ngroups) exactly once, in order, with no empty tile and
// none longer than `span`; balanced_tiles must run every round but the last
// with full tiles, start every tile of the last round on a 64-group unit, give
// those tiles sizes within one unit of each other, and use no more of them than
// there are slots. Prints "ok <cases>" or the first failure; exits 1 on failure.
#include <cstdio>
#include <vector>

#include "zs_launch.hpp"

using zs::TilePlan;

static long long cases = 0;

static bool fail(const char* what, long long ng, long long span, long long slots, long long t) {
  std::printf("FAIL %s: ngroups=%lld span=%lld slots=%lld tile=%lld\n", what, ng, span, slots, t);
  return false;
}

static bool check(const TilePlan& p, long long ng, long long span, long long slots, bool balanced) {
  ++cases;
  if (ng == 0) return p.count() == 0 ? true : fail("tiles for no groups", ng, span, slots, -1);
  long long next = 0, lo = -1, hi = -1;
  for (long long t = 0; t < p.count(); ++t) {
    int64_t b, e;
    p.range(t, ng, &b, &e);
    if (b != next) return fail("gap or overlap", ng, span, slots, t);
    if (e <= b) return fail("empty tile", ng, span, slots, t);
    if (e - b > span) return fail("tile longer than span", ng, span, slots, t);
    if (t < p.nfull && e != ng && e - b != span) return fail("short full tile", ng, span, slots, t);
    if (t >= p.nfull) {
      if ((b - p.nfull * span) % 64 != 0) return fail("split tile off its unit", ng, span, slots, t);
      const long long units = (e - b + 63) / 64;
      if (e == ng) {  // the last tile may end inside its last unit
        if (lo < 0 || units < lo) lo = units;
        if (hi < 0 || units > hi) hi = units;
      } else {
        if ((e - b) % 64 != 0) return fail("split tile not whole units", ng, span, slots, t);
        if (lo < 0 || units < lo) lo = units;
        if (hi < 0 || units > hi) hi = units;
      }
    }
    next = e;
  }
  if (next != ng) return fail("groups left uncovered", ng, span, slots, -1);
  if (!balanced) return p.nlast == 0 ? true : fail("plain plan with split tiles", ng, span, slots, -1);
  if (p.nlast > slots) return fail("more split tiles than slots", ng, span, slots, -1);
  if (p.nfull % slots != 0) return fail("full tiles not whole rounds", ng, span, slots, -1);
  if (hi - lo > 1) return fail("split tiles differ by more than a unit", ng, span, slots, -1);
  // the last round is not empty and no bigger than a round
  const long long rest = ng - p.nfull * span;
  if (rest <= 0 || rest > slots * span) return fail("last round size", ng, span, slots, -1);
  return true;
}

int main() {
  const long long spans[] = {64, 128, 1024, 4096, 8192};
  const long long slots_list[] = {1, 3, 8, 255, 256, 512};
  std::vector<long long> sizes;
  for (long long n = 0; n <= 700; ++n) sizes.push_back(n);
  for (long long base : {8192LL * 256, 8192LL * 256 * 13, 4096LL * 512 * 3})
    for (long long d = -130; d <= 130; ++d) sizes.push_back(base + d);
  for (long long n = 1000; n < 40000000; n = n * 7 / 5 + 13) sizes.push_back(n);
  sizes.push_back(34450112);   // 137,800,448 elements in groups of 4
  sizes.push_back(29296875);   // 117,187,500 elements
  sizes.push_back(1LL << 40);  // far beyond any device, still exact
  for (long long span : spans)
    for (long long slots : slots_list)
      for (long long ng : sizes) {
        if (ng > (1LL << 32) && !(span == 8192 && slots == 256)) continue;  // keep the run short
        if (!check(zs::plain_tiles(ng, span), ng, span, slots, false)) return 1;
        if (!check(zs::balanced_tiles(ng, span, slots), ng, span, slots, true)) return 1;
      }
  // no residency information: the plain plan
  const TilePlan p = zs::balanced_tiles(100000, 8192, 0);
  if (p.nlast != 0 || p.count() != (100000 + 8191) / 8192) {
    std::printf("FAIL slots=0 does not give the plain plan\n");
    return 1;
  }
  std::printf("ok %lld\n", cases);
  return 0;
}
