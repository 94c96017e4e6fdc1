// Mean of N per-rank gradient contributions for one rank's slice (the arithmetic
// of a reduce-scatter with reduce dtype fp32), with an optional deterministic
// sum of squares of the result.
//
// Pages: "Data parallelism and ZeRO memory sharding" s3.1 (the mean over ranks
// of the local gradients is the full-batch gradient); "Lesson 5: ZeRO and
// FSDP" s3 (ZeRO-1/2 step 1, each rank keeps its 1/N of the reduced gradient)
// and s7.5 (reduce_dtype float32); the same DP-and-ZeRO page, s6 (a global
// norm needs every shard's partial).
//
// Design (HBM-bound, 2N+4 bytes per element for bf16 contributions):
//   * each lane owns groups of 4 consecutive elements, lane-contiguous in
//     every stream (8-byte bf16 / 16-byte fp32 row loads, 16-byte g stores);
//   * with many contributions, a 4-wave workgroup parks 16 groups per lane in
//     LDS and writes them as one burst after the rank walk; with few, one-wave
//     workgroups store each group as soon as it is summed;
//   * row pointers sit in the kernel-argument segment (SGPR bases);
//   * ranks are walked in double-buffered chunks of C: a chunk's loads are in
//     flight while the previous chunk is added, and the fp32 sum still runs
//     in ascending rank order;
//   * one IEEE division by N (a multiply by the exact reciprocal when N is a
//     power of two), so the result is independent of the launch shape;
//   * rows are read with the nontemporal hint (each byte is used once).
#include <mutex>
#include <type_traits>

#include "zs_device.hpp"
#include "zs_launch.hpp"

namespace zs {

// Scratch of zs_reduce_grads_noalloc, for callers that cannot allocate: the
// first-level fp64 partials of the sum of squares (at most one per 256
// elements, so ZS_NOALLOC_MAX_N / 256 of them) and the finalize's second level.
// Each device holds its own copy at its own address; host code reaches it only
// through the address hipGetSymbolAddress returns for that device.
__device__ __align__(256) double scratch[kStaticPartials + kFinalizeBlocks];

namespace {

// G groups per lane: with G > 1 the lane's mean-gradient groups are parked in
// LDS during the rank walk and written out afterwards as one burst of
// nontemporal 16-byte stores (the LDS reservation also caps the workgroups
// resident per CU); with G == 1 each group is stored as soon as it is summed.
// RM walks the ranks rank-major (rank_sums_rank_major), its running sums in
// the same LDS slots.
template <int NW, int CAP, int G, int C, int BS, typename In, bool SUMSQ, bool RM = false,
          bool RAGGED = false>
__global__ __launch_bounds__(BS) void k_reduce(RowTable<CAP> rows, int world, MeanDiv div,
                                                     int64_t ngroups, int64_t n, TilePlan plan,
                                                     float* __restrict__ g,
                                                     double* __restrict__ partials) {
  extern __shared__ f32x4 gl[];  // G * BS groups when G > 1
  using L = Lanes<In>;
  const int nw = NW > 0 ? NW : world;
  double ss = 0.0;

  for (int64_t t = blockIdx.x; t < plan.count(); t += gridDim.x) {
    int64_t base, end;  // the tile's groups; each lane takes ng of them (at most G)
    plan.range(t, ngroups, &base, &end);
    const int ng = G == 1 ? 1 : (int)((end - base + BS - 1) / BS);
    // a full tile (ng == G) runs loops with compile-time trip counts
    auto tile = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
      auto sink = [&](int k, const float* acc) {
        const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = div(acc[e]);
          if (SUMSQ && qq < end) ss = fma((double)o[e], (double)o[e], ss);
        }
        if (G == 1) {
          if (qq < end) st_nt(o, reinterpret_cast<f32x4*>(g) + qq);
        } else {
          gl[k * BS + threadIdx.x] = o;
        }
      };
      if constexpr (RM)
        rank_sums_rank_major<In, C, G, CAP, BS, FULL, RAGGED>(rows, nw, base, end, ng, gl, sink);
      else rank_sums_streamed<In, C, G, CAP, BS, RAGGED>(rows, nw, base, end, FULL ? G : ng, sink);
      if (G > 1) {
        // group-major: each lane writes back its own entries; rank-major: each
        // wave writes its own run of groups
        const int NG = FULL ? G : ng;
        if constexpr (RM) __syncthreads();
        for (int k = 0; k < NG; ++k) {
          const int r = RM ? wave_run_index(NG, k) : k * BS + (int)threadIdx.x;
          const int64_t qq = base + r;
          if (qq >= end) break;
          st_nt(gl[r], reinterpret_cast<f32x4*>(g) + qq);
        }
        if constexpr (RM) __syncthreads();
      }
    };
    if (ng == G) tile(std::true_type{});
    else tile(std::false_type{});
  }

  // ragged tail (fewer than 4 elements), same order of operations
  if (blockIdx.x == 0) {
    for (int64_t i = ngroups * 4 + threadIdx.x; i < n; i += BS) {
      float s = -0.0f;
      for (int r = 0; r < nw; ++r) s += L::scalar(rows.p[r], i);
      s = div(s);
      g[i] = s;
      if (SUMSQ) ss = fma((double)s, (double)s, ss);
    }
  }

  if (SUMSQ) {
    __shared__ double lds[BS / 64];
    const double b = block_sum_fixed<BS>(ss, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
  }
}

// Element-wise variant for pointers off the 16-byte grid; identical arithmetic.
template <typename In, bool SUMSQ>
__global__ __launch_bounds__(kThreads) void k_reduce_scalar(RowTable<ZS_MAX_WORLD> rows, int world,
                                                            MeanDiv div, int64_t n,
                                                            float* __restrict__ g,
                                                            double* __restrict__ partials) {
  using L = Lanes<In>;
  double ss = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    float s = -0.0f;
    for (int r = 0; r < world; ++r) s += L::scalar(rows.p[r], i);
    s = div(s);
    g[i] = s;
    if (SUMSQ) ss = fma((double)s, (double)s, ss);
  }
  if (SUMSQ) {
    __shared__ double lds[kThreads / 64];
    const double b = block_sum_fixed(ss, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
  }
}

// Sum of partials[b*per, min((b+1)*per, count)) in a fixed order into
// out[b] (deterministic for a given count).
__global__ __launch_bounds__(kThreads) void k_sumsq_finalize(const double* __restrict__ partials,
                                                             int64_t count, int64_t per,
                                                             double* __restrict__ out) {
  const int64_t a = (int64_t)blockIdx.x * per;
  const int64_t e = a + per < count ? a + per : count;
  double s = 0.0;
  for (int64_t i = a + threadIdx.x; i < e; i += kThreads) s += partials[i];
  __shared__ double lds[kThreads / 64];
  const double b = block_sum_fixed(s, lds);
  if (threadIdx.x == 0) out[blockIdx.x] = b;
}

// One group per lane goes with one-wave workgroups (measured 4% faster at
// N=8 than 4-wave ones); staged groups with 4-wave workgroups.
// The one-wave shape reserves LDS it does not use, to cap the workgroups
// resident per CU by world size. From N = 8 up, 14 per CU (11 KiB): 1.4-2.8%
// faster than full residency at N = 8 (with and without the sum of squares),
// where 10 or 20 per CU gained less, and 1.5-3.4% faster at N = 10-15. With
// fewer contributions each workgroup moves fewer bytes per memory round trip
// and more of them must be in flight: full residency was 24-31% faster at
// N = 2-4 and 14% at N = 5, 20 per CU (8 KiB) 7% faster at N = 6 and 2% at 7.
// fp32 rows move twice the bytes per round trip: from N = 8 they take 10 per
// CU (16 KiB), 1-3% faster than 14; at N = 6-7 also 10 per CU, 3% faster than
// 20; at N = 5 13 per CU (12 KiB), 4% faster than full residency.
inline size_t one_wave_lds(int world, bool bf16) {
  if (!bf16 && world >= 5 && world <= 7) return world == 5 ? 12288 : 16384;
  if (world <= 5) return 0;
  if (world <= 7) return 8192;
  return bf16 ? 11264 : 16384;
}

template <int NW, int CAP, int G, int C, typename In, bool RM = false, bool RAGGED = false>
hipError_t run_vec(const void* const* rows, int world, int64_t n, float* g, double* partials,
                   int64_t* grid_out, hipStream_t s) {
  constexpr int BS = RM ? 512 : (G == 1 ? 64 : kThreads);
  RowTable<CAP> t;
  for (int i = 0; i < CAP; ++i) t.p[i] = i < world ? rows[i] : nullptr;
  const int64_t ngroups = n / 4;
  const int64_t span = (int64_t)BS * G;
  const size_t lds = G > 1 ? (size_t)G * BS * 16 : one_wave_lds(world, sizeof(In) == 2);
  auto go = [&](auto kernel) {
    const void* k = reinterpret_cast<const void*>(kernel);
    const TilePlan plan = span > 64 ? balanced_tiles(ngroups, span, device_slots(s, k, BS, lds))
                                    : plain_tiles(ngroups, span);
    int64_t grid = grid_for(plan.count(), 1, BS);
    if (partials && grid > max_partials(n)) grid = max_partials(n);
    *grid_out = grid;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(BS), lds, s, t, world, mean_div(world), ngroups, n,
                       plan, g, partials);
  };
  if (partials) go(k_reduce<NW, CAP, G, C, BS, In, true, RM, RAGGED>);
  else go(k_reduce<NW, CAP, G, C, BS, In, false, RM, RAGGED>);
  return hipGetLastError();
}

template <int G, int C, typename In>
hipError_t dispatch_world(const void* const* rows, int world, int64_t n, float* g,
                          double* partials, int64_t* grid, hipStream_t s) {
  switch (world) {
    case 2: return run_vec<2, 2, G, C, In>(rows, world, n, g, partials, grid, s);
    case 4: return run_vec<4, 4, G, C, In>(rows, world, n, g, partials, grid, s);
    case 8: return run_vec<8, 8, G, C, In>(rows, world, n, g, partials, grid, s);
    case 16: return run_vec<16, 16, G, C, In>(rows, world, n, g, partials, grid, s);
    case 32: return run_vec<32, 32, G, C, In>(rows, world, n, g, partials, grid, s);
    case 64: return run_vec<64, 64, G, C, In>(rows, world, n, g, partials, grid, s);
    default:
      if constexpr (G == 1 && C == 8) {
        if (world > 8 && world < 16)  // 9-15 ranks: one batch of row loads (rank_sums_streamed)
          return run_vec<0, 64, G, C, In, false, true>(rows, world, n, g, partials, grid, s);
      }
      if (world <= 64) return run_vec<0, 64, G, C, In>(rows, world, n, g, partials, grid, s);
      return run_vec<0, ZS_MAX_WORLD, G, C, In>(rows, world, n, g, partials, grid, s);
  }
}

// The rank-major shape of the single pass: 16 groups per lane in 8-wave
// workgroups, 128 KiB of LDS, the ranks walked in chunks of C (the last one
// short when C does not divide the world size).
template <typename In>
hipError_t dispatch_world_rm(const void* const* rows, int world, int64_t n, float* g,
                             double* partials, int64_t* grid, hipStream_t s) {
  constexpr int C = sizeof(In) == 2 ? 4 : 2;
  switch (world) {
    case 16: return run_vec<16, 16, 16, C, In, true>(rows, world, n, g, partials, grid, s);
    case 32: return run_vec<32, 32, 16, C, In, true>(rows, world, n, g, partials, grid, s);
    case 64: return run_vec<64, 64, 16, C, In, true>(rows, world, n, g, partials, grid, s);
    default:
      if (world % C != 0) {
        if (world <= 64) return run_vec<0, 64, 16, C, In, true, true>(rows, world, n, g, partials, grid, s);
        return run_vec<0, ZS_MAX_WORLD, 16, C, In, true, true>(rows, world, n, g, partials, grid, s);
      }
      if (world <= 64) return run_vec<0, 64, 16, C, In, true>(rows, world, n, g, partials, grid, s);
      return run_vec<0, ZS_MAX_WORLD, 16, C, In, true>(rows, world, n, g, partials, grid, s);
  }
}

// Measured on MI355X: deep staging (16 groups, 64 KiB) pays off when the
// rank walk is long, and the rank-major walk in 8-wave workgroups more so
// (at N = 33 and 30 the group-major shape ran at 30% of peak); with few
// contributions direct stores are faster.
template <typename In>
hipError_t dispatch_shape(const void* const* rows, int world, int64_t n, float* g,
                          double* partials, int64_t* grid, hipStream_t s) {
  const int gsel = tuning().reduce_g > 0 ? tuning().reduce_g : (world >= 16 ? 16 : 1);
  const bool c4 = tuning().rank_chunk == 4;
  if (tuning().reduce_g == 0 && world >= 16) return dispatch_world_rm<In>(rows, world, n, g, partials, grid, s);
  switch (gsel) {
    case 16:
      return c4 ? dispatch_world<16, 4, In>(rows, world, n, g, partials, grid, s)
                : dispatch_world<16, 8, In>(rows, world, n, g, partials, grid, s);
    case 4:
      return c4 ? dispatch_world<4, 4, In>(rows, world, n, g, partials, grid, s)
                : dispatch_world<4, 8, In>(rows, world, n, g, partials, grid, s);
    default:
      return c4 ? dispatch_world<1, 4, In>(rows, world, n, g, partials, grid, s)
                : dispatch_world<1, 8, In>(rows, world, n, g, partials, grid, s);
  }
}


}  // namespace

hipError_t launch_reduce(const void* const* rows, int world, int dtype, int64_t n, float* g,
                         double* sumsq, double* partials, hipStream_t s) {
  int64_t grid = 0;
  hipError_t err = hipSuccess;
  if (n > 0) {
    bool vec = aligned_to(g, 16);
    const uintptr_t ra = dtype == ZS_BF16 ? 7u : 15u;  // one lane group: 8 B of bf16, 16 B of fp32
    for (int i = 0; i < world; ++i) vec = vec && (reinterpret_cast<uintptr_t>(rows[i]) & ra) == 0;
    double* parts = sumsq ? partials : nullptr;
    if (vec) {
      err = dtype == ZS_BF16 ? dispatch_shape<uint16_t>(rows, world, n, g, parts, &grid, s)
                             : dispatch_shape<float>(rows, world, n, g, parts, &grid, s);
    } else {
      RowTable<ZS_MAX_WORLD> t;
      for (int i = 0; i < ZS_MAX_WORLD; ++i) t.p[i] = i < world ? rows[i] : nullptr;
      grid = max_partials(n);
      const MeanDiv d = mean_div(world);
      const dim3 gd((unsigned)grid), bd(kThreads);
      if (dtype == ZS_BF16 && parts)
        hipLaunchKernelGGL((k_reduce_scalar<uint16_t, true>), gd, bd, 0, s, t, world, d, n, g, parts);
      else if (dtype == ZS_BF16)
        hipLaunchKernelGGL((k_reduce_scalar<uint16_t, false>), gd, bd, 0, s, t, world, d, n, g, parts);
      else if (parts)
        hipLaunchKernelGGL((k_reduce_scalar<float, true>), gd, bd, 0, s, t, world, d, n, g, parts);
      else
        hipLaunchKernelGGL((k_reduce_scalar<float, false>), gd, bd, 0, s, t, world, d, n, g, parts);
      err = hipGetLastError();
    }
  }
  if (err != hipSuccess) return err;
  if (sumsq) err = launch_sumsq_finalize(partials, grid, sumsq, s);
  return err;
}

hipError_t static_partials(hipStream_t s, double** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static double* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<double*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_sumsq_finalize(double* partials, int64_t count, double* out, hipStream_t s) {
  if (count <= 16 * kThreads) {
    hipLaunchKernelGGL(k_sumsq_finalize, dim3(1), dim3(kThreads), 0, s, partials, count, count, out);
    return hipGetLastError();
  }
  const int64_t per = (count + kFinalizeBlocks - 1) / kFinalizeBlocks;
  const int64_t blocks = (count + per - 1) / per;  // <= kFinalizeBlocks
  double* second = partials + count;
  hipLaunchKernelGGL(k_sumsq_finalize, dim3((unsigned)blocks), dim3(kThreads), 0, s, partials, count,
                     per, second);
  hipLaunchKernelGGL(k_sumsq_finalize, dim3(1), dim3(kThreads), 0, s, second, blocks, blocks, out);
  return hipGetLastError();
}

}  // namespace zs
