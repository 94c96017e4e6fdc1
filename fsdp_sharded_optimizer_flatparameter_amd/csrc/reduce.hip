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
//   * each lane owns V 16-byte groups (8 bf16 or 4 fp32 elements each);
//   * row pointers sit in the kernel-argument segment (SGPR bases);
//   * ranks are walked in chunks of 8: the chunk's loads are all issued before
//     its adds, so 8*V independent 16-byte loads are in flight per lane while
//     the fp32 sum still runs in ascending rank order starting from rank 0;
//   * one IEEE division by N (a multiply by the exact reciprocal when N is a
//     power of two), so the result is independent of the launch shape;
//   * rows are read with the nontemporal hint (each byte is used once).
#include <cstdlib>

#include "zs_device.hpp"
#include "zs_launch.hpp"

namespace zs {

const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning x{0, 0, 0};
    const char* e;
    x.reduce_v = (e = std::getenv("ZS_REDUCE_V")) ? std::atoi(e) : 0;
    if (x.reduce_v != 1 && x.reduce_v != 2) x.reduce_v = 0;  // 0 = pick by world size
    x.adamw_v = (e = std::getenv("ZS_ADAMW_V")) ? std::atoi(e) : 2;
    if (x.adamw_v != 1 && x.adamw_v != 2 && x.adamw_v != 4) x.adamw_v = 2;
    x.grid_cap = (e = std::getenv("ZS_GRID_CAP")) ? std::atoll(e) : 0;
    // gridDim.x * blockDim.x must stay below 2^32; grid-stride loops cover the rest
    const int64_t kHardCap = int64_t(1) << 22;
    if (x.grid_cap <= 0 || x.grid_cap > kHardCap) x.grid_cap = kHardCap;
    return x;
  }();
  return t;
}

int64_t max_partials(int64_t n) {
  // every sum-of-squares launch uses at most one workgroup per 1024 elements
  const int64_t b = (n + 1023) / 1024;
  const int64_t kMax = 65536;
  return b < 1 ? 1 : (b > kMax ? kMax : b);
}

namespace {

constexpr int kRankChunk = 8;

MeanDiv mean_div(int world) {
  MeanDiv d;
  d.n = (float)world;
  d.pow2 = (world & (world - 1)) == 0;
  d.inv = 1.0f / (float)world;  // exact when pow2
  return d;
}

template <int NW, int CAP, int V, typename In, bool SUMSQ>
__global__ __launch_bounds__(kThreads) void k_reduce(RowTable<CAP> rows, int world, MeanDiv div,
                                                     int64_t ngroups, int64_t n,
                                                     float* __restrict__ g,
                                                     double* __restrict__ partials) {
  using L = Lanes<In>;
  constexpr int E = L::E;
  const int nw = NW > 0 ? NW : world;
  const int64_t tile = (int64_t)kThreads * V;
  double ss = 0.0;

  for (int64_t base = (int64_t)blockIdx.x * tile; base < ngroups;
       base += (int64_t)gridDim.x * tile) {
    int64_t q[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t qq = base + threadIdx.x + (int64_t)j * kThreads;
      q[j] = qq < ngroups ? qq : ngroups - 1;  // clamped: loads stay in bounds, stores skipped
    }
    float acc[V][E];
#pragma unroll
    for (int j = 0; j < V; ++j)
      L::decode(ld_nt(static_cast<const u32x4*>(rows.p[0]) + q[j]), acc[j]);

    // one chunk of ranks at a time: bounds the registers held by loads in flight
#pragma unroll 1
    for (int r0 = 1; r0 < nw; r0 += kRankChunk) {
      u32x4 buf[kRankChunk][V];
#pragma unroll
      for (int u = 0; u < kRankChunk; ++u) {
        if (r0 + u < nw) {
          const u32x4* row = static_cast<const u32x4*>(rows.p[r0 + u]);
#pragma unroll
          for (int j = 0; j < V; ++j) buf[u][j] = ld_nt(row + q[j]);
        }
      }
#pragma unroll
      for (int u = 0; u < kRankChunk; ++u) {
        if (r0 + u < nw) {
#pragma unroll
          for (int j = 0; j < V; ++j) L::add(buf[u][j], acc[j]);
        }
      }
    }

#pragma unroll
    for (int j = 0; j < V; ++j) {
      if (base + threadIdx.x + (int64_t)j * kThreads < ngroups) {
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          o[e] = div(acc[j][e]);
          if (SUMSQ) ss = fma((double)o[e], (double)o[e], ss);
        }
        f32x4* dst = reinterpret_cast<f32x4*>(g) + q[j] * (E / 4);
#pragma unroll
        for (int h = 0; h < E / 4; ++h)
          dst[h] = f32x4{o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]};
      }
    }
  }

  // ragged tail (fewer than E elements), same order of operations
  if (blockIdx.x == 0) {
    for (int64_t i = ngroups * E + threadIdx.x; i < n; i += kThreads) {
      float s = L::scalar(rows.p[0], i);
      for (int r = 1; r < nw; ++r) s += L::scalar(rows.p[r], i);
      s = div(s);
      g[i] = s;
      if (SUMSQ) ss = fma((double)s, (double)s, ss);
    }
  }

  if (SUMSQ) {
    __shared__ double lds[kThreads / 64];
    const double b = block_sum_fixed(ss, lds);
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
    float s = L::scalar(rows.p[0], i);
    for (int r = 1; r < world; ++r) s += L::scalar(rows.p[r], i);
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

// Sum of the per-workgroup partials in a fixed order (deterministic).
__global__ __launch_bounds__(kThreads) void k_sumsq_finalize(const double* __restrict__ partials,
                                                             int64_t count,
                                                             double* __restrict__ out) {
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += kThreads) s += partials[i];
  __shared__ double lds[kThreads / 64];
  const double b = block_sum_fixed(s, lds);
  if (threadIdx.x == 0) *out = b;
}

template <int NW, int CAP, int V, typename In>
hipError_t run_vec(const void* const* rows, int world, int64_t n, float* g, double* partials,
                   int64_t* grid_out, hipStream_t s) {
  RowTable<CAP> t;
  for (int i = 0; i < CAP; ++i) t.p[i] = i < world ? rows[i] : nullptr;
  constexpr int E = Lanes<In>::E;
  const int64_t ngroups = n / E;
  const int64_t tile = (int64_t)kThreads * V;
  int64_t grid = (ngroups + tile - 1) / tile;
  if (grid > tuning().grid_cap) grid = tuning().grid_cap;
  if (partials && grid > max_partials(n)) grid = max_partials(n);
  if (grid < 1) grid = 1;
  *grid_out = grid;
  if (partials)
    hipLaunchKernelGGL((k_reduce<NW, CAP, V, In, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       s, t, world, mean_div(world), ngroups, n, g, partials);
  else
    hipLaunchKernelGGL((k_reduce<NW, CAP, V, In, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       s, t, world, mean_div(world), ngroups, n, g, partials);
  return hipGetLastError();
}

template <int V, typename In>
hipError_t dispatch_world(const void* const* rows, int world, int64_t n, float* g,
                          double* partials, int64_t* grid, hipStream_t s) {
  switch (world) {
    case 2: return run_vec<2, 2, V, In>(rows, world, n, g, partials, grid, s);
    case 4: return run_vec<4, 4, V, In>(rows, world, n, g, partials, grid, s);
    case 8: return run_vec<8, 8, V, In>(rows, world, n, g, partials, grid, s);
    case 16: return run_vec<16, 16, V, In>(rows, world, n, g, partials, grid, s);
    case 32: return run_vec<32, 32, V, In>(rows, world, n, g, partials, grid, s);
    case 64: return run_vec<64, 64, V, In>(rows, world, n, g, partials, grid, s);
    default:
      if (world <= 64) return run_vec<0, 64, V, In>(rows, world, n, g, partials, grid, s);
      return run_vec<0, ZS_MAX_WORLD, V, In>(rows, world, n, g, partials, grid, s);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_reduce(const void* const* rows, int world, int dtype, int64_t n, float* g,
                         double* sumsq, double* partials, hipStream_t s) {
  int64_t grid = 0;
  hipError_t err = hipSuccess;
  if (n > 0) {
    bool vec = aligned16(g);
    for (int i = 0; i < world; ++i) vec = vec && aligned16(rows[i]);
    double* parts = sumsq ? partials : nullptr;
    if (vec) {
      const int v = tuning().reduce_v ? tuning().reduce_v : (world <= 16 ? 2 : 1);
      if (dtype == ZS_BF16)
        err = v == 2 ? dispatch_world<2, uint16_t>(rows, world, n, g, parts, &grid, s)
                     : dispatch_world<1, uint16_t>(rows, world, n, g, parts, &grid, s);
      else
        err = v == 2 ? dispatch_world<2, float>(rows, world, n, g, parts, &grid, s)
                     : dispatch_world<1, float>(rows, world, n, g, parts, &grid, s);
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
  if (sumsq) {
    hipLaunchKernelGGL(k_sumsq_finalize, dim3(1), dim3(kThreads), 0, s, partials, grid, sumsq);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace zs
