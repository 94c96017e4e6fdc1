// Gradient accumulation over micro-batches and the global-norm clip coefficient.
//
// Pages: "Lesson 5: ZeRO and FSDP" s3 (under gradient accumulation ZeRO-1 sums
// each rank's full local gradient and reduce-scatters once, ZeRO-2
// reduce-scatters every micro-batch and accumulates its 1/N) and s2 (the fp32
// accumulation buffer: 4P for ZeRO-0/1, 4P/N for ZeRO-2/3); "Data parallelism
// and ZeRO memory sharding" s6 (a global norm needs every shard's partial).
//
//   k_accum        acc = (first ? scale*mean : acc + scale*mean)   [sharded]
//                  2N + 8 bytes per element (2N + 4 on the first micro-batch)
//   k_accum_local  acc = (first ? g : acc + g), g bf16 or fp32      [unsharded]
//   k_clip         coefficient = min(1, max_norm / (sqrt(sum of partials) + 1e-6))
#include <cmath>

#include <type_traits>

#include "zs_device.hpp"
#include "zs_launch.hpp"

namespace zs {
namespace {

// G groups per lane (G*BS*4 consecutive elements per workgroup pass), in three
// steps: the previous sums of all G groups are loaded into lane-private LDS
// slots, the rank walk adds each group's scaled mean into its slot, and the G
// results are written back as one burst of 16-byte stores. The row walk then
// runs without a write stream beside it, and the LDS reservation caps the
// workgroups resident per CU. With RM the ranks are walked rank-major
// (rank_sums_rank_major), the slots holding the running sums and then the
// scaled means; after the walk and a barrier each wave reads the previous sums
// of its own run of groups, two groups in flight, and writes the new ones, as
// the single pass updates its state.
template <int NW, int CAP, int G, int BS, typename In, bool SUMSQ, bool FIRST, bool SCALE,
          bool RM = false, bool RAGGED = false>
__global__ __launch_bounds__(BS) void k_accum(RowTable<CAP> rows, int world, MeanDiv div,
                                                    float scale, int64_t ngroups, int64_t n,
                                                    TilePlan plan, float* __restrict__ acc,
                                                    double* __restrict__ partials) {
  using L = Lanes<In>;
  extern __shared__ f32x4 slot[];  // G * BS lane-private slots
  const int nw = NW > 0 ? NW : world;
  double ss = 0.0;
  for (int64_t t = blockIdx.x; t < plan.count(); t += gridDim.x) {
    int64_t base, end;  // the tile's groups; each lane takes ng of them (at most G)
    plan.range(t, ngroups, &base, &end);
    const int ng = G == 1 ? 1 : (int)((end - base + BS - 1) / BS);
    // a full tile (ng == G) runs loops with compile-time trip counts
    auto tile = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
      const int NG = FULL ? G : ng;
      if constexpr (RM) {
        constexpr int C = sizeof(In) == 2 ? 4 : 2;
        rank_sums_rank_major<In, C, G, CAP, BS, FULL, RAGGED>(rows, nw, base, end, ng, slot, [&](int k, const float* s) {
          f32x4 u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            u[e] = div(s[e]);
            if (SCALE) u[e] *= scale;
          }
          slot[k * BS + threadIdx.x] = u;
        });
        // each wave finishes its own run of groups
        __syncthreads();
        auto qidx = [&](int k) { return base + (int64_t)wave_run_index(NG, k); };
        auto finish = [&](int k, const f32x4& prev) {
          const int64_t qq = qidx(k);
          if (qq >= end) return;
          const f32x4 u = slot[wave_run_index(NG, k)];
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = FIRST ? u[e] : prev[e] + u[e];
            if (SUMSQ) ss = fma((double)o[e], (double)o[e], ss);
          }
          st_nt(o, reinterpret_cast<f32x4*>(acc) + qq);
        };
        auto prev_of = [&](int k) {
          const int64_t q = qidx(k) < end ? qidx(k) : end - 1;
          return ld_nt(reinterpret_cast<const f32x4*>(acc) + q);
        };
        if (FIRST) {
#pragma unroll
          for (int k = 0; k < NG; ++k) finish(k, f32x4{0.f, 0.f, 0.f, 0.f});
        } else if constexpr (FULL) {
          f32x4 p0 = prev_of(0), p1;
#pragma unroll 1
          for (int k = 0; k < G; k += 2) {
            if (k + 1 < G) p1 = prev_of(k + 1);
            finish(k, p0);
            if (k + 1 >= G) break;
            if (k + 2 < G) p0 = prev_of(k + 2);
            finish(k + 1, p1);
          }
        } else {
          // pairs whose two prefetches both exist, then the last one or two groups
          f32x4 p0 = prev_of(0), p1;
          int k = 0;
#pragma unroll 1
          for (; k + 2 < ng; k += 2) {
            p1 = prev_of(k + 1);
            finish(k, p0);
            p0 = prev_of(k + 2);
            finish(k + 1, p1);
          }
          if (k + 1 < ng) {
            p1 = prev_of(k + 1);
            finish(k, p0);
            finish(k + 1, p1);
          } else {
            finish(k, p0);
          }
        }
        __syncthreads();  // the next tile's walk rewrites slots other waves read
        return;
      }
      if (!FIRST) {
#pragma unroll
        for (int k = 0; k < G; ++k) {
          const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
          const int64_t q = qq < end ? qq : end - 1;
          slot[k * BS + threadIdx.x] = ld_nt(reinterpret_cast<const f32x4*>(acc) + q);
        }
      }
      rank_sums_streamed<In, 8, G, CAP, BS, RAGGED>(rows, nw, base, end, NG, [&](int k, const float* s) {
        const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float u = div(s[e]);
          if (SCALE) u *= scale;
          o[e] = FIRST ? u : slot[k * BS + threadIdx.x][e] + u;
          if (SUMSQ && qq < end) ss = fma((double)o[e], (double)o[e], ss);
        }
        slot[k * BS + threadIdx.x] = o;
      });
      for (int k = 0; k < NG; ++k) {  // each lane writes back only its own slots
        const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
        if (qq >= end) break;
        st_nt(slot[k * BS + threadIdx.x], reinterpret_cast<f32x4*>(acc) + qq);
      }
    };
    if (ng == G) tile(std::true_type{});
    else tile(std::false_type{});
  }
  if (blockIdx.x == 0) {  // ragged tail
    for (int64_t i = ngroups * 4 + threadIdx.x; i < n; i += BS) {
      float s = -0.0f;
      for (int r = 0; r < nw; ++r) s += L::scalar(rows.p[r], i);
      float u = div(s);
      if (SCALE) u *= scale;
      const float o = FIRST ? u : acc[i] + u;
      acc[i] = o;
      if (SUMSQ) ss = fma((double)o, (double)o, ss);
    }
  }
  if (SUMSQ) {
    __shared__ double lds[BS / 64];
    const double b = block_sum_fixed<BS>(ss, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
  }
}

// Element-wise variant for pointers off the vector grid; identical arithmetic.
template <typename In, bool SUMSQ, bool FIRST, bool SCALE>
__global__ __launch_bounds__(kThreads) void k_accum_scalar(RowTable<ZS_MAX_WORLD> rows, int world,
                                                           MeanDiv div, float scale, int64_t n,
                                                           float* __restrict__ acc,
                                                           double* __restrict__ partials) {
  using L = Lanes<In>;
  double ss = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    float s = -0.0f;
    for (int r = 0; r < world; ++r) s += L::scalar(rows.p[r], i);
    float u = div(s);
    if (SCALE) u *= scale;
    const float o = FIRST ? u : acc[i] + u;
    acc[i] = o;
    if (SUMSQ) ss = fma((double)o, (double)o, ss);
  }
  if (SUMSQ) {
    __shared__ double lds[kThreads / 64];
    const double b = block_sum_fixed(ss, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
  }
}

template <typename In, bool FIRST, int BS = kThreads>
__global__ __launch_bounds__(BS) void k_accum_local(const In* __restrict__ g, int64_t ngroups,
                                                    int64_t n, float* __restrict__ acc, int vec) {
  using L = Lanes<In>;
  using Vec = typename L::Vec;
  if (vec) {
    for (int64_t q = (int64_t)blockIdx.x * BS + threadIdx.x; q < ngroups;
         q += (int64_t)gridDim.x * BS) {
      const Vec w = ld_nt(reinterpret_cast<const Vec*>(g) + q);
      float x[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
      L::add(w, x);  // -0 + g == g exactly: the widened gradient
      f32x4 o;
      if (FIRST) {
        o = f32x4{x[0], x[1], x[2], x[3]};
      } else {
        const f32x4 a = ld_nt(reinterpret_cast<const f32x4*>(acc) + q);
        o = f32x4{a[0] + x[0], a[1] + x[1], a[2] + x[2], a[3] + x[3]};
      }
      st_nt(o, reinterpret_cast<f32x4*>(acc) + q);
    }
  }
  const int64_t start = vec ? ngroups * 4 : 0;
  for (int64_t i = start + (int64_t)blockIdx.x * BS + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * BS) {
    const float x = L::scalar(g, i);
    acc[i] = FIRST ? x : acc[i] + x;
  }
}

__global__ void k_clip(const double* __restrict__ partials, int count, double max_norm,
                       float* __restrict__ coef, double* __restrict__ norm_out) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  double total = 0.0;
  for (int i = 0; i < count; ++i) total += partials[i];  // fixed order
  const double norm = sqrt(total);
  double c = max_norm / (norm + 1e-6);
  if (c > 1.0) c = 1.0;  // a NaN norm keeps a NaN coefficient
  *coef = (float)c;
  if (norm_out) *norm_out = norm;
}


// Measured on MI355X: with many contributions the rank-major shape of the
// single pass (16 groups per lane in 8-wave workgroups, 128 KiB of LDS; the
// last chunk of ranks short where the chunk does not divide the world size);
// with few, the shape of the single pass.
// ZS_ACCUM_SHAPE=1 selects the earlier shapes for comparison (4-wave
// workgroups of 16 groups with many contributions, of 4 with few).
template <int G, int BS, int NW, int CAP, typename In, bool SUMSQ, bool FIRST, bool SCALE, bool RM = false,
          bool RAGGED = false>
void launch_accum_shape(const RowTable<CAP>& t, int world, int64_t n, float* acc, float scale,
                        double* partials, int64_t* grid_out, size_t lds, hipStream_t s) {
  const int64_t ngroups = n / 4;
  const int64_t span = (int64_t)BS * G;
  if (lds < (size_t)G * BS * sizeof(f32x4)) lds = (size_t)G * BS * sizeof(f32x4);
  auto kernel = k_accum<NW, CAP, G, BS, In, SUMSQ, FIRST, SCALE, RM, RAGGED>;
  const TilePlan plan =
      span > 64 ? balanced_tiles(ngroups, span, device_slots(s, reinterpret_cast<const void*>(kernel), BS, lds))
                : plain_tiles(ngroups, span);
  int64_t grid = grid_for(plan.count(), 1, BS);
  if (SUMSQ && grid > max_partials(n)) grid = max_partials(n);
  *grid_out = grid;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(BS), lds, s, t, world, mean_div(world), scale,
                     ngroups, n, plan, acc, partials);
}

template <int NW, int CAP, typename In, bool SUMSQ, bool FIRST, bool SCALE>
void run_accum(const void* const* rows, int world, int64_t n, float* acc, float scale,
               double* partials, int64_t* grid_out, hipStream_t s) {
  RowTable<CAP> t;
  for (int i = 0; i < CAP; ++i) t.p[i] = i < world ? rows[i] : nullptr;
  constexpr int rm_c = sizeof(In) == 2 ? 4 : 2;
  bool ragged = false;  // a short last chunk of ranks (world sizes the chunk does not divide)
  if constexpr (NW == 0) ragged = world % rm_c != 0;
  if (world >= 16 && tuning().accum_shape == 0) {
    if constexpr (NW == 0) {
      if (ragged) {
        launch_accum_shape<16, 512, NW, CAP, In, SUMSQ, FIRST, SCALE, true, true>(t, world, n, acc, scale, partials,
                                                                                  grid_out, 0, s);
        return;
      }
    }
    launch_accum_shape<16, 512, NW, CAP, In, SUMSQ, FIRST, SCALE, true>(t, world, n, acc, scale, partials, grid_out, 0, s);
  } else if (world >= 16)
    launch_accum_shape<16, 256, NW, CAP, In, SUMSQ, FIRST, SCALE>(t, world, n, acc, scale, partials, grid_out, 0, s);
  else if (tuning().accum_shape == 1)
    launch_accum_shape<4, 256, NW, CAP, In, SUMSQ, FIRST, SCALE>(t, world, n, acc, scale, partials, grid_out, 0, s);
  else {
    // one wave: at N = 8 13 KiB of LDS, 12 workgroups per CU (3% faster than
    // 10 on the GPT-2 shard); with fewer contributions more workgroups must be
    // in flight: full residency measured 41% faster at N = 2 and 33% at N = 4,
    // 20 per CU (8 KiB) 23% faster at N = 6 (both 3-4% slower at N = 8). The
    // one-batch walk of N = 9-15 over bf16 rows takes 16 per CU (10 KiB): 7-8%
    // faster than 12 at N = 9-12, 1% at 14-15 (and 3-4% slower with fp32 rows).
    // fp32 rows at N = 5-7 take 13 per CU (12 KiB): 2-5% faster than full
    // residency at N = 5 and than 20 per CU at N = 6-7
    constexpr bool bf16 = sizeof(In) == 2;
    const size_t lds =
        (!bf16 && world >= 5 && world <= 7)
            ? 12288
            : (world <= 5 ? 0 : (world <= 7 ? 8192 : (bf16 && world > 8 && world < 16 ? 10240 : 13312)));
    if constexpr (NW == 0 && CAP == 64) {
      if (world > 8 && world < 16) {  // 9-15 ranks: one batch of row loads (rank_sums_streamed)
        launch_accum_shape<1, 64, NW, CAP, In, SUMSQ, FIRST, SCALE, false, true>(t, world, n, acc, scale, partials,
                                                                                 grid_out, lds, s);
        return;
      }
    }
    launch_accum_shape<1, 64, NW, CAP, In, SUMSQ, FIRST, SCALE>(t, world, n, acc, scale, partials, grid_out, lds, s);
  }
}

template <typename In, bool SUMSQ, bool FIRST, bool SCALE>
void dispatch_world(const void* const* rows, int world, int64_t n, float* acc, float scale,
                    double* partials, int64_t* grid, hipStream_t s) {
  switch (world) {
    case 8: run_accum<8, 8, In, SUMSQ, FIRST, SCALE>(rows, world, n, acc, scale, partials, grid, s); break;
    case 64: run_accum<64, 64, In, SUMSQ, FIRST, SCALE>(rows, world, n, acc, scale, partials, grid, s); break;
    default:
      if (world <= 64) run_accum<0, 64, In, SUMSQ, FIRST, SCALE>(rows, world, n, acc, scale, partials, grid, s);
      else run_accum<0, ZS_MAX_WORLD, In, SUMSQ, FIRST, SCALE>(rows, world, n, acc, scale, partials, grid, s);
  }
}

template <typename In, bool SUMSQ>
void dispatch_flags(bool first, bool scaled, bool vec, const void* const* rows, int world, int64_t n,
                    float* acc, float scale, double* partials, int64_t* grid, hipStream_t s) {
  if (!vec) {
    RowTable<ZS_MAX_WORLD> t;
    for (int i = 0; i < ZS_MAX_WORLD; ++i) t.p[i] = i < world ? rows[i] : nullptr;
    *grid = max_partials(n);
    const dim3 gd((unsigned)*grid), bd(kThreads);
    const MeanDiv d = mean_div(world);
    if (first && scaled) hipLaunchKernelGGL((k_accum_scalar<In, SUMSQ, true, true>), gd, bd, 0, s, t, world, d, scale, n, acc, partials);
    else if (first) hipLaunchKernelGGL((k_accum_scalar<In, SUMSQ, true, false>), gd, bd, 0, s, t, world, d, scale, n, acc, partials);
    else if (scaled) hipLaunchKernelGGL((k_accum_scalar<In, SUMSQ, false, true>), gd, bd, 0, s, t, world, d, scale, n, acc, partials);
    else hipLaunchKernelGGL((k_accum_scalar<In, SUMSQ, false, false>), gd, bd, 0, s, t, world, d, scale, n, acc, partials);
    return;
  }
  if (first && scaled) dispatch_world<In, SUMSQ, true, true>(rows, world, n, acc, scale, partials, grid, s);
  else if (first) dispatch_world<In, SUMSQ, true, false>(rows, world, n, acc, scale, partials, grid, s);
  else if (scaled) dispatch_world<In, SUMSQ, false, true>(rows, world, n, acc, scale, partials, grid, s);
  else dispatch_world<In, SUMSQ, false, false>(rows, world, n, acc, scale, partials, grid, s);
}


}  // namespace

hipError_t launch_accumulate(const void* const* rows, int world, int dtype, int64_t n, float* acc,
                             float scale, bool first, double* sumsq, double* partials,
                             hipStream_t s) {
  int64_t grid = 0;
  if (n > 0) {
    bool vec = aligned_to(acc, 16);
    for (int i = 0; i < world; ++i) vec = vec && aligned_to(rows[i], dtype == ZS_BF16 ? 8 : 16);
    const bool scaled = scale != 1.0f;
    if (dtype == ZS_BF16) {
      if (sumsq) dispatch_flags<uint16_t, true>(first, scaled, vec, rows, world, n, acc, scale, partials, &grid, s);
      else dispatch_flags<uint16_t, false>(first, scaled, vec, rows, world, n, acc, scale, partials, &grid, s);
    } else {
      if (sumsq) dispatch_flags<float, true>(first, scaled, vec, rows, world, n, acc, scale, partials, &grid, s);
      else dispatch_flags<float, false>(first, scaled, vec, rows, world, n, acc, scale, partials, &grid, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sumsq) return launch_sumsq_finalize(partials, grid, sumsq, s);
  return hipSuccess;
}

hipError_t launch_accumulate_local(const void* g, int dtype, int64_t n, float* acc, bool first,
                                   hipStream_t s) {
  if (n == 0) return hipSuccess;
  const bool vec = aligned_to(acc, 16) && aligned_to(g, dtype == ZS_BF16 ? 8 : 16);
  const int64_t ngroups = n / 4;
  // one-wave workgroups, one 4-element group per lane, full residency: 4.5%
  // faster than 4-wave workgroups on the 7.5B shard's size (a 12 KiB or 32 KiB
  // reservation, or two groups per lane, were slower)
  constexpr int BS = 64;
  const dim3 gd((unsigned)grid_for(vec ? ngroups : n, BS, BS)), bd(BS);
  if (dtype == ZS_BF16) {
    if (first) hipLaunchKernelGGL((k_accum_local<uint16_t, true, BS>), gd, bd, 0, s, static_cast<const uint16_t*>(g), ngroups, n, acc, (int)vec);
    else hipLaunchKernelGGL((k_accum_local<uint16_t, false, BS>), gd, bd, 0, s, static_cast<const uint16_t*>(g), ngroups, n, acc, (int)vec);
  } else {
    if (first) hipLaunchKernelGGL((k_accum_local<float, true, BS>), gd, bd, 0, s, static_cast<const float*>(g), ngroups, n, acc, (int)vec);
    else hipLaunchKernelGGL((k_accum_local<float, false, BS>), gd, bd, 0, s, static_cast<const float*>(g), ngroups, n, acc, (int)vec);
  }
  return hipGetLastError();
}

hipError_t launch_clip(const double* partials, int count, double max_norm, float* coef,
                       double* norm, hipStream_t s) {
  hipLaunchKernelGGL(k_clip, dim3(1), dim3(64), 0, s, partials, count, max_norm, coef, norm);
  return hipGetLastError();
}

}  // namespace zs
