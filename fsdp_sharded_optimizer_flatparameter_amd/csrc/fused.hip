// One pass over the rank's slice: mean of the N contributions, AdamW on the
// fp32 master/m/v, bf16 store into the all-gather slot.
//
// The arithmetic is exactly that of the reduce kernel followed by the AdamW
// kernel (same rank order, same division, same AdamW element routine), so the
// results are bit-identical to the two-call path; only the fp32 gradient's
// round trip through HBM (8 bytes per element) disappears:
//   bytes per element = 2N (bf16 rows) + 12 (read theta, m, v) + 12 (write) + 2.
// Lanes own groups of 4 consecutive elements, lane-contiguous in every stream.
// Pages: "Lesson 5: ZeRO and FSDP" s3 (ZeRO-1/2 steps 1-2, reduce-scatter
// result -> local update -> BF16), "Data parallelism and ZeRO memory
// sharding" s3.1 and s4.2.
#include <type_traits>

#include "zs_device.hpp"

#include "zs_launch.hpp"

namespace zs {
namespace {

// Two phases per workgroup over G groups per lane (G*BS*4 consecutive elements):
//   1. the rank walk only -- the mean gradient of each group is parked in LDS;
//   2. AdamW over the fp32 state of the same groups, the state read and
//      written as 16-byte vectors per group: after the group-major walk each
//      lane reads back its own LDS entries (no barrier); after the rank-major
//      walk a barrier lets each wave take its own run of groups
//      (wave_run_index).
// Keeping the row streams and the state read-modify-write apart in time, and
// the LDS reservation (which caps the workgroups resident per CU), keeps fewer
// DRAM pages open at once; both were measured to raise HBM throughput.
// RM selects the rank-major walk (rank_sums_rank_major: each chunk of C ranks
// is added into all G groups before the next chunk is read, so every row is
// read as one long run per chunk), otherwise the group-major one
// (rank_sums_streamed).
template <int NW, int CAP, int G, int C, int BS, typename In, bool CAST, bool SCALE, bool RM,
          bool RAGGED = false>
__global__ __launch_bounds__(BS) void k_fused(RowTable<CAP> rows, int world, MeanDiv div,
                                                    int64_t ngroups, int64_t n, TilePlan plan,
                                                    float* __restrict__ th, float* __restrict__ m,
                                                    float* __restrict__ v, AdamConsts c,
                                                    const float* __restrict__ scale,
                                                    uint16_t* __restrict__ out, int om) {
  extern __shared__ f32x4 gl[];  // G * BS mean-gradient groups (plus any occupancy pad)
  using L = Lanes<In>;
  const int nw = NW > 0 ? NW : world;
  const float sc = SCALE ? *scale : 1.0f;

  for (int64_t t = blockIdx.x; t < plan.count(); t += gridDim.x) {
    int64_t base, end;  // the tile's groups; each lane takes ng of them (at most G)
    plan.range(t, ngroups, &base, &end);
    const int ng = G == 1 ? 1 : (int)((end - base + BS - 1) / BS);
    // a full tile (ng == G) runs loops with compile-time trip counts
    auto tile = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
      auto sink = [&](int k, const float* acc) {
        f32x4 gv;
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[e] = SCALE ? div(acc[e]) * sc : div(acc[e]);
        gl[k * BS + threadIdx.x] = gv;
      };
      // EARLY: with few bf16 contributions the state loads of a one-group tile
      // are issued before its row loads, so that the workgroup waits for
      // memory once instead of twice. Measured against loading the state after
      // the walk: 7.8% faster at N = 2, 8.9% at 3, 7.2% at 5, 5.5% at 7, but
      // 1.3% slower at N = 8, which keeps the later loads.
      constexpr bool EARLY = sizeof(In) == 2 && G == 1 && !RM && !RAGGED && (NW == 0 || NW <= 4);
      [[maybe_unused]] f32x4 eT, eM, eW;
      if constexpr (EARLY) {
        const int64_t qq = base + threadIdx.x;
        const int64_t q = qq < end ? qq : end - 1;
        eT = ld_nt(reinterpret_cast<const f32x4*>(th) + q);
        eM = ld_nt(reinterpret_cast<const f32x4*>(m) + q);
        eW = ld_nt(reinterpret_cast<const f32x4*>(v) + q);
      }
      if constexpr (RM)
        rank_sums_rank_major<In, C, G, CAP, BS, FULL, RAGGED>(rows, nw, base, end, ng, gl, sink);
      else rank_sums_streamed<In, C, G, CAP, BS, RAGGED>(rows, nw, base, end, FULL ? G : ng, sink);
      // phase 2: with bf16 contributions double-buffered (group k+1's state
      // loads are in flight while group k is updated and stored); after the
      // rank-major walk each wave updates its own run of groups
      [[maybe_unused]] const int NG = FULL ? G : ng;
      if constexpr (RM) __syncthreads();
      auto ridx = [&](int k) -> int {
        if constexpr (RM) return wave_run_index(NG, k);
        else return k * BS + (int)threadIdx.x;
      };
      auto qidx = [&](int k) { return base + (int64_t)ridx(k); };
      auto load = [&](int k, f32x4& T, f32x4& M, f32x4& W) {
        const int64_t q = qidx(k) < end ? qidx(k) : end - 1;
        T = ld_nt(reinterpret_cast<const f32x4*>(th) + q);
        M = ld_nt(reinterpret_cast<const f32x4*>(m) + q);
        W = ld_nt(reinterpret_cast<const f32x4*>(v) + q);
      };
      auto update = [&](int k, f32x4& T, f32x4& M, f32x4& W) {  // every lane calls it
        const int64_t qq = qidx(k);
        const bool ok = qq < end;
        uint32_t lo = 0, hi = 0;  // the bf16 group, packed on live lanes only
        if (ok) {
          const f32x4 gv = gl[ridx(k)];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float tt = T[e], mm = M[e], vv = W[e];
            adamw_elem(tt, mm, vv, gv[e], c);
            T[e] = tt;
            M[e] = mm;
            W[e] = vv;
          }
          st_nt(T, reinterpret_cast<f32x4*>(th) + qq);
          st_nt(M, reinterpret_cast<f32x4*>(m) + qq);
          st_nt(W, reinterpret_cast<f32x4*>(v) + qq);
          if (CAST) {
            lo = pack_bf16x2(T[0], T[1]);
            hi = pack_bf16x2(T[2], T[3]);
            if (!(om & 1)) store_bf16_even(out, qq, lo, hi, om);
          }
        }
        if (CAST && (om & 1)) store_bf16_odd(out, qq, lo, hi, ok, om);
      };
      if constexpr (sizeof(In) == 4 && !RM) {
        // fp32 contributions, group-major walk: all G groups' state loads are
        // issued before the first update (measured 2% faster than two in
        // flight at N=64); groups past ng load group end-1 and store nothing
        f32x4 T[G], M[G], W[G];
#pragma unroll
        for (int k = 0; k < G; ++k) load(k, T[k], M[k], W[k]);
#pragma unroll
        for (int k = 0; k < G; ++k) update(k, T[k], M[k], W[k]);
      } else if constexpr (EARLY) {
        update(0, eT, eM, eW);
      } else if constexpr (FULL) {
        f32x4 T0, M0, W0, T1, M1, W1;
        load(0, T0, M0, W0);
#pragma unroll 1
        for (int k = 0; k < G; k += 2) {
          if (k + 1 < G) load(k + 1, T1, M1, W1);
          update(k, T0, M0, W0);
          if (k + 1 >= G) break;
          if (k + 2 < G) load(k + 2, T0, M0, W0);
          update(k + 1, T1, M1, W1);
        }
      } else {
        // pairs whose two prefetches both exist, then the last one or two groups
        f32x4 T0, M0, W0, T1, M1, W1;
        load(0, T0, M0, W0);
        int k = 0;
#pragma unroll 1
        for (; k + 2 < ng; k += 2) {
          load(k + 1, T1, M1, W1);
          update(k, T0, M0, W0);
          load(k + 2, T0, M0, W0);
          update(k + 1, T1, M1, W1);
        }
        if (k + 1 < ng) {
          load(k + 1, T1, M1, W1);
          update(k, T0, M0, W0);
          update(k + 1, T1, M1, W1);
        } else {
          update(k, T0, M0, W0);
        }
      }
      if constexpr (RM) __syncthreads();  // the next tile's walk rewrites entries other waves read
    };
    if (ng == G) tile(std::true_type{});
    else tile(std::false_type{});
  }
  if (blockIdx.x == 0) {  // ragged tail (fewer than 4 elements)
    for (int64_t i = ngroups * 4 + threadIdx.x; i < n; i += BS) {
      float s = -0.0f;
      for (int r = 0; r < nw; ++r) s += L::scalar(rows.p[r], i);
      float gg = div(s);
      if (SCALE) gg *= sc;
      float tt = th[i], mm = m[i], vv = v[i];
      adamw_elem(tt, mm, vv, gg, c);
      th[i] = tt;
      m[i] = mm;
      v[i] = vv;
      if (CAST) out[i] = (uint16_t)f32_to_bf16(tt);
    }
  }
}

template <typename In, bool CAST, bool SCALE>
__global__ __launch_bounds__(kThreads) void k_fused_scalar(RowTable<ZS_MAX_WORLD> rows, int world,
                                                           MeanDiv div, int64_t n,
                                                           float* __restrict__ th,
                                                           float* __restrict__ m,
                                                           float* __restrict__ v, AdamConsts c,
                                                           const float* __restrict__ scale,
                                                           uint16_t* __restrict__ out) {
  using L = Lanes<In>;
  const float sc = SCALE ? *scale : 1.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    float s = -0.0f;
    for (int r = 0; r < world; ++r) s += L::scalar(rows.p[r], i);
    float gg = div(s);
    if (SCALE) gg *= sc;
    float tt = th[i], mm = m[i], vv = v[i];
    adamw_elem(tt, mm, vv, gg, c);
    th[i] = tt;
    m[i] = mm;
    v[i] = vv;
    if (CAST) out[i] = (uint16_t)f32_to_bf16(tt);
  }
}



struct Shape {
  int bs;      // workgroup size: 512 or 256 (8 or 4 waves), or 64 (one wave)
  int g;       // groups per lane staged in LDS
  size_t lds;  // dynamic LDS bytes per workgroup (>= g * bs * 16)
  bool rm;     // rank-major walk
};

// Ranks per chunk of the rank-major walk: about 2 KiB of row loads per lane
// group in flight, double-buffered (4 bf16 or 2 fp32 rows).
template <typename In>
constexpr int rm_chunk() { return sizeof(In) == 2 ? 4 : 2; }

// Measured on MI355X. With many contributions the row walk dominates: 8-wave
// workgroups walking the ranks rank-major over 16 staged groups (128 KiB of
// LDS, one workgroup per CU) read every row in 64 KiB runs and ran the 7.5B
// shard at N=64 3.5% faster, and the 70B chunk with fp32 rows 10% faster, than
// 4-wave workgroups walking group-major over 16 groups (64 KiB, two per CU).
// World sizes the chunk width does not divide take the same walk, the last
// 1-3 ranks added by a short second walk: at N = 33 and 30 with bf16 rows the
// group-major shape had run at 34-35% of peak, this one at 76-78%. With few
// contributions the state read-modify-write dominates: one-wave workgroups
// of a single group each, with a 16 KiB reservation (10 waves per CU), ran
// the Llama-3-8B shard at N=8 11% faster than 4-wave workgroups (which were
// best with 2 groups and 64 KiB); residency matters sharply there (5 waves
// per CU ran 35% slower, 20 waves 8% slower).
Shape fused_shape(int world, bool bf16) {
  Shape sh;
  const bool many = world >= 16;
  sh.bs = tuning().fused_bs > 0 ? tuning().fused_bs : (many ? 512 : 64);
  sh.rm = sh.bs == 512;
  sh.g = tuning().fused_g > 0 ? tuning().fused_g : (many ? 16 : 1);
  if (sh.bs == 64 && sh.g > 4) sh.g = 4;  // one-wave workgroups are built for 1, 2 or 4 groups
  if (sh.rm) sh.g = 16;                     // the rank-major shape is built for 16 groups
  const size_t need = (size_t)sh.g * sh.bs * 16;
  // one-wave workgroups: 10 per CU (16 KiB) at N = 8; 20 per CU (8 KiB)
  // below, which measured 4% faster at N = 2, 3% at N = 6 and the same at N = 4
  // (and 4.6% slower at N = 8); with bf16 rows 13 per CU (12 KiB) at N = 9-15,
  // 8% faster at N = 10, 6% at 12 and 2% at 15 (and 2% slower at N = 8). fp32
  // rows move twice the bytes per round trip and want fewer workgroups: from
  // N = 8, 8 per CU (20 KiB) measured 0.3-3.5% faster than 10 and 12 per CU
  // 2-4% slower; at N = 4-7, 10 per CU 7-9% faster than 20, and at N = 2-3 13
  // per CU (12 KiB), 6% faster at N = 2
  const size_t fp32_wave = world <= 3 ? 12288 : (world <= 7 ? 16384 : 20480);
  const size_t one_wave =
      !bf16 ? fp32_wave : (world <= 7 ? 8192 : (world > 8 && world < 16 ? 12288 : 16384));
  sh.lds = tuning().fused_lds > 0 ? (size_t)tuning().fused_lds : (sh.bs == 64 ? one_wave : 65536);
  if (sh.lds < need) sh.lds = need;
  return sh;
}

template <int NW, int CAP, int G, int C, int BS, typename In, bool RM = false, bool RAGGED = false>
void run_fused(const void* const* rows, int world, int64_t n, float* th, float* m, float* v,
               const AdamConsts& c, const float* scale, uint16_t* out, size_t lds, hipStream_t s) {
  RowTable<CAP> t;
  for (int i = 0; i < CAP; ++i) t.p[i] = i < world ? rows[i] : nullptr;
  const int64_t ngroups = n / 4;
  const MeanDiv d = mean_div(world);
  const int om = out ? bf16_out_mode(out) : 0;
  auto go = [&](auto kernel) {
    const void* k = reinterpret_cast<const void*>(kernel);
    const TilePlan plan = BS * G > 64 ? balanced_tiles(ngroups, (int64_t)BS * G, device_slots(s, k, BS, lds))
                                      : plain_tiles(ngroups, (int64_t)BS * G);
    const dim3 gd((unsigned)grid_for(plan.count(), 1, BS)), bd(BS);
    hipLaunchKernelGGL(kernel, gd, bd, lds, s, t, world, d, ngroups, n, plan, th, m, v, c, scale, out, om);
  };
  if (out && scale) go(k_fused<NW, CAP, G, C, BS, In, true, true, RM, RAGGED>);
  else if (out) go(k_fused<NW, CAP, G, C, BS, In, true, false, RM, RAGGED>);
  else if (scale) go(k_fused<NW, CAP, G, C, BS, In, false, true, RM, RAGGED>);
  else go(k_fused<NW, CAP, G, C, BS, In, false, false, RM, RAGGED>);
}

template <typename In, int G, int C, int BS>
void dispatch_world(const void* const* rows, int world, int64_t n, float* th, float* m, float* v,
                    const AdamConsts& c, const float* scale, uint16_t* out, size_t lds, hipStream_t s) {
  switch (world) {
    case 2: run_fused<2, 2, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 4: run_fused<4, 4, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 8: run_fused<8, 8, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 16: run_fused<16, 16, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 32: run_fused<32, 32, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 64: run_fused<64, 64, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    default:
      if constexpr (G == 1 && C == 8 && BS == 64) {
        if (world > 8 && world < 16) {  // 9-15 ranks: one batch of row loads (rank_sums_streamed)
          run_fused<0, 64, G, C, BS, In, false, true>(rows, world, n, th, m, v, c, scale, out, lds, s);
          break;
        }
      }
      if (world <= 64) run_fused<0, 64, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s);
      else run_fused<0, ZS_MAX_WORLD, G, C, BS, In>(rows, world, n, th, m, v, c, scale, out, lds, s);
  }
}

template <typename In, int C>
void dispatch_g(const Shape& sh, const void* const* rows, int world, int64_t n, float* th, float* m,
                float* v, const AdamConsts& c, const float* scale, uint16_t* out, hipStream_t s) {
  if (sh.bs == 64) {
    switch (sh.g) {
      case 2: dispatch_world<In, 2, C, 64>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
      case 4: dispatch_world<In, 4, C, 64>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
      default: dispatch_world<In, 1, C, 64>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
    }
    return;
  }
  switch (sh.g) {
    case 1: dispatch_world<In, 1, C, 256>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
    case 2: dispatch_world<In, 2, C, 256>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
    case 8: dispatch_world<In, 8, C, 256>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
    case 16: dispatch_world<In, 16, C, 256>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
    default: dispatch_world<In, 4, C, 256>(rows, world, n, th, m, v, c, scale, out, sh.lds, s); break;
  }
}

template <typename In>
void dispatch_world_rm(const void* const* rows, int world, int64_t n, float* th, float* m, float* v,
                       const AdamConsts& c, const float* scale, uint16_t* out, size_t lds, hipStream_t s) {
  constexpr int C = rm_chunk<In>();
  switch (world) {
    case 16: run_fused<16, 16, 16, C, 512, In, true>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 32: run_fused<32, 32, 16, C, 512, In, true>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    case 64: run_fused<64, 64, 16, C, 512, In, true>(rows, world, n, th, m, v, c, scale, out, lds, s); break;
    default:
      if (world % C != 0) {  // a short last chunk
        if (world <= 64) run_fused<0, 64, 16, C, 512, In, true, true>(rows, world, n, th, m, v, c, scale, out, lds, s);
        else run_fused<0, ZS_MAX_WORLD, 16, C, 512, In, true, true>(rows, world, n, th, m, v, c, scale, out, lds, s);
      } else if (world <= 64) {
        run_fused<0, 64, 16, C, 512, In, true>(rows, world, n, th, m, v, c, scale, out, lds, s);
      } else {
        run_fused<0, ZS_MAX_WORLD, 16, C, 512, In, true>(rows, world, n, th, m, v, c, scale, out, lds, s);
      }
  }
}

template <typename In>
void dispatch(const void* const* rows, int world, int64_t n, float* th, float* m, float* v,
              const AdamConsts& c, const float* scale, uint16_t* out, hipStream_t s) {
  const Shape sh = fused_shape(world, sizeof(In) == 2);
  if (sh.rm) dispatch_world_rm<In>(rows, world, n, th, m, v, c, scale, out, sh.lds, s);
  else if (tuning().rank_chunk == 4) dispatch_g<In, 4>(sh, rows, world, n, th, m, v, c, scale, out, s);
  else dispatch_g<In, 8>(sh, rows, world, n, th, m, v, c, scale, out, s);
}


}  // namespace

hipError_t launch_fused(const void* const* rows, int world, int dtype, int64_t n, float* th,
                        float* m, float* v, const zs_adamw_hparams& hp, const float* scale,
                        uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const AdamConsts c = adam_consts(hp);
  bool vec = aligned_to(th, 16) && aligned_to(m, 16) && aligned_to(v, 16) && (!out || aligned_to(out, 2));
  for (int i = 0; i < world; ++i) vec = vec && aligned_to(rows[i], dtype == ZS_BF16 ? 8 : 16);
  if (vec) {
    if (dtype == ZS_BF16) dispatch<uint16_t>(rows, world, n, th, m, v, c, scale, out, s);
    else dispatch<float>(rows, world, n, th, m, v, c, scale, out, s);
  } else {
    RowTable<ZS_MAX_WORLD> t;
    for (int i = 0; i < ZS_MAX_WORLD; ++i) t.p[i] = i < world ? rows[i] : nullptr;
    const dim3 gd((unsigned)grid_for(n, 4 * kThreads)), bd(kThreads);
    const MeanDiv d = mean_div(world);
#define ZS_FS(IN, CA, SC) \
  hipLaunchKernelGGL((k_fused_scalar<IN, CA, SC>), gd, bd, 0, s, t, world, d, n, th, m, v, c, scale, out)
    if (dtype == ZS_BF16) {
      if (out && scale) ZS_FS(uint16_t, true, true);
      else if (out) ZS_FS(uint16_t, true, false);
      else if (scale) ZS_FS(uint16_t, false, true);
      else ZS_FS(uint16_t, false, false);
    } else {
      if (out && scale) ZS_FS(float, true, true);
      else if (out) ZS_FS(float, true, false);
      else if (scale) ZS_FS(float, false, true);
      else ZS_FS(float, false, false);
    }
#undef ZS_FS
  }
  return hipGetLastError();
}

}  // namespace zs
