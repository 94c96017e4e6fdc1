// One pass over the rank's slice: mean of the N contributions, AdamW on the
// fp32 master/m/v, bf16 store into the all-gather slot.
//
// The arithmetic is exactly that of the reduce kernel followed by the AdamW
// kernel (same rank order, same division, same AdamW element routine), so the
// results are bit-identical to the two-call path; only the fp32 gradient's
// round trip through HBM (8 bytes per element) disappears:
//   bytes per element = 2N (bf16 rows) + 12 (read theta, m, v) + 12 (write) + 2.
// Pages: "Lesson 5: ZeRO and FSDP" s3 (ZeRO-1/2 steps 1-2, reduce-scatter
// result -> local update -> BF16), "Data parallelism and ZeRO memory
// sharding" s3.1 and s4.2.
#include "zs_device.hpp"
#include "zs_launch.hpp"

namespace zs {
namespace {

constexpr int kRankChunk = 8;

MeanDiv mean_div(int world) {
  MeanDiv d;
  d.n = (float)world;
  d.pow2 = (world & (world - 1)) == 0;
  d.inv = 1.0f / (float)world;
  return d;
}

template <int NW, int CAP, typename In, bool CAST, bool SCALE>
__global__ __launch_bounds__(kThreads) void k_fused(RowTable<CAP> rows, int world, MeanDiv div,
                                                    int64_t ngroups, int64_t n,
                                                    float* __restrict__ th, float* __restrict__ m,
                                                    float* __restrict__ v, AdamConsts c,
                                                    const float* __restrict__ scale,
                                                    uint16_t* __restrict__ out) {
  using L = Lanes<In>;
  constexpr int E = L::E;
  constexpr int H = E / 4;  // fp32 16-byte vectors per group
  const int nw = NW > 0 ? NW : world;
  const float sc = SCALE ? *scale : 1.0f;

  for (int64_t base = (int64_t)blockIdx.x * kThreads; base < ngroups;
       base += (int64_t)gridDim.x * kThreads) {
    const int64_t qq = base + threadIdx.x;
    const int64_t q = qq < ngroups ? qq : ngroups - 1;

    // optimizer state first, so its loads are in flight during the rank sum
    f32x4 T[H], M[H], W[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      T[h] = ld_nt(reinterpret_cast<const f32x4*>(th) + q * H + h);
      M[h] = ld_nt(reinterpret_cast<const f32x4*>(m) + q * H + h);
      W[h] = ld_nt(reinterpret_cast<const f32x4*>(v) + q * H + h);
    }

    float acc[E];
    L::decode(ld_nt(static_cast<const u32x4*>(rows.p[0]) + q), acc);
#pragma unroll 1
    for (int r0 = 1; r0 < nw; r0 += kRankChunk) {
      u32x4 buf[kRankChunk];
#pragma unroll
      for (int u = 0; u < kRankChunk; ++u)
        if (r0 + u < nw) buf[u] = ld_nt(static_cast<const u32x4*>(rows.p[r0 + u]) + q);
#pragma unroll
      for (int u = 0; u < kRankChunk; ++u)
        if (r0 + u < nw) L::add(buf[u], acc);
    }
    if (qq >= ngroups) continue;
#pragma unroll
    for (int h = 0; h < H; ++h) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float gg = div(acc[4 * h + e]);
        if (SCALE) gg *= sc;
        float tt = T[h][e], mm = M[h][e], vv = W[h][e];
        adamw_elem(tt, mm, vv, gg, c);
        T[h][e] = tt;
        M[h][e] = mm;
        W[h][e] = vv;
      }
      st_nt(T[h], reinterpret_cast<f32x4*>(th) + q * H + h);
      st_nt(M[h], reinterpret_cast<f32x4*>(m) + q * H + h);
      st_nt(W[h], reinterpret_cast<f32x4*>(v) + q * H + h);
      if (CAST) {
        const u32x2 b{pack_bf16x2(T[h][0], T[h][1]), pack_bf16x2(T[h][2], T[h][3])};
        st_nt(b, reinterpret_cast<u32x2*>(out) + q * H + h);
      }
    }
  }
  if (blockIdx.x == 0) {  // ragged tail
    for (int64_t i = ngroups * E + threadIdx.x; i < n; i += kThreads) {
      float s = L::scalar(rows.p[0], i);
      for (int r = 1; r < nw; ++r) s += L::scalar(rows.p[r], i);
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
    float s = L::scalar(rows.p[0], i);
    for (int r = 1; r < world; ++r) s += L::scalar(rows.p[r], i);
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

int64_t grid_for(int64_t units, int64_t per_block) {
  int64_t gsz = (units + per_block - 1) / per_block;
  if (gsz > tuning().grid_cap) gsz = tuning().grid_cap;
  return gsz < 1 ? 1 : gsz;
}

template <int NW, int CAP, typename In>
void run_fused(const void* const* rows, int world, int64_t n, float* th, float* m, float* v,
               const AdamConsts& c, const float* scale, uint16_t* out, hipStream_t s) {
  RowTable<CAP> t;
  for (int i = 0; i < CAP; ++i) t.p[i] = i < world ? rows[i] : nullptr;
  const int64_t ngroups = n / Lanes<In>::E;
  const dim3 gd((unsigned)grid_for(ngroups, kThreads)), bd(kThreads);
  const MeanDiv d = mean_div(world);
  if (out && scale)
    hipLaunchKernelGGL((k_fused<NW, CAP, In, true, true>), gd, bd, 0, s, t, world, d, ngroups, n, th, m, v, c, scale, out);
  else if (out)
    hipLaunchKernelGGL((k_fused<NW, CAP, In, true, false>), gd, bd, 0, s, t, world, d, ngroups, n, th, m, v, c, scale, out);
  else if (scale)
    hipLaunchKernelGGL((k_fused<NW, CAP, In, false, true>), gd, bd, 0, s, t, world, d, ngroups, n, th, m, v, c, scale, out);
  else
    hipLaunchKernelGGL((k_fused<NW, CAP, In, false, false>), gd, bd, 0, s, t, world, d, ngroups, n, th, m, v, c, scale, out);
}

template <typename In>
void dispatch(const void* const* rows, int world, int64_t n, float* th, float* m, float* v,
              const AdamConsts& c, const float* scale, uint16_t* out, hipStream_t s) {
  switch (world) {
    case 2: run_fused<2, 2, In>(rows, world, n, th, m, v, c, scale, out, s); break;
    case 4: run_fused<4, 4, In>(rows, world, n, th, m, v, c, scale, out, s); break;
    case 8: run_fused<8, 8, In>(rows, world, n, th, m, v, c, scale, out, s); break;
    case 16: run_fused<16, 16, In>(rows, world, n, th, m, v, c, scale, out, s); break;
    case 32: run_fused<32, 32, In>(rows, world, n, th, m, v, c, scale, out, s); break;
    case 64: run_fused<64, 64, In>(rows, world, n, th, m, v, c, scale, out, s); break;
    default:
      if (world <= 64) run_fused<0, 64, In>(rows, world, n, th, m, v, c, scale, out, s);
      else run_fused<0, ZS_MAX_WORLD, In>(rows, world, n, th, m, v, c, scale, out, s);
  }
}

bool al(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

hipError_t launch_fused(const void* const* rows, int world, int dtype, int64_t n, float* th,
                        float* m, float* v, const zs_adamw_hparams& hp, const float* scale,
                        uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const AdamConsts c = adam_consts(hp);
  bool vec = al(th, 16) && al(m, 16) && al(v, 16) && (!out || al(out, 8));
  for (int i = 0; i < world; ++i) vec = vec && al(rows[i], 16);
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
