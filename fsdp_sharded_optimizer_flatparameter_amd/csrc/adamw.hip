// AdamW on the rank's fp32 master/m/v slice, with the bf16 copy for the
// all-gather fused into the same pass; and the standalone fp32 -> bf16 cast.
//
// Pages: "Lesson 5: ZeRO and FSDP" s3 (ZeRO-1/2 step 2: each rank updates its
// own 1/N of the fp32 state and master weights locally and converts them to
// BF16; ZeRO-3 item 4: no communication) and Fig. 5-4 (write back the BF16
// parameter shard); "Data parallelism and ZeRO memory sharding" s4.2 (the
// bias-corrected step, eps outside the square root); "FSDP" (Latent Atlas)
// s8.2 step 6 and s9.3 (hyper-parameters). Decoupled weight decay.
//
// HBM-bound: 28 bytes per element (read g, theta, m, v; write theta, m, v),
// +2 with the fused bf16 store. Lanes move 16-byte vectors of 4 fp32 and
// aligned 8-byte words of 4 bf16 (a rank's bf16 slot can sit 2, 4 or 6 bytes
// past an 8-byte boundary when S is not a multiple of 4; the words then
// straddle neighbouring lanes' groups).
#include <cmath>

#include "zs_device.hpp"
#include "zs_launch.hpp"

namespace zs {

AdamConsts adam_consts(const zs_adamw_hparams& hp) {
  const double t = (double)hp.step;
  const double bc1 = 1.0 - std::pow(hp.beta1, t);
  const double bc2 = 1.0 - std::pow(hp.beta2, t);
  AdamConsts c;
  c.b1 = (float)hp.beta1;
  c.omb1 = (float)(1.0 - hp.beta1);
  c.b2 = (float)hp.beta2;
  c.omb2 = (float)(1.0 - hp.beta2);
  c.step_size = (float)(hp.lr / bc1);
  c.decay = (float)(1.0 - hp.lr * hp.weight_decay);
  c.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  c.eps = (float)hp.eps;
  return c;
}

namespace {

template <int V, int BS, bool CAST, bool SCALE>
__global__ __launch_bounds__(BS) void k_adamw(float* __restrict__ th, float* __restrict__ m,
                                                    float* __restrict__ v,
                                                    const float* __restrict__ g, int64_t ngroups,
                                                    int64_t n, AdamConsts c,
                                                    const float* __restrict__ scale,
                                                    uint16_t* __restrict__ out, int om) {
  const float sc = SCALE ? *scale : 1.0f;
  const int64_t tile = (int64_t)BS * V;
  for (int64_t base = (int64_t)blockIdx.x * tile; base < ngroups;
       base += (int64_t)gridDim.x * tile) {
    int64_t q[V];
    f32x4 G[V], T[V], M[V], W[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t qq = base + threadIdx.x + (int64_t)j * BS;
      q[j] = qq < ngroups ? qq : ngroups - 1;
      G[j] = ld_nt(reinterpret_cast<const f32x4*>(g) + q[j]);
      T[j] = ld_nt(reinterpret_cast<const f32x4*>(th) + q[j]);
      M[j] = ld_nt(reinterpret_cast<const f32x4*>(m) + q[j]);
      W[j] = ld_nt(reinterpret_cast<const f32x4*>(v) + q[j]);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const bool ok = base + threadIdx.x + (int64_t)j * BS < ngroups;
      uint32_t lo = 0, hi = 0;  // the bf16 group, packed on live lanes only
      if (ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float tt = T[j][e], mm = M[j][e], vv = W[j][e];
          const float gg = SCALE ? G[j][e] * sc : G[j][e];
          adamw_elem(tt, mm, vv, gg, c);
          T[j][e] = tt;
          M[j][e] = mm;
          W[j][e] = vv;
        }
        st_nt(T[j], reinterpret_cast<f32x4*>(th) + q[j]);
        st_nt(M[j], reinterpret_cast<f32x4*>(m) + q[j]);
        st_nt(W[j], reinterpret_cast<f32x4*>(v) + q[j]);
        if (CAST) {
          lo = pack_bf16x2(T[j][0], T[j][1]);
          hi = pack_bf16x2(T[j][2], T[j][3]);
          if (!(om & 1)) store_bf16_even(out, q[j], lo, hi, om);
        }
      }
      if (CAST && (om & 1)) store_bf16_odd(out, q[j], lo, hi, ok, om);  // every lane
    }
  }
  if (blockIdx.x == 0) {  // ragged tail
    for (int64_t i = ngroups * 4 + threadIdx.x; i < n; i += BS) {
      float tt = th[i], mm = m[i], vv = v[i];
      const float gg = SCALE ? g[i] * sc : g[i];
      adamw_elem(tt, mm, vv, gg, c);
      th[i] = tt;
      m[i] = mm;
      v[i] = vv;
      if (CAST) out[i] = (uint16_t)f32_to_bf16(tt);
    }
  }
}

// Element-wise variant for pointers off the vector grid; identical arithmetic.
template <bool CAST, bool SCALE>
__global__ __launch_bounds__(kThreads) void k_adamw_scalar(float* __restrict__ th,
                                                           float* __restrict__ m,
                                                           float* __restrict__ v,
                                                           const float* __restrict__ g, int64_t n,
                                                           AdamConsts c,
                                                           const float* __restrict__ scale,
                                                           uint16_t* __restrict__ out) {
  const float sc = SCALE ? *scale : 1.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    float tt = th[i], mm = m[i], vv = v[i];
    const float gg = SCALE ? g[i] * sc : g[i];
    adamw_elem(tt, mm, vv, gg, c);
    th[i] = tt;
    m[i] = mm;
    v[i] = vv;
    if (CAST) out[i] = (uint16_t)f32_to_bf16(tt);
  }
}

// Elements [head, head + 4 * ngroups) go as 16-byte fp32 loads and 8-byte bf16
// stores, lane-contiguous; block 0 converts [0, head) and the tail past them.
template <int V, int BS>
__global__ __launch_bounds__(BS) void k_cast(const float* __restrict__ src, int64_t head,
                                             int64_t ngroups, int64_t n, uint16_t* __restrict__ out,
                                             int om) {
  const int64_t tile = (int64_t)BS * V;
  const float* vsrc = src + head;
  uint16_t* vout = out + head;
  for (int64_t base = (int64_t)blockIdx.x * tile; base < ngroups;
       base += (int64_t)gridDim.x * tile) {
    f32x4 x[V];
    int64_t q[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t qq = base + threadIdx.x + (int64_t)j * BS;
      q[j] = qq < ngroups ? qq : ngroups - 1;
      x[j] = ld_nt(reinterpret_cast<const f32x4*>(vsrc) + q[j]);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const bool ok = base + threadIdx.x + (int64_t)j * BS < ngroups;
      const uint32_t lo = pack_bf16x2(x[j][0], x[j][1]), hi = pack_bf16x2(x[j][2], x[j][3]);
      if (om & 1) store_bf16_odd(vout, q[j], lo, hi, ok, om);  // every lane
      else if (ok) store_bf16_even(vout, q[j], lo, hi, om);
    }
  }
  if (blockIdx.x == 0) {
    for (int64_t i = threadIdx.x; i < head; i += BS) out[i] = (uint16_t)f32_to_bf16(src[i]);
    for (int64_t i = head + ngroups * 4 + threadIdx.x; i < n; i += BS)
      out[i] = (uint16_t)f32_to_bf16(src[i]);
  }
}

__global__ __launch_bounds__(kThreads) void k_cast_scalar(const float* __restrict__ src, int64_t n,
                                                          uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    out[i] = (uint16_t)f32_to_bf16(src[i]);
}

// One-wave workgroups under a 16 KiB reservation (10 waves per CU) measured
// 7% faster than 4-wave workgroups under 32 KiB.
constexpr int kAdamBS = 64;

template <int V, bool CAST, bool SCALE>
void run_adamw(float* th, float* m, float* v, const float* g, int64_t n, const AdamConsts& c,
               const float* scale, uint16_t* out, hipStream_t s) {
  const int64_t ngroups = n / 4;
  const int64_t grid = grid_for(ngroups, (int64_t)kAdamBS * V, kAdamBS);
  const int om = out ? bf16_out_mode(out) : 0;
  hipLaunchKernelGGL((k_adamw<V, kAdamBS, CAST, SCALE>), dim3((unsigned)grid), dim3(kAdamBS),
                     (size_t)tuning().adamw_lds, s, th, m, v, g, ngroups, n, c, scale, out, om);
}

template <bool CAST, bool SCALE>
void pick_v(float* th, float* m, float* v, const float* g, int64_t n, const AdamConsts& c,
            const float* scale, uint16_t* out, hipStream_t s) {
  switch (tuning().adamw_v) {
    case 1: run_adamw<1, CAST, SCALE>(th, m, v, g, n, c, scale, out, s); break;
    case 4: run_adamw<4, CAST, SCALE>(th, m, v, g, n, c, scale, out, s); break;
    default: run_adamw<2, CAST, SCALE>(th, m, v, g, n, c, scale, out, s); break;
  }
}

}  // namespace

hipError_t launch_adamw(float* th, float* m, float* v, const float* g, int64_t n,
                        const zs_adamw_hparams& hp, const float* scale, uint16_t* out,
                        hipStream_t s) {
  if (n == 0) return hipSuccess;
  const AdamConsts c = adam_consts(hp);
  const bool vec = aligned_to(th, 16) && aligned_to(m, 16) && aligned_to(v, 16) && aligned_to(g, 16) && (!out || aligned_to(out, 2));
  if (vec) {
    if (out && scale) pick_v<true, true>(th, m, v, g, n, c, scale, out, s);
    else if (out) pick_v<true, false>(th, m, v, g, n, c, scale, out, s);
    else if (scale) pick_v<false, true>(th, m, v, g, n, c, scale, out, s);
    else pick_v<false, false>(th, m, v, g, n, c, scale, out, s);
  } else {
    const dim3 gd((unsigned)grid_for(n, 4 * kThreads)), bd(kThreads);
    if (out && scale) hipLaunchKernelGGL((k_adamw_scalar<true, true>), gd, bd, 0, s, th, m, v, g, n, c, scale, out);
    else if (out) hipLaunchKernelGGL((k_adamw_scalar<true, false>), gd, bd, 0, s, th, m, v, g, n, c, scale, out);
    else if (scale) hipLaunchKernelGGL((k_adamw_scalar<false, true>), gd, bd, 0, s, th, m, v, g, n, c, scale, out);
    else hipLaunchKernelGGL((k_adamw_scalar<false, false>), gd, bd, 0, s, th, m, v, g, n, c, scale, out);
  }
  return hipGetLastError();
}

hipError_t launch_cast(const float* src, int64_t n, uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (aligned_to(src, 16) && aligned_to(out, 2)) {
    // The vector part starts where the waves' aligned 8-byte words fall on a
    // 128-byte boundary, so that each wave stores whole cache lines: HBM3E
    // turns a partial-line write into a read-modify-write, and the rank-63
    // slot of the 7.5B shard (8 bytes off the 16-byte grid) ran at 70% of
    // peak against 83% for an aligned slot. The words begin at each group for
    // an output on an 8-byte boundary and 3 or 1 elements into it for one 2
    // or 6 bytes past (see store_bf16_odd); an output 4 bytes past stores
    // 4-byte halves, whose waves straddle a line at either end whatever the
    // shift. The shift is a multiple of 4 elements, so the fp32 loads stay
    // 16-byte aligned.
    const uintptr_t a = reinterpret_cast<uintptr_t>(out);
    const uintptr_t lead = ((8u - (a & 7u)) & 7u) / 2u;  // elements to the next 8-byte boundary
    int64_t head = (int64_t)(((128u - ((a + 2u * lead) & 127u)) & 127u) / 2u);
    if (head > n) head = n;
    const int64_t ngroups = (n - head) / 4;
    const dim3 gd((unsigned)grid_for(ngroups, 2 * kAdamBS, kAdamBS));
    hipLaunchKernelGGL((k_cast<2, kAdamBS>), gd, dim3(kAdamBS), 0, s, src, head, ngroups, n, out,
                       bf16_out_mode(out + head));
  } else {
    const dim3 gd((unsigned)grid_for(n, 4 * kThreads));
    hipLaunchKernelGGL(k_cast_scalar, gd, dim3(kThreads), 0, s, src, n, out);
  }
  return hipGetLastError();
}

}  // namespace zs
