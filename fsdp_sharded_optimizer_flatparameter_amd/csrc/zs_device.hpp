// Device-side building blocks shared by the zs kernels (gfx950, wave64).
//
// Every kernel of the sharded update is a streaming pass over HBM: each lane
// moves whole 16-byte vectors (global_load_dwordx4 / global_store_dwordx4),
// single-use streams carry the nontemporal hint so they do not evict lines
// that are reused, and arithmetic is plain fp32 VALU work (no MFMA: there is
// no contraction on this path).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "zs.h"

namespace zs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 wave64 per workgroup

// ---- streaming memory access -------------------------------------------------

// Every pointer these helpers take is device (global) memory. Pointers that
// come out of a table in memory (the parameter descriptors) are generic to the
// compiler, which would access them with FLAT instructions; a FLAT store counts
// on the LDS/scalar-load counter as well, so every wait for a shuffle or a
// descriptor load would also wait for the stores in flight. The casts below
// give the compiler the global address space.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

// Nontemporal: each byte these kernels stream is used once (cached loads or
// stores measured 10-20% slower for every kernel of the step).
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)p);
}
template <typename T>
__device__ __forceinline__ void st_nt(T v, T* p) {
  __builtin_nontemporal_store(v, (gptr<T>)p);
}

// Plain (cached) element accesses to global memory.
template <typename T>
__device__ __forceinline__ T ld_g(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <typename T>
__device__ __forceinline__ void st_g(T v, T* p) {
  *(gptr<T>)p = v;
}

// ---- bf16 <-> fp32 -----------------------------------------------------------
// bf16 is the upper half of an IEEE fp32 pattern; widening is exact.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest with ties to even, computed on the integer
// pattern: adding 0x7fff plus the lowest kept bit carries into the kept half
// exactly when the dropped half is above one half, or equal to it with an odd
// kept half. NaN keeps its sign and top payload and gets the quiet bit.
// Overflow carries into the exponent and yields infinity.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// bf16 stores of a lane's 4-element group q into out[4q .. 4q + 3], packed as
// pack_bf16x2 gives them (lo = elements 0-1, hi = 2-3). `d` is out's distance
// from an 8-byte boundary in elements (0..3, uniform across the launch: a
// rank's slot of the all-gather buffer starts at element r*S, so it follows S).
//
// d even: one 8-byte store (d == 0) or two aligned 4-byte stores (d == 2), by
// the lane alone; callers issue it inside their live-lane branch.
__device__ __forceinline__ void store_bf16_even(uint16_t* out, int64_t q, uint32_t lo, uint32_t hi,
                                                int d) {
  uint16_t* p = out + 4 * q;
  if (d == 0) {
    st_nt(u32x2{lo, hi}, reinterpret_cast<u32x2*>(p));
  } else {
    st_nt(lo, reinterpret_cast<uint32_t*>(p));
    st_nt(hi, reinterpret_cast<uint32_t*>(p) + 1);
  }
}

// d odd (odd S): called by every lane of the wave (it shuffles across it),
// lane i+1 holding group q+1; `ok` is false for lanes past the end of the
// range, which store nothing and should pass constants (packed inside the
// callers' live-lane branch, so that the wave never waits for such a lane's
// pending loads). Each lane stores the aligned 8-byte word that starts
// s = 4 - d elements into its group -- its own last d elements and the next
// lane's first s, taken by a wave shuffle -- instead of four 2-byte stores
// (measured 1.5% faster for the single pass on the 7.5B shard and 3% on the
// Llama-3-8B shard; for d == 2 the shuffle was 0.5% slower than the two
// 4-byte stores). Only a lane whose neighbour is missing (the wave's first and
// last lanes, and the last group of the range) writes those elements one by
// one.
__device__ __forceinline__ void store_bf16_odd(uint16_t* out, int64_t q, uint32_t lo, uint32_t hi,
                                               bool ok, int d) {
  uint16_t* p = out + 4 * q;
  const int lane = threadIdx.x & 63;
  const uint64_t live = __ballot(ok);
  const uint32_t nlo = __shfl_down(lo, 1, 64), nhi = __shfl_down(hi, 1, 64);
  if (!ok) return;
  const bool has_next = lane < 63 && ((live >> (lane + 1)) & 1u);
  const bool has_prev = lane > 0 && ((live >> (lane - 1)) & 1u);
  const int s = 4 - d;
  const uint64_t own = (uint64_t)lo | ((uint64_t)hi << 32);
  if (has_next) {
    const uint64_t nxt = (uint64_t)nlo | ((uint64_t)nhi << 32);
    const uint64_t w = (own >> (16 * s)) | (nxt << (16 * d));
    st_nt(u32x2{(uint32_t)w, (uint32_t)(w >> 32)}, reinterpret_cast<u32x2*>(p + s));
  } else {
    for (int e = s; e < 4; ++e) st_nt((uint16_t)(own >> (16 * e)), p + e);
  }
  if (!has_prev)
    for (int e = 0; e < s; ++e) st_nt((uint16_t)(own >> (16 * e)), p + e);
}

// Host: the `d` of store_bf16_even / store_bf16_odd for an output pointer
// (2-byte aligned).
inline int bf16_out_mode(const void* out) {
  return (int)((reinterpret_cast<uintptr_t>(out) & 7u) >> 1);
}

// ---- gradient contributions ----------------------------------------------------

// Row pointers travel in the kernel-argument segment: uniform across the grid,
// they land in SGPRs and every row load is a global_load with a scalar base.
template <int CAP>
struct RowTable {
  const void* p[CAP];
};

// A lane's unit of work is a group of 4 consecutive elements in every stream:
// 8 bytes of bf16 or 16 bytes of fp32 contributions, 16 bytes of each fp32
// state array and 8 bytes of bf16 output. Lane i of a wave takes group
// base + i, so every load and store instruction of a wave covers one
// contiguous span (512 B or 1 KiB) of its stream.
template <typename In>
struct Lanes;
template <>
struct Lanes<uint16_t> {
  typedef u32x2 Vec;  // 4 bf16
  __device__ __forceinline__ static void add(const Vec& w, float* acc) {
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
  }
  __device__ __forceinline__ static float scalar(const void* row, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(row)[i]);
  }
};
template <>
struct Lanes<float> {
  typedef u32x4 Vec;  // 4 fp32
  __device__ __forceinline__ static void add(const Vec& w, float* acc) {
    acc[0] += __uint_as_float(w.x); acc[1] += __uint_as_float(w.y);
    acc[2] += __uint_as_float(w.z); acc[3] += __uint_as_float(w.w);
  }
  __device__ __forceinline__ static float scalar(const void* row, int64_t i) {
    return static_cast<const float*>(row)[i];
  }
};

// Rank sums of the first `ng` (at most G) groups per lane -- group k at index
// base + k*BS + lane, BS the workgroup size, lanes past `end` loading group
// end-1 and discarding it -- streamed as one double-buffered sequence of rank
// chunks that runs across
// group boundaries: while chunk i is added, chunk i+1 (the next ranks of the
// same group, or the first ranks of the next group) is already in flight, so a
// lane never waits a full memory round trip between two groups. Each group's
// sum starts from -0.0, the additive identity of IEEE addition (-0 + x == x for
// every x, signed zeros included), and adds ranks in ascending order, so it
// equals c_0 + c_1 + ... + c_{N-1} evaluated left to right in fp32.
// sink(k, acc) receives group k's finished sums.
//
// RAGGED (one group per lane, 9 to 16 ranks, C = 8): the ranks are loaded in
// one batch whose row count a switch makes a compile-time constant. The
// chunked walk's second chunk had its row loads predicated on the world size,
// which made the wave wait for every load in flight: the single pass ran at
// 52-61% of peak for N = 10-15, against 78% at N = 8. With one chunk (up to 8
// ranks) the chunked walk is fine, and the launchers keep it; compiled into
// the same kernel, the batch code made N = 5 and 7 1.5-5% slower.
template <typename In, int C, int G, int CAP, int BS = kThreads, bool RAGGED = false, typename Sink>
__device__ __forceinline__ void rank_sums_streamed(const RowTable<CAP>& rows, int nw, int64_t base,
                                                   int64_t end, int ng, Sink&& sink) {
  using L = Lanes<In>;
  using Vec = typename L::Vec;
  if constexpr (G == 1 && RAGGED) {
    if (nw > 8 && nw <= 16) {
      auto batch = [&](auto rr) {
        constexpr int R = decltype(rr)::value;
        const int64_t qq = base + threadIdx.x;
        const int64_t q = qq < end ? qq : end - 1;  // clamped: loads stay in bounds
        Vec v[R];
#pragma unroll
        for (int u = 0; u < R; ++u) v[u] = ld_nt(static_cast<const Vec*>(rows.p[u]) + q);
        float acc[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
#pragma unroll
        for (int u = 0; u < R; ++u) L::add(v[u], acc);
        sink(0, acc);
      };
      switch (nw) {
        case 9: batch(std::integral_constant<int, 9>{}); return;
        case 10: batch(std::integral_constant<int, 10>{}); return;
        case 11: batch(std::integral_constant<int, 11>{}); return;
        case 12: batch(std::integral_constant<int, 12>{}); return;
        case 13: batch(std::integral_constant<int, 13>{}); return;
        case 14: batch(std::integral_constant<int, 14>{}); return;
        case 15: batch(std::integral_constant<int, 15>{}); return;
        default: batch(std::integral_constant<int, 16>{}); return;
      }
    }
  }
  const int nch = (nw + C - 1) / C;  // chunks per group
  const int total = (G == 1 ? 1 : ng) * nch;
  auto load = [&](int idx, Vec* buf) {
    const int k = idx / nch;
    const int r0 = (idx - k * nch) * C;
    const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
    const int64_t q = qq < end ? qq : end - 1;  // clamped: loads stay in bounds
#pragma unroll
    for (int u = 0; u < C; ++u)
      if (r0 + u < nw) buf[u] = ld_nt(static_cast<const Vec*>(rows.p[r0 + u]) + q);
  };
  float acc[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
  auto consume = [&](int idx, const Vec* buf) {
    const int k = idx / nch;
    const int r0 = (idx - k * nch) * C;
#pragma unroll
    for (int u = 0; u < C; ++u)
      if (r0 + u < nw) L::add(buf[u], acc);
    if (r0 + C >= nw) {
      sink(k, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = -0.0f;
    }
  };
  Vec a[C], b[C];
  load(0, a);
#pragma unroll 1
  for (int idx = 0; idx < total; idx += 2) {
    if (idx + 1 < total) load(idx + 1, b);
    consume(idx, a);
    if (idx + 1 >= total) break;
    if (idx + 2 < total) load(idx + 2, a);
    consume(idx + 1, b);
  }
}

// Rank sums of G groups per lane in rank-major order: the C ranks of one chunk
// are added into all G groups' running sums before the next chunk is read, so
// a workgroup reads each row as one contiguous run of G*BS*4 elements per
// chunk (64 KiB of bf16 rows for G = 16, BS = 512) instead of G separate runs
// of BS*4. The running sums live in `sums` (LDS, G*BS vectors; each lane
// touches only its own entries, so no barrier is involved), initialised to
// -0.0 here; each element still adds c_0, c_1, ..., c_{N-1} in that order in
// fp32, so the result is bit-identical to rank_sums_streamed. The loads of
// step i+1 (C rows of one group) are in flight while step i is added.
// Only the first `ng` (at most G) groups per lane are walked, lanes past `end`
// loading group end-1 and discarding it; FULL (ng == G) takes the loop with a
// compile-time step count. Without RAGGED nw must be a multiple of C; with it
// the nw % C (1..C-1) ranks after the last whole chunk are added by a second,
// shorter walk over the groups whose rank count is a compile-time constant, so
// that no load of either walk is conditional (predicated row loads made the
// wave wait for every load in flight at each step: 50-54% of peak at N = 33
// against 83-87% at N = 48). sink(k, acc) receives group k's finished sums
// after its last rank.
//
// The full-tile loop prefetches across the first step of each pair only: its
// second prefetch is conditional, so the wave waits for all outstanding loads
// before the pair's second add. That half-pipelined loop measured faster for
// bf16 rows at N=64 than prefetching both steps of every pair (3% for the
// single pass and the reduce on the 7.5B shard) and much faster than no
// prefetch (23-31%); with fp32 rows the two prefetching loops measured within
// 1.2% of each other.
template <typename In, int C, int G, int CAP, int BS, bool FULL, bool RAGGED = false, typename Sink>
__device__ __forceinline__ void rank_sums_rank_major(const RowTable<CAP>& rows, int nw, int64_t base,
                                                     int64_t end, int ng, f32x4* sums, Sink&& sink) {
  using L = Lanes<In>;
  using Vec = typename L::Vec;
  const int nch = nw / C;                 // whole chunks
  const int rem = RAGGED ? nw - nch * C : 0;  // ranks after them
#pragma unroll
  for (int k = 0; k < G; ++k) sums[k * BS + threadIdx.x] = f32x4{-0.0f, -0.0f, -0.0f, -0.0f};
  auto load = [&](int c, int k, Vec* buf) {
    const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
    const int64_t q = qq < end ? qq : end - 1;  // clamped: loads stay in bounds
#pragma unroll
    for (int u = 0; u < C; ++u) buf[u] = ld_nt(static_cast<const Vec*>(rows.p[c * C + u]) + q);
  };
  auto consume = [&](int c, int k, const Vec* buf) {
    const f32x4 s = sums[k * BS + threadIdx.x];
    float acc[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
    for (int u = 0; u < C; ++u) L::add(buf[u], acc);
    if ((!RAGGED || rem == 0) && c + 1 == nch) sink(k, acc);
    else sums[k * BS + threadIdx.x] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  };
  Vec a[C], b[C];
  if constexpr (FULL) {
    // step idx reads chunk idx / G of group idx % G
    const int total = nch * G;
    load(0, 0, a);
#pragma unroll 1
    for (int idx = 0; idx < total; idx += 2) {
      if (idx + 1 < total) load((idx + 1) / G, (idx + 1) % G, b);
      consume(idx / G, idx % G, a);
      if (idx + 1 >= total) break;
      if (idx + 2 < total) load((idx + 2) / G, (idx + 2) % G, a);
      consume((idx + 1) / G, (idx + 1) % G, b);
    }
  } else {
    // (c, k) advance group-fastest over ng groups; pairs whose two prefetches
    // both exist run in the loop, the last one or two steps after it
    const int total = nch * ng;
    auto next = [&](int& c, int& k) {
      if (++k == ng) {
        k = 0;
        ++c;
      }
    };
    int c0 = 0, k0 = 0, c1 = 0, k1 = 0;
    load(c0, k0, a);
    int idx = 0;
#pragma unroll 1
    for (; idx + 2 < total; idx += 2) {
      c1 = c0;
      k1 = k0;
      next(c1, k1);
      load(c1, k1, b);
      consume(c0, k0, a);
      c0 = c1;
      k0 = k1;
      next(c0, k0);
      load(c0, k0, a);
      consume(c1, k1, b);
    }
    if (idx + 1 < total) {
      c1 = c0;
      k1 = k0;
      next(c1, k1);
      load(c1, k1, b);
      consume(c0, k0, a);
      consume(c1, k1, b);
    } else {
      consume(c0, k0, a);
    }
  }
  if constexpr (RAGGED) {
    // ranks nch*C .. nw-1, R of them, over the same groups; the group loop is
    // the full-tile loop's, with R rows per step
    auto tail = [&](auto rr) {
      constexpr int R = decltype(rr)::value;
      const int NG = FULL ? G : ng;
      auto tload = [&](int k, Vec* buf) {
        const int64_t qq = base + (int64_t)k * BS + threadIdx.x;
        const int64_t q = qq < end ? qq : end - 1;
#pragma unroll
        for (int u = 0; u < R; ++u) buf[u] = ld_nt(static_cast<const Vec*>(rows.p[nch * C + u]) + q);
      };
      auto tcons = [&](int k, const Vec* buf) {
        const f32x4 s = sums[k * BS + threadIdx.x];
        float acc[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
        for (int u = 0; u < R; ++u) L::add(buf[u], acc);
        sink(k, acc);
      };
      Vec ta[R], tb[R];
      tload(0, ta);
#pragma unroll 1
      for (int k = 0; k < NG; k += 2) {
        if (k + 1 < NG) tload(k + 1, tb);
        tcons(k, ta);
        if (k + 1 >= NG) break;
        if (k + 2 < NG) tload(k + 2, ta);
        tcons(k + 1, tb);
      }
    };
    if (rem == 1) tail(std::integral_constant<int, 1>{});
    if constexpr (C > 2) {
      if (rem == 2) tail(std::integral_constant<int, 2>{});
      if (rem == 3) tail(std::integral_constant<int, 3>{});
    }
    static_assert(C <= 4, "the tail walk is built for chunks of up to 4 ranks");
  }
}

// Index, within the tile, of the group that a lane takes at step k of the pass
// after a rank-major walk over ng groups per lane. The walk leaves group r's
// result in entry r of its LDS array (step k of lane i writes entry k*BS + i).
// After a barrier, wave w takes the ng*64 consecutive groups from w*ng*64 on,
// 64 per step, so each wave streams its own run of the state arrays. In the
// walk's order (all waves at step k on groups k*BS .. k*BS + BS - 1, one front
// per array) the single pass measured 1.1-1.6% slower on the 7.5B shard and
// the 70B chunk.
__device__ __forceinline__ int wave_run_index(int ng, int k) {
  return (int)(threadIdx.x >> 6) * (ng * 64) + k * 64 + (int)(threadIdx.x & 63);
}

// Division of the rank sum by N. For N a power of two the product with the
// exact reciprocal is the same correctly rounded value, so both branches give
// the IEEE quotient.
struct MeanDiv {
  float inv;   // 1/N, exact when pow2
  float n;     // N as fp32
  int pow2;
  __device__ __forceinline__ float operator()(float s) const { return pow2 ? s * inv : s / n; }
};

// Host: the divisor of a launch over `world` contributions.
inline MeanDiv mean_div(int world) {
  MeanDiv d;
  d.n = (float)world;
  d.pow2 = (world & (world - 1)) == 0;
  d.inv = 1.0f / (float)world;  // exact when world is a power of two
  return d;
}

// ---- AdamW ---------------------------------------------------------------------

// fp32 constants derived on the host (in double) from zs_adamw_hparams.
struct AdamConsts {
  float b1, omb1;         // beta1, 1 - beta1
  float b2, omb2;         // beta2, 1 - beta2
  float step_size;        // lr / (1 - beta1^t)
  float decay;            // 1 - lr * weight_decay
  float inv_sqrt_bc2;     // 1 / sqrt(1 - beta2^t)
  float eps;
};

// One element of the decoupled-decay, bias-corrected AdamW step.
//   m' = b1 m + (1-b1) g,  v' = b2 v + (1-b2) g^2,
//   theta' = theta (1 - lr wd) - step_size m' / (sqrt(v') / sqrt(1-b2^t) + eps)
__device__ __forceinline__ void adamw_elem(float& th, float& m, float& v, float g,
                                           const AdamConsts& c) {
  m = fmaf(c.b1, m, c.omb1 * g);
  v = fmaf(c.b2, v, c.omb2 * (g * g));
  const float denom = fmaf(sqrtf(v), c.inv_sqrt_bc2, c.eps);
  th = fmaf(th, c.decay, -((c.step_size * m) / denom));
}

// ---- block reduction of per-thread fp64 partials (fixed order) ------------------

template <int BS = kThreads>
__device__ __forceinline__ double block_sum_fixed(double x, double* lds /* >= BS/64 */) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = x;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
    for (int w = 0; w < BS / 64; ++w) s += lds[w];
  }
  return s;  // valid in thread 0
}

}  // namespace zs
