// FlatParameter pack (per-parameter tensors -> the rank's fp32 master slice)
// and unshard copy-out (gathered flat bf16 buffer -> per-parameter tensors).
//
// Also the per-parameter dim-0 variants ("Lesson 5: ZeRO and FSDP" s7.2 and
// Fig. 5-5: each parameter sharded on dim 0; "03 - FSDP (ZeRO-3)" s4).
//
// Pages: "Lesson 5: ZeRO and FSDP" s7.1 point 1 (all parameters of a wrapped
// unit flattened into one 1-D tensor that is split along DP; contiguous slice
// views of the gathered tensor become the parameters) and point 3 (tail
// padding when the count does not divide by the world size); "FSDP" (Latent
// Atlas) s5.1 (even, contiguous split); "03 - FSDP (ZeRO-3)" s1 and s3 (the
// all-gather result is copied out per parameter).
//
// Every kernel walks a contiguous range -- the flat buffer, the rank's shard,
// or the rank-major gather buffer -- in chunks, one chunk per workgroup
// iteration. The workgroup finds the parameters that overlap its chunk by
// binary search over the parameter offsets -- one-wave workgroups search the
// device table with wave-uniform scalar loads; wider ones, which every kernel
// can also be built for, stage the offsets in LDS -- then copies each overlap
// with 16-byte vectors. A bf16 copy whose source and destination sit at different
// offsets from the 16-byte grid is realigned in registers (each destination
// vector is funnel-shifted from two source vectors, the second taken from the
// neighbour lane), and the copy-outs move each chunk edge inside a piece to
// the destination's 16-byte grid so that only a piece's own ends go element by
// element; the pack's fp32-widening copy falls back to lane-contiguous element
// accesses there (still coalesced: 64 lanes touch 64 consecutive elements).
// Every access lies inside the parameter's own [0, numel) range, inside the
// flat or gather buffer, or inside the shard.
#include "zs_device.hpp"
#include "zs_launch.hpp"

namespace zs {
namespace {

// The copy-outs run one-wave workgroups over short chunks: many small
// workgroups keep more of the chip's memory pipeline busy than fewer large
// ones (a plain 2 GiB bf16 copy: 83% of peak with one 16-byte vector per lane
// and 1 KiB per workgroup, 77% with 256 lanes and 16 KiB), and in one wave the
// chunk's first parameter is found without LDS or barriers. Measured against
// 256 lanes over 8192 elements, in alternating rounds: the flat copy-out 2-4%
// faster with 2048-element chunks (a 2 GiB parameter, the Llama-3-8B and 70B
// blocks); the dim-0 copy-out 7% (Llama-3-8B block, N = 8), 12% (GPT-2,
// N = 8) and 1% (GPT-2, N = 5) faster with 1024-element chunks. Since the
// stores go out as global (not FLAT) stores, 1024-element chunks are also the
// best for the flat copy-out: 2.2-3.9% faster than 2048 on those blocks, the
// 2 GiB parameter and GPT-2's unit (512 elements: 6-35% slower).
constexpr int kCopyBS = 64;
constexpr int64_t kCopyChunk = 1024;
constexpr int64_t kCopyDim0Chunk = 1024;
constexpr int kLdsParams = 1024;   // offsets cached in LDS up to this many parameters
// The packs take one-wave workgroups as well (fp32 writes, 12 of their 16
// bytes per element). The flat pack works 1024-element chunks under a 12 KiB
// LDS reservation that holds it to 13 workgroups per CU: 6% faster than 256
// lanes over 8192 elements with 4 workgroups per CU on the 7.5B shard, 8% on
// GPT-2's shard at N = 5. The dim-0 pack works 256-element chunks at full
// residency: 13% faster on the Llama-3-8B block at N = 8 and on the 70B block
// at N = 64.
constexpr int kPackBS = 64;
constexpr int64_t kPackChunk = 1024;
constexpr unsigned kPackLds = 12288;
constexpr int64_t kPackDim0Chunk = 256;

// Largest p with off[p] <= f (off ascending, off[0] == 0 <= f).
__device__ __forceinline__ int find_param(const int64_t* off_lds, const zs_param_desc* desc,
                                          int nparams, bool use_lds, int64_t f) {
  int lo = 0, hi = nparams - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t o = use_lds ? off_lds[mid] : desc[mid].flat_offset;
    if (o <= f) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t h) { return bf16_to_f32(h); }

// 4 source elements -> one fp32 16-byte vector.
__device__ __forceinline__ f32x4 load4(const float* p) {
  return ld_nt(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ f32x4 load4(const uint16_t* p) {
  const u32x2 w = ld_nt(reinterpret_cast<const u32x2*>(p));
  return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
}

// Workgroup-cooperative copy of len elements src -> dst (fp32 destination).
template <typename Src, int BS = kThreads>
__device__ void seg_to_f32(const Src* __restrict__ src, float* __restrict__ dst, int64_t len) {
  const uintptr_t da = reinterpret_cast<uintptr_t>(dst);
  int64_t head = (int64_t)(((16u - (da & 15u)) & 15u) / 4u);
  if (head > len) head = len;
  const bool vec = (reinterpret_cast<uintptr_t>(src + head) & (4 * sizeof(Src) - 1)) == 0;
  if (!vec) {
    for (int64_t i = threadIdx.x; i < len; i += BS) st_g(widen(ld_g(src + i)), dst + i);
    return;
  }
  for (int64_t i = threadIdx.x; i < head; i += BS) st_g(widen(ld_g(src + i)), dst + i);
  const int64_t nv = (len - head) / 4;
  const Src* s = src + head;
  float* d = dst + head;
  for (int64_t i = threadIdx.x; i < nv; i += BS)
    st_nt(load4(s + 4 * i), reinterpret_cast<f32x4*>(d + 4 * i));
  for (int64_t i = head + 4 * nv + threadIdx.x; i < len; i += BS) st_g(widen(ld_g(src + i)), dst + i);
}

// Destination vectors [k_begin, k_end) of a bf16 copy whose source runs SH
// elements (1..7) past a 16-byte boundary when the destination sits on one:
// destination vector k takes elements SH + 8k .. SH + 8k + 7 of the aligned
// source vectors sa[k] and sa[k + 1]. Each lane loads its own sa[k] and gets
// sa[k + 1] from the next lane by a wave shuffle, then funnel-shifts the pair
// into one aligned store. Each lane keeps 4 source vectors in flight: with one
// at a time the realigning copy was bound by load latency.
// In one-wave workgroups lane 63's neighbour is lane 0 of the next group of
// 64 vectors, which the wave already holds, and the one vector after the last
// of a round is loaded together with the round by the lane that needs it, so a
// round costs one memory round trip. (Loading that vector after the shuffle,
// as wider workgroups still do, made every round wait for memory twice.)
// The caller keeps every loaded vector, sa[k_begin] .. sa[k_end], inside
// memory the copy may read: the copied range itself, or the same piece's
// elements around it (see seg_bf16).
template <int SH, int BS>
__device__ void realign_bf16(const u32x4* __restrict__ sa, u32x4* __restrict__ da, int64_t k_begin,
                             int64_t k_end) {
  constexpr int q = SH / 2;          // whole 32-bit words to skip
  constexpr bool half = (SH & 1) != 0;  // plus one bf16
  constexpr int U = 4;               // source vectors in flight per lane
  const int lane = threadIdx.x & 63;
  auto emit = [&](const u32x4& lo, const u32x4& hi, int64_t k) {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = half ? (w[q + t] >> 16) | (w[q + t + 1] << 16) : w[q + t];
    st_nt(o, da + k);
  };
  auto next_lane = [](const u32x4& x) {  // lane i receives lane i+1's vector
    return u32x4{(uint32_t)__shfl_down(x.x, 1, 64), (uint32_t)__shfl_down(x.y, 1, 64),
                 (uint32_t)__shfl_down(x.z, 1, 64), (uint32_t)__shfl_down(x.w, 1, 64)};
  };
  if constexpr (BS == 64) {
    for (int64_t kb = k_begin; kb < k_end; kb += U * 64) {
      const int64_t kx = kb + U * 64 < k_end ? kb + U * 64 : k_end;  // this round: [kb, kx)
      u32x4 lo[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t k = kb + (int64_t)j * 64 + lane;
        lo[j] = k < kx ? ld_nt(sa + k) : u32x4{0u, 0u, 0u, 0u};
      }
      // sa[kx], the neighbour of the round's last vector, by the lane holding it
      u32x4 ext{0u, 0u, 0u, 0u};
      if (lane == (int)((kx - 1 - kb) & 63)) ext = ld_nt(sa + kx);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t k = kb + (int64_t)j * 64 + lane;
        u32x4 hi = next_lane(lo[j]);
        if (j + 1 < U) {
          const u32x4 nx{(uint32_t)__shfl(lo[j + 1].x, 0, 64), (uint32_t)__shfl(lo[j + 1].y, 0, 64),
                         (uint32_t)__shfl(lo[j + 1].z, 0, 64), (uint32_t)__shfl(lo[j + 1].w, 0, 64)};
          if (lane == 63) hi = nx;
        }
        if (k >= kx) continue;
        if (k + 1 == kx) hi = ext;
        emit(lo[j], hi, k);
      }
    }
  } else {
    for (int64_t kb = k_begin; kb < k_end; kb += U * BS) {  // uniform across the workgroup
      u32x4 lo[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t k = kb + (int64_t)j * BS + threadIdx.x;
        lo[j] = k < k_end ? ld_nt(sa + k) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t k = kb + (int64_t)j * BS + threadIdx.x;
        u32x4 hi = next_lane(lo[j]);  // sa[k + 1]: the next lane's vector of the same round
        if (k >= k_end) continue;
        if (lane == 63 || k + 1 >= k_end) hi = ld_nt(sa + k + 1);
        emit(lo[j], hi, k);
      }
    }
  }
}

// Workgroup-cooperative copy of len bf16 elements. When source and destination
// reach the 16-byte grid at the same element, each lane issues two 16-byte
// loads before their stores (32 bytes in flight per lane instead of 16:
// measured 2.5% faster for both copy-outs; four or more were no better, and
// the fp32-widening copy above is fastest one vector at a time). Otherwise the
// destination vectors go through realign_bf16 and only the ends are copied
// element by element. Destination vector k reads the aligned source vectors
// that hold source elements head + 8k - sh .. head + 8k + 8; the first and the
// last destination vectors need one that reaches up to 7 elements before or
// after the range, which they read only when that stays inside the range or
// the caller allows it: `lead` / `trail` promise that at least 8 elements of
// the same piece precede src / follow src + len (an interior edge of a piece
// that a workgroup's chunk cuts). Otherwise those two vectors go element by
// element.
template <int BS>
__device__ void seg_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                         int64_t len, bool lead = false, bool trail = false) {
  static_assert(BS >= 16, "each lane copies at most one element of each end");
  const uintptr_t da = reinterpret_cast<uintptr_t>(dst);
  int64_t head = (int64_t)(((16u - (da & 15u)) & 15u) / 2u);
  if (head > len) head = len;
  const int sh = (int)((reinterpret_cast<uintptr_t>(src + head) & 15u) / 2u);
  // The ends that go element by element ([0, e0) and [e1, len), at most 15
  // elements each) are loaded before the vectors and stored after them, so
  // that their loads share the vectors' round trip to memory.
  auto ends = [&](int64_t e0, int64_t e1, auto&& vectors) {
    const int64_t t = threadIdx.x;
    const bool hl = t < e0, tl = e1 + t < len;
    uint16_t hv = 0, tv = 0;
    if (hl) hv = ld_g(src + t);
    if (tl) tv = ld_g(src + e1 + t);
    vectors();
    if (hl) st_g(hv, dst + t);
    if (tl) st_g(tv, dst + e1 + t);
  };
  if (sh != 0) {
    const int64_t nv = (len - head) / 8;  // destination vectors
    const int64_t kb = (lead || head >= sh) ? 0 : 1;                  // first realigned vector
    const int64_t ke = (trail || len - head - 8 * nv >= 8 - sh) ? nv : nv - 1;  // one past the last
    if (ke - kb < 1) {
      for (int64_t i = threadIdx.x; i < len; i += BS) st_g(ld_g(src + i), dst + i);
      return;
    }
    // element by element: the head (and destination vector 0 unless it is
    // realigned), then the last destination vector unless it is realigned,
    // and the tail
    const u32x4* sa = reinterpret_cast<const u32x4*>(src + head - sh);
    u32x4* dv = reinterpret_cast<u32x4*>(dst + head);
    ends(head + 8 * kb, head + 8 * ke, [&] {
      switch (sh) {
        case 1: realign_bf16<1, BS>(sa, dv, kb, ke); break;
        case 2: realign_bf16<2, BS>(sa, dv, kb, ke); break;
        case 3: realign_bf16<3, BS>(sa, dv, kb, ke); break;
        case 4: realign_bf16<4, BS>(sa, dv, kb, ke); break;
        case 5: realign_bf16<5, BS>(sa, dv, kb, ke); break;
        case 6: realign_bf16<6, BS>(sa, dv, kb, ke); break;
        default: realign_bf16<7, BS>(sa, dv, kb, ke); break;
      }
    });
    return;
  }
  const int64_t nv = (len - head) / 8;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + head);
  u32x4* d = reinterpret_cast<u32x4*>(dst + head);
  ends(head, head + 8 * nv, [&] {
    int64_t i = threadIdx.x;
    for (; i + BS < nv; i += 2 * BS) {
      const u32x4 a = ld_nt(s + i), b = ld_nt(s + i + BS);
      st_nt(a, d + i);
      st_nt(b, d + i + BS);
    }
    if (i < nv) st_nt(ld_nt(s + i), d + i);
  });
}

template <int BS = kThreads>
__device__ void zero_f32(float* __restrict__ p, int64_t len) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  int64_t head = (int64_t)(((16u - (a & 15u)) & 15u) / 4u);
  if (head > len) head = len;
  for (int64_t i = threadIdx.x; i < head; i += BS) st_g(0.0f, p + i);
  const int64_t nv = (len - head) / 4;
  f32x4* d = reinterpret_cast<f32x4*>(p + head);
  for (int64_t i = threadIdx.x; i < nv; i += BS) st_nt(f32x4{0.f, 0.f, 0.f, 0.f}, d + i);
  for (int64_t i = head + 4 * nv + threadIdx.x; i < len; i += BS) st_g(0.0f, p + i);
}

// Stage parameter offsets in LDS when the table fits (BS: the workgroup size).
template <int BS = kThreads>
__device__ bool stage_offsets(int64_t* off_lds, const zs_param_desc* desc, int nparams) {
  const bool use = nparams <= kLdsParams;
  if (use)
    for (int i = threadIdx.x; i < nparams; i += BS) off_lds[i] = desc[i].flat_offset;
  __syncthreads();
  return use;
}

// Flat range [f0, fe) -> inclusive parameter index range, shared through LDS.
__device__ void chunk_params(const int64_t* off_lds, const zs_param_desc* desc, int nparams,
                             bool use_lds, int64_t f0, int64_t fe, int* lo, int* hi) {
  __shared__ int s_lo, s_hi;
  if (threadIdx.x == 0) s_lo = find_param(off_lds, desc, nparams, use_lds, f0);
  if (threadIdx.x == 64) s_hi = find_param(off_lds, desc, nparams, use_lds, fe - 1);
  __syncthreads();
  *lo = __builtin_amdgcn_readfirstlane(s_lo);
  *hi = __builtin_amdgcn_readfirstlane(s_hi);
  __syncthreads();  // s_lo / s_hi are rewritten by the next chunk
}

// Largest p with key(p) <= f, every lane computing the same search: in a
// one-wave workgroup the indices are wave-uniform, so the table is read with
// scalar loads and no LDS staging or barrier is needed.
template <typename Key>
__device__ __forceinline__ int find_uniform(int nparams, int64_t f, Key key) {
  int lo = 0, hi = nparams - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key(mid) <= f) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The rank's slice [flat_begin, flat_begin + shard) of the padded flat unit,
// CH elements per workgroup iteration. One-wave workgroups (BS == 64) find the
// chunk's first parameter by a wave-uniform search (find_uniform); larger ones
// stage the offsets in LDS.
template <typename Src, int BS, int64_t CH>
__global__ __launch_bounds__(BS) void k_pack(const zs_param_desc* __restrict__ desc,
                                             int nparams, int64_t total, int64_t flat_begin,
                                             int64_t shard, float* __restrict__ master,
                                             float* __restrict__ m, float* __restrict__ v) {
  [[maybe_unused]] __shared__ int64_t off_lds[BS == 64 ? 1 : kLdsParams];
  bool use_lds = false;
  if constexpr (BS != 64) use_lds = nparams > 0 ? stage_offsets<BS>(off_lds, desc, nparams) : false;
  for (int64_t k0 = (int64_t)blockIdx.x * CH; k0 < shard; k0 += (int64_t)gridDim.x * CH) {
    const int64_t k1 = k0 + CH < shard ? k0 + CH : shard;
    const int64_t f0 = flat_begin + k0, f1 = flat_begin + k1;
    const int64_t fe = f1 < total ? f1 : total;  // end of real data inside the chunk
    if (m) zero_f32<BS>(m + k0, k1 - k0);
    if (v) zero_f32<BS>(v + k0, k1 - k0);
    auto part = [&](int p) {
      const int64_t off = desc[p].flat_offset, cnt = desc[p].numel;
      const int64_t a = f0 > off ? f0 : off;
      const int64_t b = fe < off + cnt ? fe : off + cnt;
      if (a >= b) return;
      const Src* src = static_cast<const Src*>(desc[p].ptr) + (a - off);
      seg_to_f32<Src, BS>(src, master + (a - flat_begin), b - a);
    };
    if (f0 < fe) {
      if constexpr (BS == 64) {
        for (int p = find_uniform(nparams, f0, [&](int i) { return desc[i].flat_offset; });
             p < nparams && desc[p].flat_offset < fe; ++p)
          part(p);
      } else {
        static_assert(BS >= 128, "chunk_params searches on threads 0 and 64");
        int lo, hi;
        chunk_params(off_lds, desc, nparams, use_lds, f0, fe, &lo, &hi);
        for (int p = lo; p <= hi; ++p) part(p);
      }
    }
    const int64_t z0 = f0 > total ? f0 : total;  // tail padding -> +0.0
    if (z0 < f1) zero_f32<BS>(master + (z0 - flat_begin), f1 - z0);
  }
}

// An edge f of a workgroup's part of a piece n elements long (in the piece's
// coordinates; destination element f at dst + f): an interior edge moves
// forward to the next element whose destination lies on the 16-byte grid, at
// most to n. The two workgroups that meet at f compute the same edge, so their
// parts still tile the piece, and neither writes half of a destination vector
// or copies elements one by one there.
__device__ __forceinline__ int64_t dst_edge(const uint16_t* dst, int64_t f, int64_t n) {
  if (f <= 0 || f >= n) return f;
  const int64_t adv = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(dst + f) & 15u)) & 15u) / 2u);
  return f + adv < n ? f + adv : n;
}

// The part [a, b) (flat coordinates) of parameter p that a workgroup copies,
// its edges moved by dst_edge.
template <int BS>
__device__ __forceinline__ void copy_param_part(const uint16_t* __restrict__ gathered,
                                                const zs_param_desc& d, int64_t a, int64_t b) {
  uint16_t* dp = static_cast<uint16_t*>(d.ptr);
  const int64_t xa = dst_edge(dp, a - d.flat_offset, d.numel), xb = dst_edge(dp, b - d.flat_offset, d.numel);
  if (xa < xb)
    seg_bf16<BS>(gathered + d.flat_offset + xa, dp + xa, xb - xa, xa >= 8, d.numel - xb >= 8);
}

// BS lanes copy chunks of CH elements of the flat range. One-wave workgroups
// (BS == 64) find the chunk's first parameter by a wave-uniform search and walk
// forward; larger ones stage the offsets in LDS and search behind barriers.
template <int BS, int64_t CH>
__global__ __launch_bounds__(BS) void k_copy_out(const uint16_t* __restrict__ gathered,
                                                 const zs_param_desc* __restrict__ desc,
                                                 int nparams, int64_t total) {
  if constexpr (BS == 64) {
    for (int64_t f0 = (int64_t)blockIdx.x * CH; f0 < total; f0 += (int64_t)gridDim.x * CH) {
      const int64_t fe = f0 + CH < total ? f0 + CH : total;
      const int lo = find_uniform(nparams, f0, [&](int i) { return desc[i].flat_offset; });
      for (int p = lo; p < nparams; ++p) {
        const zs_param_desc d = desc[p];
        if (d.flat_offset >= fe) break;
        const int64_t a = f0 > d.flat_offset ? f0 : d.flat_offset;
        const int64_t b = fe < d.flat_offset + d.numel ? fe : d.flat_offset + d.numel;
        if (a < b) copy_param_part<BS>(gathered, d, a, b);
      }
    }
  } else {
    static_assert(BS >= 128, "chunk_params searches on threads 0 and 64");
    __shared__ int64_t off_lds[kLdsParams];
    const bool use_lds = stage_offsets<BS>(off_lds, desc, nparams);
    for (int64_t f0 = (int64_t)blockIdx.x * CH; f0 < total; f0 += (int64_t)gridDim.x * CH) {
      const int64_t fe = f0 + CH < total ? f0 + CH : total;
      int lo, hi;
      chunk_params(off_lds, desc, nparams, use_lds, f0, fe, &lo, &hi);
      for (int p = lo; p <= hi; ++p) {
        const zs_param_desc d = desc[p];
        const int64_t a = f0 > d.flat_offset ? f0 : d.flat_offset;
        const int64_t b = fe < d.flat_offset + d.numel ? fe : d.flat_offset + d.numel;
        if (a < b) copy_param_part<BS>(gathered, d, a, b);
      }
    }
  }
}

// ---- per-parameter dim-0 sharding ------------------------------------------------

// Largest p with key(p) <= f over a table sorted by that key.
template <typename Key>
__device__ __forceinline__ int find_by(const int64_t* key_lds, bool use_lds, int nparams, int64_t f,
                                       Key key) {
  int lo = 0, hi = nparams - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t o = use_lds ? key_lds[mid] : key(mid);
    if (o <= f) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int64_t valid_part(const zs_dim0_desc& d, int rank) {
  const int64_t v = d.numel - (int64_t)rank * d.chunk;
  return v < 0 ? 0 : (v > d.chunk ? d.chunk : v);
}

// Rank r's shard: for each parameter its rows [r*c, (r+1)*c), zero past dim 0.
// Workgroup shapes as in k_pack.
template <typename Src, int BS, int64_t CH>
__global__ __launch_bounds__(BS) void k_pack_dim0(const zs_dim0_desc* __restrict__ desc,
                                                  int nparams, int rank, int64_t local_total,
                                                  float* __restrict__ master,
                                                  float* __restrict__ m,
                                                  float* __restrict__ v) {
  auto lkey = [&](int i) { return desc[i].local_offset; };
  [[maybe_unused]] __shared__ int64_t key[BS == 64 ? 1 : kLdsParams];
  [[maybe_unused]] __shared__ int s_lo, s_hi;
  const bool use_lds = BS != 64 && nparams <= kLdsParams;
  if constexpr (BS != 64) {
    if (use_lds)
      for (int i = threadIdx.x; i < nparams; i += BS) key[i] = desc[i].local_offset;
    __syncthreads();
  }
  for (int64_t k0 = (int64_t)blockIdx.x * CH; k0 < local_total; k0 += (int64_t)gridDim.x * CH) {
    const int64_t k1 = k0 + CH < local_total ? k0 + CH : local_total;
    if (m) zero_f32<BS>(m + k0, k1 - k0);
    if (v) zero_f32<BS>(v + k0, k1 - k0);
    auto part = [&](int p) {
      const zs_dim0_desc d = desc[p];
      const int64_t a = k0 > d.local_offset ? k0 : d.local_offset;
      const int64_t b = k1 < d.local_offset + d.chunk ? k1 : d.local_offset + d.chunk;
      if (a >= b) return;
      const int64_t ja = a - d.local_offset, jb = b - d.local_offset;  // within the chunk
      const int64_t val = valid_part(d, rank);
      const int64_t je = jb < val ? jb : val;  // real rows end
      if (ja < je)
        seg_to_f32<Src, BS>(static_cast<const Src*>(d.ptr) + (int64_t)rank * d.chunk + ja, master + a,
                            je - ja);
      const int64_t z0 = ja > val ? ja : val;  // padding rows
      if (z0 < jb) zero_f32<BS>(master + d.local_offset + z0, jb - z0);
    };
    if constexpr (BS == 64) {
      for (int p = find_uniform(nparams, k0, lkey); p < nparams && desc[p].local_offset < k1; ++p) part(p);
    } else {
      static_assert(BS >= 128, "the piece search runs on threads 0 and 64");
      if (threadIdx.x == 0) s_lo = find_by(key, use_lds, nparams, k0, lkey);
      if (threadIdx.x == 64) s_hi = find_by(key, use_lds, nparams, k1 - 1, lkey);
      __syncthreads();
      const int lo = __builtin_amdgcn_readfirstlane(s_lo), hi = __builtin_amdgcn_readfirstlane(s_hi);
      __syncthreads();
      for (int p = lo; p <= hi; ++p) part(p);
    }
  }
}

// Full parameters from the rank-major gathered buffer [N * L]. The workgroups
// walk the gathered buffer in order (one compact read window; walking the
// parameters in order instead reads N windows at once and measured 2-9%
// slower) and scatter each piece -- rank r's part of one parameter's chunk --
// to that parameter's rows [r*c, r*c + valid). Padding rows are not copied.
// Workgroup shapes as in k_copy_out.
template <int BS, int64_t CH>
__global__ __launch_bounds__(BS) void k_copy_out_dim0(const uint16_t* __restrict__ gathered,
                                                      const zs_dim0_desc* __restrict__ desc,
                                                      int nparams, int world,
                                                      int64_t local_total) {
  auto piece = [&](int p, int64_t r, int64_t j0, int64_t j1) {  // rank r's [j0, j1) of parameter p
    const zs_dim0_desc d = desc[p];
    const int64_t a = j0 > d.local_offset ? j0 : d.local_offset;
    const int64_t b = j1 < d.local_offset + d.chunk ? j1 : d.local_offset + d.chunk;
    if (a >= b) return;
    const int64_t ja = a - d.local_offset, jb = b - d.local_offset;  // within the chunk
    const int64_t val = valid_part(d, (int)r);
    const int64_t je = jb < val ? jb : val;  // real rows end
    if (ja >= je) return;
    uint16_t* dp = static_cast<uint16_t*>(d.ptr) + r * d.chunk;  // the piece: val elements
    const int64_t xa = dst_edge(dp, ja, val), xb = dst_edge(dp, je, val);
    if (xa < xb)
      seg_bf16<BS>(gathered + r * local_total + d.local_offset + xa, dp + xa, xb - xa, xa >= 8,
                   val - xb >= 8);
  };
  const int64_t src_total = (int64_t)world * local_total;
  if constexpr (BS == 64) {
    auto lkey = [&](int i) { return desc[i].local_offset; };
    for (int64_t g0 = (int64_t)blockIdx.x * CH; g0 < src_total; g0 += (int64_t)gridDim.x * CH) {
      const int64_t ge = g0 + CH < src_total ? g0 + CH : src_total;
      for (int64_t gp = g0; gp < ge;) {  // the chunk's pieces inside one rank's shard
        const int64_t r = gp / local_total;
        const int64_t rend = (r + 1) * local_total < ge ? (r + 1) * local_total : ge;
        const int64_t j0 = gp - r * local_total, j1 = rend - r * local_total;
        for (int p = find_uniform(nparams, j0, lkey); p < nparams && desc[p].local_offset < j1; ++p)
          piece(p, r, j0, j1);
        gp = rend;
      }
    }
  } else {
    static_assert(BS >= 128, "the piece search runs on threads 0 and 64");
    __shared__ int64_t key[kLdsParams];
    __shared__ int s_lo, s_hi;
    const bool use_lds = nparams <= kLdsParams;
    if (use_lds)
      for (int i = threadIdx.x; i < nparams; i += BS) key[i] = desc[i].local_offset;
    __syncthreads();
    auto lkey = [&](int i) { return desc[i].local_offset; };
    for (int64_t g0 = (int64_t)blockIdx.x * CH; g0 < src_total; g0 += (int64_t)gridDim.x * CH) {
      const int64_t ge = g0 + CH < src_total ? g0 + CH : src_total;
      int64_t gp = g0;
      while (gp < ge) {  // the chunk's pieces inside one rank's shard (uniform loop)
        const int64_t r = gp / local_total;
        const int64_t rend = (r + 1) * local_total < ge ? (r + 1) * local_total : ge;
        const int64_t j0 = gp - r * local_total, j1 = rend - r * local_total;
        if (threadIdx.x == 0) s_lo = find_by(key, use_lds, nparams, j0, lkey);
        if (threadIdx.x == 64) s_hi = find_by(key, use_lds, nparams, j1 - 1, lkey);
        __syncthreads();
        const int lo = __builtin_amdgcn_readfirstlane(s_lo), hi = __builtin_amdgcn_readfirstlane(s_hi);
        __syncthreads();
        for (int p = lo; p <= hi; ++p) piece(p, r, j0, j1);
        gp = rend;
      }
    }
  }
}

}  // namespace

hipError_t launch_pack(const zs_param_desc* d_desc, int nparams, int64_t total, int src_dtype,
                       int64_t flat_begin, int64_t shard, float* master, float* m, float* v,
                       hipStream_t s) {
  if (shard == 0) return hipSuccess;
  constexpr int BS = kPackBS;
  constexpr int64_t CH = kPackChunk;
  const dim3 gd((unsigned)grid_for(shard, CH, BS)), bd(BS);
  if (src_dtype == ZS_BF16)
    hipLaunchKernelGGL((k_pack<uint16_t, BS, CH>), gd, bd, kPackLds, s, d_desc, nparams, total,
                       flat_begin, shard, master, m, v);
  else
    hipLaunchKernelGGL((k_pack<float, BS, CH>), gd, bd, kPackLds, s, d_desc, nparams, total,
                       flat_begin, shard, master, m, v);
  return hipGetLastError();
}

hipError_t launch_pack_dim0(const zs_dim0_desc* d_desc, int nparams, int src_dtype, int rank,
                            int64_t local_total, float* master, float* m, float* v, hipStream_t s) {
  if (local_total == 0) return hipSuccess;
  constexpr int BS = kPackBS;
  constexpr int64_t CH = kPackDim0Chunk;
  const dim3 gd((unsigned)grid_for(local_total, CH, BS)), bd(BS);
  if (src_dtype == ZS_BF16)
    hipLaunchKernelGGL((k_pack_dim0<uint16_t, BS, CH>), gd, bd, 0, s, d_desc, nparams, rank,
                       local_total, master, m, v);
  else
    hipLaunchKernelGGL((k_pack_dim0<float, BS, CH>), gd, bd, 0, s, d_desc, nparams, rank,
                       local_total, master, m, v);
  return hipGetLastError();
}

hipError_t launch_copy_out_dim0(const uint16_t* gathered, const zs_dim0_desc* d_desc, int nparams,
                                int world, int64_t total, int64_t local_total, hipStream_t s) {
  if (total == 0) return hipSuccess;
  constexpr int BS = kCopyBS;
  constexpr int64_t CH = kCopyDim0Chunk;
  hipLaunchKernelGGL((k_copy_out_dim0<BS, CH>), dim3((unsigned)grid_for((int64_t)world * local_total, CH, BS)),
                     dim3(BS), 0, s, gathered, d_desc, nparams, world, local_total);
  return hipGetLastError();
}

hipError_t launch_copy_out(const uint16_t* gathered, const zs_param_desc* d_desc, int nparams,
                           int64_t total, hipStream_t s) {
  if (total == 0 || nparams == 0) return hipSuccess;
  constexpr int BS = kCopyBS;
  constexpr int64_t CH = kCopyChunk;
  hipLaunchKernelGGL((k_copy_out<BS, CH>), dim3((unsigned)grid_for(total, CH, BS)), dim3(BS), 0, s,
                     gathered, d_desc, nparams, total);
  return hipGetLastError();
}

}  // namespace zs
