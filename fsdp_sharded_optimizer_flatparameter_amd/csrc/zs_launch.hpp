// Host-side launchers of the zs kernels (internal to libzs; the public surface is zs.h).
// Each launcher assumes its arguments were validated by the C-ABI entry point.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zs.h"

namespace zs {

struct AdamConsts;

// Launch-shape knobs. Defaults are the measured best on MI355X; each can be
// overridden once per process through the environment (ZS_ADAMW_V,
// ZS_ADAMW_LDS, ZS_RANK_CHUNK, ZS_FUSED_G,
// ZS_FUSED_LDS, ZS_FUSED_BS, ZS_ACCUM_SHAPE, ZS_REDUCE_G, ZS_GRID_CAP) for sweeps. None of them changes any result.
struct Tuning {
  int adamw_v;     // 16-byte groups per lane per tile in AdamW (1, 2 or 4)
  int64_t adamw_lds;  // LDS bytes reserved per AdamW workgroup (caps residency)
  int rank_chunk;  // ranks per load chunk of the double-buffered rank walk (4 or 8)
  int fused_g;     // groups per lane staged in LDS by the single-pass kernel (0 = by world size)
  int64_t fused_lds;  // LDS bytes reserved per workgroup of the single-pass kernel (0 = default)
  int fused_bs;    // workgroup size of the single-pass kernel (64, 256, or 512 = the
                   // rank-major shape; 0 = by world size)
  int accum_shape;  // ZeRO-2 accumulation with few contributions: 0 one-wave, 1 four-wave
  int reduce_g;    // groups per lane staged in LDS by the reduce kernel (0 = by world size)
  int64_t grid_cap;  // upper bound on workgroups of the streaming kernels
};
const Tuning& tuning();

// Workgroups of a streaming launch over `units` work items, `per_block` per
// workgroup of `threads` lanes, capped by the grid cap and by the 32-bit
// work-item count of a dispatch (the kernels grid-stride past the cap).
inline int64_t grid_for(int64_t units, int64_t per_block, int64_t threads = 256) {
  int64_t g = (units + per_block - 1) / per_block;
  const int64_t hard = (int64_t)0xffffffff / threads;
  if (g > hard) g = hard;
  if (g > tuning().grid_cap) g = tuning().grid_cap;
  return g < 1 ? 1 : g;
}

// The tiles of one launch of a streaming kernel over `ngroups` lane groups.
// Tiles [0, nfull) cover `span` groups each (the last of them clipped at
// ngroups); the groups after them -- `units` units of 64, the last one clipped
// -- are split evenly over tiles [nfull, nfull + nlast). Tile t is handled by
// workgroup t mod gridDim.x.
struct TilePlan {
  int64_t span;
  int64_t nfull;
  int64_t units;
  int64_t nlast;
  __host__ __device__ int64_t count() const { return nfull + nlast; }
  // Groups [*b, *e) of tile t < count(); never empty.
  __host__ __device__ void range(int64_t t, int64_t ngroups, int64_t* b, int64_t* e) const {
    if (t < nfull) {
      *b = t * span;
      *e = *b + span < ngroups ? *b + span : ngroups;
      return;
    }
    const int64_t o = nfull * span, j = t - nfull;
    *b = o + 64 * (j * units / nlast);
    const int64_t hi = o + 64 * ((j + 1) * units / nlast);
    *e = hi < ngroups ? hi : ngroups;
  }
};

// One tile per `span` groups.
inline TilePlan plain_tiles(int64_t ngroups, int64_t span) {
  return TilePlan{span, (ngroups + span - 1) / span, 0, 0};
}

// Tiles for a launch whose workgroups all take about the same time per group,
// `slots` of them resident on the device at once: every round but the last
// runs full tiles, and the groups of the last round are spread over all
// `slots` workgroups (at least 64 groups each) instead of leaving the rest of
// the device idle while a partly filled round finishes. The rank walks with
// 16-group tiles, one 8-wave workgroup per CU, ran 1.3-1.8% slower per element
// at 16.4, 13.5 and 14.5 rounds than at 16, 13 and 14 (fp32 rows at N=64, the
// 70B chunk; bf16 rows at N=64).
inline TilePlan balanced_tiles(int64_t ngroups, int64_t span, int64_t slots) {
  if (slots <= 0 || ngroups <= 0) return plain_tiles(ngroups, span);
  const int64_t tiles = (ngroups + span - 1) / span;
  const int64_t rounds = (tiles + slots - 1) / slots;
  TilePlan p;
  p.span = span;
  p.nfull = (rounds - 1) * slots;  // nfull * span < ngroups: the last round is not empty
  p.units = (ngroups - p.nfull * span + 63) / 64;
  p.nlast = p.units < slots ? p.units : slots;
  return p;
}

// Workgroups of `kernel` (bs lanes, lds bytes of dynamic LDS) that the device
// of stream s (the current device for the null stream) holds at once: its
// compute units times the kernel's occupancy per CU. Looked up once per
// device and kernel; 0 where the runtime cannot say.
int64_t device_slots(hipStream_t s, const void* kernel, int bs, size_t lds);

inline bool aligned_to(const void* p, unsigned a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Largest number of first-level partial sums a sum-of-squares launch over n
// elements writes (one per tile of at least 256 elements, capped); the
// workspace holds that many doubles plus kFinalizeBlocks.
int64_t max_partials(int64_t n);
// Second-level partials the sum-of-squares finalize may use, stored after the
// first-level ones in the caller's workspace.
constexpr int64_t kFinalizeBlocks = 256;

// First-level partials the library's own scratch holds (zs_reduce_grads_noalloc):
// one per 256 elements of the largest shard it accepts with a sum of squares.
constexpr int64_t kStaticPartials = ZS_NOALLOC_MAX_N / 256;
static_assert(ZS_NOALLOC_MAX_N % 256 == 0, "whole tiles");

// Device address of that scratch on the device of stream `s` (the current
// device for the null stream), looked up once per device; allocates nothing.
hipError_t static_partials(hipStream_t s, double** out);

// Deterministic fp64 sum of partials[0, count) into *out: one workgroup for a
// short list, else kFinalizeBlocks workgroups over fixed contiguous ranges
// (their sums go to partials[count, count + kFinalizeBlocks)) and a second pass.
hipError_t launch_sumsq_finalize(double* partials, int64_t count, double* out, hipStream_t s);

AdamConsts adam_consts(const zs_adamw_hparams& hp);

hipError_t launch_reduce(const void* const* rows, int world, int dtype, int64_t n, float* g,
                         double* sumsq, double* partials, hipStream_t s);

hipError_t launch_adamw(float* th, float* m, float* v, const float* g, int64_t n,
                        const zs_adamw_hparams& hp, const float* scale, uint16_t* out,
                        hipStream_t s);

hipError_t launch_cast(const float* src, int64_t n, uint16_t* out, hipStream_t s);

hipError_t launch_fused(const void* const* rows, int world, int dtype, int64_t n, float* th,
                        float* m, float* v, const zs_adamw_hparams& hp, const float* scale,
                        uint16_t* out, hipStream_t s);

hipError_t launch_accumulate(const void* const* rows, int world, int dtype, int64_t n, float* acc,
                             float scale, bool first, double* sumsq, double* partials,
                             hipStream_t s);

hipError_t launch_accumulate_local(const void* g, int dtype, int64_t n, float* acc, bool first,
                                   hipStream_t s);

hipError_t launch_clip(const double* partials, int count, double max_norm, float* coef,
                       double* norm, hipStream_t s);

hipError_t launch_pack(const zs_param_desc* d_desc, int nparams, int64_t total, int src_dtype,
                       int64_t flat_begin, int64_t shard, float* master, float* m, float* v,
                       hipStream_t s);

hipError_t launch_pack_dim0(const zs_dim0_desc* d_desc, int nparams, int src_dtype, int rank,
                            int64_t local_total, float* master, float* m, float* v, hipStream_t s);

hipError_t launch_copy_out_dim0(const uint16_t* gathered, const zs_dim0_desc* d_desc, int nparams,
                                int world, int64_t total, int64_t local_total, hipStream_t s);

hipError_t launch_copy_out(const uint16_t* gathered, const zs_param_desc* d_desc, int nparams,
                           int64_t total, hipStream_t s);

}  // namespace zs
