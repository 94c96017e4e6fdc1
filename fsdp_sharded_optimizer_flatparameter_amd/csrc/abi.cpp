// extern "C" entry points of libzs: argument validation on the host, then the
// launchers. Nothing here allocates memory or keeps state between calls.
#include <cmath>
#include <cstdint>

#include "zs.h"
#include "zs_launch.hpp"

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a+na) and [b, b+nb) (bytes) intersect?
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

inline int64_t elem_size(int32_t dtype) { return dtype == ZS_BF16 ? 2 : 4; }

zs_status check_hparams(const zs_adamw_hparams* hp) {
  if (!hp) return ZS_ERR_NULL;
  const double v[5] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  for (double x : v)
    if (!std::isfinite(x)) return ZS_ERR_HPARAM;
  if (hp->lr < 0 || hp->eps < 0 || hp->weight_decay < 0) return ZS_ERR_HPARAM;
  if (!(hp->beta1 >= 0 && hp->beta1 < 1) || !(hp->beta2 >= 0 && hp->beta2 < 1)) return ZS_ERR_HPARAM;
  if (hp->step < 1) return ZS_ERR_HPARAM;
  return ZS_OK;
}

zs_status check_rows(const void* const* rows, int32_t world, int32_t dtype, int64_t n) {
  if (world < 1 || world > ZS_MAX_WORLD) return ZS_ERR_WORLD;
  if (dtype != ZS_F32 && dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (n < 0) return ZS_ERR_SIZE;
  if (n == 0) return ZS_OK;  // nothing is read: rows (and their entries) may be NULL
  if (!rows) return ZS_ERR_NULL;
  for (int32_t q = 0; q < world; ++q) {
    if (!rows[q]) return ZS_ERR_NULL;
    if (!aligned(rows[q], (uintptr_t)elem_size(dtype))) return ZS_ERR_ALIGN;
  }
  return ZS_OK;
}

// Device work goes through launch(): a HIP error already pending on this thread
// (left by an earlier, unrelated call) is handed back as ZS_ERR_HIP before
// anything is enqueued, and stays pending for the caller; otherwise the status
// is that of this call's own launches.
template <typename F>
zs_status launch(F&& f) {
  if (hipPeekAtLastError() != hipSuccess) return ZS_ERR_HIP;
  return f() == hipSuccess ? ZS_OK : ZS_ERR_HIP;
}

// The sum of squares' workspace and result are written while the rows are read
// and `out` (n fp32) is written: none of them may share bytes.
zs_status check_sumsq_buffers(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                              const void* out, const void* sumsq, const void* ws, size_t ws_bytes) {
  const int64_t wb = (int64_t)ws_bytes;
  if (overlaps(sumsq, 8, ws, wb) || overlaps(sumsq, 8, out, n * 4) || overlaps(ws, wb, out, n * 4))
    return ZS_ERR_OVERLAP;
  for (int32_t q = 0; q < world && n > 0; ++q) {
    const int64_t rb = n * elem_size(dtype);
    if (overlaps(rows[q], rb, sumsq, 8) || overlaps(rows[q], rb, ws, wb)) return ZS_ERR_OVERLAP;
  }
  return ZS_OK;
}

// The gradient scale is read by every workgroup while the state is written.
bool scale_overlaps(const float* scale, const void* a, const void* b, const void* c, int64_t n,
                    const void* bf16_out) {
  return scale && (overlaps(scale, 4, a, n * 4) || overlaps(scale, 4, b, n * 4) ||
                   overlaps(scale, 4, c, n * 4) || (bf16_out && overlaps(scale, 4, bf16_out, n * 2)));
}

}  // namespace

extern "C" {

int32_t zs_version(void) { return 100; /* 0.1.0 */ }

const char* zs_status_string(zs_status s) {
  switch (s) {
    case ZS_OK: return "ZS_OK";
    case ZS_ERR_NULL: return "ZS_ERR_NULL";
    case ZS_ERR_SIZE: return "ZS_ERR_SIZE";
    case ZS_ERR_WORLD: return "ZS_ERR_WORLD";
    case ZS_ERR_RANK: return "ZS_ERR_RANK";
    case ZS_ERR_DTYPE: return "ZS_ERR_DTYPE";
    case ZS_ERR_HPARAM: return "ZS_ERR_HPARAM";
    case ZS_ERR_SHARD: return "ZS_ERR_SHARD";
    case ZS_ERR_WORKSPACE: return "ZS_ERR_WORKSPACE";
    case ZS_ERR_LAYOUT: return "ZS_ERR_LAYOUT";
    case ZS_ERR_ALIGN: return "ZS_ERR_ALIGN";
    case ZS_ERR_OVERLAP: return "ZS_ERR_OVERLAP";
    case ZS_ERR_HIP: return "ZS_ERR_HIP";
    default: return "ZS_ERR_UNKNOWN";
  }
}

// S of a unit of t elements over `world` ranks: ceil(t / world) rounded up to a
// multiple of `align`; ZS_ERR_SIZE when it or S * world overflows int64.
static zs_status shard_length(int64_t t, int32_t world, int64_t align, int64_t* s_out) {
  int64_t s = t / world + (t % world != 0);
  if (align > 1) {
    if (s > INT64_MAX - (align - 1)) return ZS_ERR_SIZE;
    s = (s + align - 1) / align * align;
  }
  if (s > INT64_MAX / world) return ZS_ERR_SIZE;
  *s_out = s;
  return ZS_OK;
}

zs_status zs_flat_layout(const int64_t* numels, int32_t nparams, int32_t world, int64_t align,
                         int64_t* offsets_out, int64_t* total_out, int64_t* padded_out,
                         int64_t* shard_out) {
  if (nparams < 0 || align < 1) return ZS_ERR_SIZE;
  if (world < 1) return ZS_ERR_WORLD;
  if (nparams > 0 && !numels) return ZS_ERR_NULL;
  int64_t t = 0;
  for (int32_t i = 0; i < nparams; ++i) {
    if (numels[i] < 0) return ZS_ERR_SIZE;
    if (numels[i] > INT64_MAX - t) return ZS_ERR_SIZE;
    t += numels[i];
  }
  int64_t s = 0;
  if (const zs_status st = shard_length(t, world, align, &s)) return st;
  if (offsets_out) {
    int64_t run = 0;
    for (int32_t i = 0; i < nparams; ++i) {
      offsets_out[i] = run;
      run += numels[i];
    }
  }
  if (total_out) *total_out = t;
  if (padded_out) *padded_out = s * world;
  if (shard_out) *shard_out = s;
  return ZS_OK;
}

zs_status zs_check_layout(const zs_param_desc* host_desc, int32_t nparams, int64_t total,
                          int32_t dtype) {
  if (dtype != ZS_F32 && dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (nparams < 0 || total < 0) return ZS_ERR_SIZE;
  if (nparams == 0) return total == 0 ? ZS_OK : ZS_ERR_LAYOUT;
  if (!host_desc) return ZS_ERR_NULL;
  int64_t run = 0;
  for (int32_t i = 0; i < nparams; ++i) {
    const zs_param_desc& d = host_desc[i];
    if (d.numel < 0) return ZS_ERR_SIZE;
    if (d.flat_offset != run) return ZS_ERR_LAYOUT;
    if (d.numel > 0 && !d.ptr) return ZS_ERR_NULL;
    if (d.numel > 0 && !aligned(d.ptr, (uintptr_t)elem_size(dtype))) return ZS_ERR_ALIGN;
    if (d.numel > INT64_MAX - run) return ZS_ERR_SIZE;
    run += d.numel;
  }
  return run == total ? ZS_OK : ZS_ERR_LAYOUT;
}

size_t zs_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return (size_t)(zs::max_partials(n) + zs::kFinalizeBlocks) * sizeof(double);
}

zs_status zs_pack_shard(const zs_param_desc* d_desc, int32_t nparams, int64_t total_numel,
                        int32_t src_dtype, int32_t world, int32_t rank, int64_t align,
                        int64_t shard_numel, float* master, float* exp_avg, float* exp_avg_sq,
                        hipStream_t stream) {
  if (nparams < 0 || total_numel < 0 || shard_numel < 0 || align < 1) return ZS_ERR_SIZE;
  if (nparams == 0 && total_numel != 0) return ZS_ERR_SIZE;
  if (world < 1) return ZS_ERR_WORLD;
  if (rank < 0 || rank >= world) return ZS_ERR_RANK;
  if (src_dtype != ZS_F32 && src_dtype != ZS_BF16) return ZS_ERR_DTYPE;
  int64_t s = 0;
  if (const zs_status st = shard_length(total_numel, world, align, &s)) return st;
  if (shard_numel != s) return ZS_ERR_SHARD;
  if (shard_numel == 0) return ZS_OK;
  if (!master || (nparams > 0 && !d_desc)) return ZS_ERR_NULL;
  if (!aligned(master, 4) || (exp_avg && !aligned(exp_avg, 4)) ||
      (exp_avg_sq && !aligned(exp_avg_sq, 4)) || !aligned(d_desc, 8))
    return ZS_ERR_ALIGN;
  const int64_t b = shard_numel * 4;
  if (overlaps(master, b, exp_avg, exp_avg ? b : 0) ||
      overlaps(master, b, exp_avg_sq, exp_avg_sq ? b : 0) ||
      overlaps(exp_avg, exp_avg ? b : 0, exp_avg_sq, exp_avg_sq ? b : 0))
    return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_pack(d_desc, nparams, total_numel, src_dtype,
                                    (int64_t)rank * shard_numel, shard_numel, master, exp_avg,
                                    exp_avg_sq, stream); });
}

zs_status zs_reduce_grads(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                          float* grad_out, double* sumsq_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  zs_status st = check_rows(rows, world, dtype, n);
  if (st != ZS_OK) return st;
  if (n > 0 && !grad_out) return ZS_ERR_NULL;
  if (grad_out && !aligned(grad_out, 4)) return ZS_ERR_ALIGN;
  if (sumsq_out) {
    if (!aligned(sumsq_out, 8)) return ZS_ERR_ALIGN;
    if (!workspace || workspace_bytes < zs_workspace_bytes(n)) return ZS_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return ZS_ERR_ALIGN;
    st = check_sumsq_buffers(rows, world, dtype, n, grad_out, sumsq_out, workspace, workspace_bytes);
    if (st != ZS_OK) return st;
  }
  if (n == 0) {
    if (!sumsq_out) return ZS_OK;
    // an empty shard's sum of squares is 0; written by the finalize kernel
    return launch([&] { return zs::launch_reduce(rows, world, dtype, 0, grad_out, sumsq_out,
                                        static_cast<double*>(workspace), stream); });
  }
  for (int32_t q = 0; q < world; ++q)
    if (overlaps(grad_out, n * 4, rows[q], n * elem_size(dtype))) return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_reduce(rows, world, dtype, n, grad_out, sumsq_out,
                                      static_cast<double*>(workspace), stream); });
}

zs_status zs_reduce_grads_noalloc(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                                  float* grad_out, double* sumsq_out, hipStream_t stream) {
  zs_status st = check_rows(rows, world, dtype, n);
  if (st != ZS_OK) return st;
  if (n > 0 && !grad_out) return ZS_ERR_NULL;
  if (grad_out && !aligned(grad_out, 4)) return ZS_ERR_ALIGN;
  if (sumsq_out) {
    if (n > ZS_NOALLOC_MAX_N) return ZS_ERR_WORKSPACE;  // beyond the library's scratch
    if (!aligned(sumsq_out, 8)) return ZS_ERR_ALIGN;
    st = check_sumsq_buffers(rows, world, dtype, n, grad_out, sumsq_out, nullptr, 0);
    if (st != ZS_OK) return st;
  }
  if (n == 0 && !sumsq_out) return ZS_OK;
  for (int32_t q = 0; q < world && n > 0; ++q)
    if (overlaps(grad_out, n * 4, rows[q], n * elem_size(dtype))) return ZS_ERR_OVERLAP;
  return launch([&] {
    double* partials = nullptr;
    if (sumsq_out) {
      const hipError_t e = zs::static_partials(stream, &partials);
      if (e != hipSuccess) return e;
    }
    return zs::launch_reduce(rows, world, dtype, n, grad_out, sumsq_out, partials, stream);
  });
}

zs_status zs_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, const float* grad,
                        int64_t n, const zs_adamw_hparams* hp, const float* grad_scale,
                        uint16_t* bf16_out, hipStream_t stream) {
  if (n < 0) return ZS_ERR_SIZE;
  zs_status st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (n == 0) return ZS_OK;
  if (!master || !exp_avg || !exp_avg_sq || !grad) return ZS_ERR_NULL;
  if (!aligned(master, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) ||
      !aligned(grad, 4) || (bf16_out && !aligned(bf16_out, 2)) ||
      (grad_scale && !aligned(grad_scale, 4)))
    return ZS_ERR_ALIGN;
  const int64_t b = n * 4;
  if (overlaps(master, b, exp_avg, b) || overlaps(master, b, exp_avg_sq, b) ||
      overlaps(exp_avg, b, exp_avg_sq, b) || overlaps(grad, b, master, b) ||
      overlaps(grad, b, exp_avg, b) || overlaps(grad, b, exp_avg_sq, b))
    return ZS_ERR_OVERLAP;
  if (bf16_out && (overlaps(bf16_out, n * 2, master, b) || overlaps(bf16_out, n * 2, exp_avg, b) ||
                   overlaps(bf16_out, n * 2, exp_avg_sq, b) || overlaps(bf16_out, n * 2, grad, b)))
    return ZS_ERR_OVERLAP;
  if (scale_overlaps(grad_scale, master, exp_avg, exp_avg_sq, n, bf16_out)) return ZS_ERR_OVERLAP;
  return launch([&] {
    return zs::launch_adamw(master, exp_avg, exp_avg_sq, grad, n, *hp, grad_scale, bf16_out, stream);
  });
}

zs_status zs_cast_for_gather(const float* master, int64_t n, uint16_t* gather_slot,
                             hipStream_t stream) {
  if (n < 0) return ZS_ERR_SIZE;
  if (n == 0) return ZS_OK;
  if (!master || !gather_slot) return ZS_ERR_NULL;
  if (!aligned(master, 4) || !aligned(gather_slot, 2)) return ZS_ERR_ALIGN;
  if (overlaps(master, n * 4, gather_slot, n * 2)) return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_cast(master, n, gather_slot, stream); });
}

zs_status zs_copy_out(const uint16_t* gathered, int64_t gathered_numel, const zs_param_desc* d_desc,
                      int32_t nparams, int64_t total_numel, hipStream_t stream) {
  if (nparams < 0 || total_numel < 0 || gathered_numel < 0) return ZS_ERR_SIZE;
  if (total_numel > gathered_numel) return ZS_ERR_SIZE;
  if (nparams == 0 && total_numel != 0) return ZS_ERR_SIZE;
  if (total_numel == 0) return ZS_OK;
  if (!gathered || !d_desc) return ZS_ERR_NULL;
  if (!aligned(gathered, 2) || !aligned(d_desc, 8)) return ZS_ERR_ALIGN;
  return launch([&] { return zs::launch_copy_out(gathered, d_desc, nparams, total_numel, stream); });
}

zs_status zs_dim0_layout(const int64_t* dim0, const int64_t* rowsize, int32_t nparams, int32_t world,
                         int64_t* chunk_out, int64_t* local_offsets_out, int64_t* local_total_out) {
  if (nparams < 0) return ZS_ERR_SIZE;
  if (world < 1) return ZS_ERR_WORLD;
  if (nparams > 0 && (!dim0 || !rowsize)) return ZS_ERR_NULL;
  int64_t t = 0;
  for (int32_t i = 0; i < nparams; ++i) {
    if (dim0[i] < 0 || rowsize[i] < 0) return ZS_ERR_SIZE;
    const int64_t rows = dim0[i] / world + (dim0[i] % world != 0);
    if (rowsize[i] > 0 && rows > INT64_MAX / world / rowsize[i]) return ZS_ERR_SIZE;
    const int64_t c = rows * rowsize[i];
    if (c > INT64_MAX - t) return ZS_ERR_SIZE;
    if (chunk_out) chunk_out[i] = c;
    if (local_offsets_out) local_offsets_out[i] = t;
    t += c;
  }
  if (local_total_out) *local_total_out = t;
  return ZS_OK;
}

zs_status zs_check_dim0_layout(const zs_dim0_desc* host_desc, int32_t nparams, int32_t world,
                               int64_t total, int64_t local_total, int32_t dtype) {
  if (dtype != ZS_F32 && dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (nparams < 0 || total < 0 || local_total < 0) return ZS_ERR_SIZE;
  if (world < 1) return ZS_ERR_WORLD;
  if (nparams == 0) return total == 0 && local_total == 0 ? ZS_OK : ZS_ERR_LAYOUT;
  if (!host_desc) return ZS_ERR_NULL;
  int64_t run = 0, lrun = 0;
  for (int32_t i = 0; i < nparams; ++i) {
    const zs_dim0_desc& d = host_desc[i];
    if (d.numel < 0 || d.chunk < 0) return ZS_ERR_SIZE;
    if (d.flat_offset != run || d.local_offset != lrun) return ZS_ERR_LAYOUT;
    if (d.numel > 0 && !d.ptr) return ZS_ERR_NULL;
    if (d.numel > 0 && !aligned(d.ptr, (uintptr_t)elem_size(dtype))) return ZS_ERR_ALIGN;
    // the N chunks must cover the parameter: numel <= world * chunk
    if (d.chunk < d.numel / world + (d.numel % world != 0)) return ZS_ERR_LAYOUT;
    if (d.numel > INT64_MAX - run || d.chunk > INT64_MAX - lrun) return ZS_ERR_SIZE;
    run += d.numel;
    lrun += d.chunk;
  }
  if (lrun > INT64_MAX / world) return ZS_ERR_SIZE;
  return run == total && lrun == local_total ? ZS_OK : ZS_ERR_LAYOUT;
}

zs_status zs_pack_shard_dim0(const zs_dim0_desc* d_desc, int32_t nparams, int32_t src_dtype,
                             int32_t world, int32_t rank, int64_t local_total, float* master,
                             float* exp_avg, float* exp_avg_sq, hipStream_t stream) {
  if (nparams < 0 || local_total < 0) return ZS_ERR_SIZE;
  if (nparams == 0 && local_total != 0) return ZS_ERR_SIZE;
  if (world < 1) return ZS_ERR_WORLD;
  if (rank < 0 || rank >= world) return ZS_ERR_RANK;
  if (src_dtype != ZS_F32 && src_dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (local_total == 0) return ZS_OK;
  if (!master || !d_desc) return ZS_ERR_NULL;
  if (!aligned(master, 4) || (exp_avg && !aligned(exp_avg, 4)) ||
      (exp_avg_sq && !aligned(exp_avg_sq, 4)) || !aligned(d_desc, 8))
    return ZS_ERR_ALIGN;
  const int64_t b = local_total * 4;
  if (overlaps(master, b, exp_avg, exp_avg ? b : 0) ||
      overlaps(master, b, exp_avg_sq, exp_avg_sq ? b : 0) ||
      overlaps(exp_avg, exp_avg ? b : 0, exp_avg_sq, exp_avg_sq ? b : 0))
    return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_pack_dim0(d_desc, nparams, src_dtype, rank, local_total, master,
                                         exp_avg, exp_avg_sq, stream); });
}

zs_status zs_copy_out_dim0(const uint16_t* gathered, int64_t gathered_numel,
                           const zs_dim0_desc* d_desc, int32_t nparams, int32_t world,
                           int64_t total, int64_t local_total, hipStream_t stream) {
  if (nparams < 0 || total < 0 || local_total < 0 || gathered_numel < 0) return ZS_ERR_SIZE;
  if (world < 1) return ZS_ERR_WORLD;
  if (nparams == 0 && (total != 0 || local_total != 0)) return ZS_ERR_SIZE;
  if (local_total > INT64_MAX / world || world * local_total > gathered_numel) return ZS_ERR_SIZE;
  if (total > world * local_total) return ZS_ERR_SIZE;
  if (total == 0) return ZS_OK;
  if (!gathered || !d_desc) return ZS_ERR_NULL;
  if (!aligned(gathered, 2) || !aligned(d_desc, 8)) return ZS_ERR_ALIGN;
  return launch([&] {
    return zs::launch_copy_out_dim0(gathered, d_desc, nparams, world, total, local_total, stream);
  });
}

zs_status zs_sharded_step(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                          float* master, float* exp_avg, float* exp_avg_sq,
                          const zs_adamw_hparams* hp, const float* grad_scale,
                          uint16_t* bf16_out, hipStream_t stream) {
  zs_status st = check_rows(rows, world, dtype, n);
  if (st != ZS_OK) return st;
  st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (n == 0) return ZS_OK;
  if (!master || !exp_avg || !exp_avg_sq) return ZS_ERR_NULL;
  if (!aligned(master, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) ||
      (bf16_out && !aligned(bf16_out, 2)) || (grad_scale && !aligned(grad_scale, 4)))
    return ZS_ERR_ALIGN;
  const int64_t b = n * 4;
  if (overlaps(master, b, exp_avg, b) || overlaps(master, b, exp_avg_sq, b) ||
      overlaps(exp_avg, b, exp_avg_sq, b))
    return ZS_ERR_OVERLAP;
  for (int32_t q = 0; q < world; ++q) {
    const int64_t rb = n * elem_size(dtype);
    if (overlaps(rows[q], rb, master, b) || overlaps(rows[q], rb, exp_avg, b) ||
        overlaps(rows[q], rb, exp_avg_sq, b) || (bf16_out && overlaps(rows[q], rb, bf16_out, n * 2)))
      return ZS_ERR_OVERLAP;
  }
  if (bf16_out && (overlaps(bf16_out, n * 2, master, b) || overlaps(bf16_out, n * 2, exp_avg, b) ||
                   overlaps(bf16_out, n * 2, exp_avg_sq, b)))
    return ZS_ERR_OVERLAP;
  if (scale_overlaps(grad_scale, master, exp_avg, exp_avg_sq, n, bf16_out)) return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_fused(rows, world, dtype, n, master, exp_avg, exp_avg_sq, *hp,
                                     grad_scale, bf16_out, stream); });
}

zs_status zs_accumulate_grads(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                              float* acc, float scale, int32_t first, double* sumsq_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  zs_status st = check_rows(rows, world, dtype, n);
  if (st != ZS_OK) return st;
  if (!std::isfinite(scale)) return ZS_ERR_HPARAM;
  if (n > 0 && !acc) return ZS_ERR_NULL;
  if (acc && !aligned(acc, 4)) return ZS_ERR_ALIGN;
  if (sumsq_out) {
    if (!aligned(sumsq_out, 8)) return ZS_ERR_ALIGN;
    if (!workspace || workspace_bytes < zs_workspace_bytes(n)) return ZS_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return ZS_ERR_ALIGN;
    st = check_sumsq_buffers(rows, world, dtype, n, acc, sumsq_out, workspace, workspace_bytes);
    if (st != ZS_OK) return st;
  }
  if (n == 0 && !sumsq_out) return ZS_OK;
  for (int32_t q = 0; q < world && n > 0; ++q)
    if (overlaps(acc, n * 4, rows[q], n * elem_size(dtype))) return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_accumulate(rows, world, dtype, n, acc, scale, first != 0, sumsq_out,
                                          static_cast<double*>(workspace), stream); });
}

zs_status zs_accumulate_local(const void* grad, int32_t dtype, int64_t n, float* acc,
                              int32_t first, hipStream_t stream) {
  if (dtype != ZS_F32 && dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (n < 0) return ZS_ERR_SIZE;
  if (n == 0) return ZS_OK;
  if (!grad || !acc) return ZS_ERR_NULL;
  if (!aligned(grad, (uintptr_t)elem_size(dtype)) || !aligned(acc, 4)) return ZS_ERR_ALIGN;
  if (overlaps(grad, n * elem_size(dtype), acc, n * 4)) return ZS_ERR_OVERLAP;
  return launch([&] { return zs::launch_accumulate_local(grad, dtype, n, acc, first != 0, stream); });
}

zs_status zs_clip_coefficient(const double* partials, int32_t count, double max_norm,
                              float* coef_out, double* norm_out, hipStream_t stream) {
  if (count < 1) return ZS_ERR_SIZE;
  if (!std::isfinite(max_norm) || !(max_norm > 0)) return ZS_ERR_HPARAM;
  if (!partials || !coef_out) return ZS_ERR_NULL;
  if (!aligned(partials, 8) || !aligned(coef_out, 4) || (norm_out && !aligned(norm_out, 8)))
    return ZS_ERR_ALIGN;
  return launch([&] { return zs::launch_clip(partials, count, max_norm, coef_out, norm_out, stream); });
}

}  // extern "C"
