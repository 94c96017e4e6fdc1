// Standalone C-ABI driver: the sharded update through libzs with nothing but
// the HIP runtime (no Python, no PyTorch). Test infrastructure: the GPU test
// writes the inputs, runs this program, and checks its outputs.
//
//   zs_driver IN OUT
//
// IN (little-endian): int32 world, int32 dtype (0 fp32, 1 bf16), int64 n,
//   int64 step, double lr, beta1, beta2, eps, weight_decay, int32 nparams,
//   int64 numel[nparams] (a split of n into parameters), then the rows
//   (world * n elements of dtype), theta, m, v (n fp32 each).
// OUT: g[n] fp32, sumsq fp64, theta' m' v' [n] fp32 and bf16[n] from the two
//   calls (zs_reduce_grads + zs_adamw_step), the same four from
//   zs_sharded_step on a second copy of the state, the bf16 slot copied out
//   into the nparams parameters by zs_copy_out (n bf16, concatenated), and
//   the fp32 master that zs_pack_shard (world 1) builds from theta split into
//   the same parameters (n fp32); then zs_cast_for_gather of the two-call
//   theta' (n bf16); two zs_accumulate_grads calls (scale 0.5, first then
//   not, the second with the sum of squares: n fp32 + fp64); two
//   zs_accumulate_local calls on rows 0 and 1 % world (n fp32);
//   zs_clip_coefficient of that sum of squares with max_norm 1e-3 (fp32
//   coefficient + fp64 norm); and the dim-0 path with the parameters taken as
//   1-D: L (int64), the last rank's zs_pack_shard_dim0 master (L fp32) and the
//   unshard of all ranks' packed shards -- each rank packed, the whole cast to
//   bf16, copied out by zs_copy_out_dim0 (n bf16, concatenated).
// Exit status: 0 on success, 2 on a usage or I/O error, 3 on a HIP error, and
// 10 + |status| when an entry point returns an error.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "zs.h"

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      std::exit(3);                                                                 \
    }                                                                               \
  } while (0)
#define ZS_OK_OR_EXIT(x)                                                            \
  do {                                                                              \
    zs_status s_ = (x);                                                             \
    if (s_ != ZS_OK) {                                                              \
      std::fprintf(stderr, "%s -> %s\n", #x, zs_status_string(s_));                 \
      std::exit(10 - s_ > 255 ? 255 : 10 - s_);                                     \
    }                                                                               \
  } while (0)

namespace {

template <typename T>
bool get(FILE* f, T* p, size_t count = 1) { return std::fread(p, sizeof(T), count, f) == count; }
template <typename T>
bool put(FILE* f, const T* p, size_t count = 1) { return std::fwrite(p, sizeof(T), count, f) == count; }

template <typename T>
T* dev_copy(const T* host, size_t count) {
  T* d = nullptr;
  HIP_OK(hipMalloc(&d, count * sizeof(T) + 16));
  if (host) HIP_OK(hipMemcpy(d, host, count * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

template <typename T>
std::vector<T> host_copy(const T* dev, size_t count) {
  std::vector<T> h(count);
  HIP_OK(hipMemcpy(h.data(), dev, count * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) return 2;
  int32_t world = 0, dtype = 0, nparams = 0;
  int64_t n = 0;
  zs_adamw_hparams hp{};
  bool ok = get(in, &world) && get(in, &dtype) && get(in, &n) && get(in, &hp.step) &&
            get(in, &hp.lr) && get(in, &hp.beta1) && get(in, &hp.beta2) && get(in, &hp.eps) &&
            get(in, &hp.weight_decay) && get(in, &nparams);
  if (!ok || world < 1 || n < 1 || nparams < 1) return 2;
  std::vector<int64_t> numel(nparams);
  const size_t esz = dtype == ZS_BF16 ? 2 : 4;
  std::vector<unsigned char> rows_h((size_t)world * n * esz);
  std::vector<float> th(n), m(n), v(n);
  ok = get(in, numel.data(), numel.size()) && get(in, rows_h.data(), rows_h.size()) &&
       get(in, th.data(), n) && get(in, m.data(), n) && get(in, v.data(), n);
  std::fclose(in);
  if (!ok) return 2;

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  std::vector<const void*> rows(world);
  for (int32_t q = 0; q < world; ++q) rows[q] = dev_copy(rows_h.data() + (size_t)q * n * esz, n * esz);
  float *d_th = dev_copy(th.data(), n), *d_m = dev_copy(m.data(), n), *d_v = dev_copy(v.data(), n);
  float *f_th = dev_copy(th.data(), n), *f_m = dev_copy(m.data(), n), *f_v = dev_copy(v.data(), n);
  float* d_g = dev_copy<float>(nullptr, n);
  uint16_t* d_out = dev_copy<uint16_t>(nullptr, n);
  uint16_t* f_out = dev_copy<uint16_t>(nullptr, n);
  double* d_sumsq = dev_copy<double>(nullptr, 1);
  const size_t ws_bytes = zs_workspace_bytes(n);
  void* d_ws = nullptr;
  HIP_OK(hipMalloc(&d_ws, ws_bytes));

  // the two-call path and the single pass on a copy of the state
  ZS_OK_OR_EXIT(zs_reduce_grads(rows.data(), world, dtype, n, d_g, d_sumsq, d_ws, ws_bytes, s));
  ZS_OK_OR_EXIT(zs_adamw_step(d_th, d_m, d_v, d_g, n, &hp, nullptr, d_out, s));
  ZS_OK_OR_EXIT(zs_sharded_step(rows.data(), world, dtype, n, f_th, f_m, f_v, &hp, nullptr, f_out, s));

  // unshard copy-out of the bf16 slot into nparams parameters, and the pack of
  // theta (split the same way) as a world-1 shard
  std::vector<int64_t> offsets(nparams);
  int64_t total = 0, padded = 0, shard = 0;
  ZS_OK_OR_EXIT(zs_flat_layout(numel.data(), nparams, 1, 1, offsets.data(), &total, &padded, &shard));
  if (total != n) return 2;
  std::vector<zs_param_desc> out_desc(nparams), src_desc(nparams);
  std::vector<uint16_t*> outs(nparams);
  std::vector<float*> srcs(nparams);
  for (int32_t i = 0; i < nparams; ++i) {
    outs[i] = dev_copy<uint16_t>(nullptr, numel[i]);
    srcs[i] = dev_copy(th.data() + offsets[i], numel[i]);
    out_desc[i] = zs_param_desc{outs[i], offsets[i], numel[i]};
    src_desc[i] = zs_param_desc{srcs[i], offsets[i], numel[i]};
  }
  ZS_OK_OR_EXIT(zs_check_layout(out_desc.data(), nparams, total, ZS_BF16));
  ZS_OK_OR_EXIT(zs_check_layout(src_desc.data(), nparams, total, ZS_F32));
  zs_param_desc* d_out_desc = dev_copy(out_desc.data(), nparams);
  zs_param_desc* d_src_desc = dev_copy(src_desc.data(), nparams);
  ZS_OK_OR_EXIT(zs_copy_out(d_out, n, d_out_desc, nparams, total, s));
  float* d_master = dev_copy<float>(nullptr, n);
  ZS_OK_OR_EXIT(zs_pack_shard(d_src_desc, nparams, total, ZS_F32, 1, 0, 1, shard, d_master, nullptr,
                              nullptr, s));
  // bf16 cast alone of the two-call theta'
  uint16_t* c_out = dev_copy<uint16_t>(nullptr, n);
  ZS_OK_OR_EXIT(zs_cast_for_gather(d_th, n, c_out, s));

  // gradient accumulation over two micro-batches (the same rows twice), then
  // the clipping coefficient from its sum of squares
  float* acc = dev_copy<float>(nullptr, n);
  double* acc_ss = dev_copy<double>(nullptr, 1);
  ZS_OK_OR_EXIT(zs_accumulate_grads(rows.data(), world, dtype, n, acc, 0.5f, 1, nullptr, nullptr, 0, s));
  ZS_OK_OR_EXIT(zs_accumulate_grads(rows.data(), world, dtype, n, acc, 0.5f, 0, acc_ss, d_ws, ws_bytes, s));
  float* lacc = dev_copy<float>(nullptr, n);
  ZS_OK_OR_EXIT(zs_accumulate_local(rows[0], dtype, n, lacc, 1, s));
  ZS_OK_OR_EXIT(zs_accumulate_local(rows[1 % world], dtype, n, lacc, 0, s));
  float* coef = dev_copy<float>(nullptr, 1);
  double* norm = dev_copy<double>(nullptr, 1);
  ZS_OK_OR_EXIT(zs_clip_coefficient(acc_ss, 1, 1e-3, coef, norm, s));

  // dim-0 sharding of the same parameters taken as 1-D tensors
  std::vector<int64_t> d0(numel), rs(nparams, 1), chunk(nparams), loff(nparams);
  int64_t L = 0;
  ZS_OK_OR_EXIT(zs_dim0_layout(d0.data(), rs.data(), nparams, world, chunk.data(), loff.data(), &L));
  std::vector<zs_dim0_desc> src0(nparams), dst0(nparams);
  std::vector<uint16_t*> outs0(nparams);
  for (int32_t i = 0; i < nparams; ++i) {
    outs0[i] = dev_copy<uint16_t>(nullptr, numel[i]);
    src0[i] = zs_dim0_desc{srcs[i], offsets[i], numel[i], chunk[i], loff[i]};
    dst0[i] = zs_dim0_desc{outs0[i], offsets[i], numel[i], chunk[i], loff[i]};
  }
  ZS_OK_OR_EXIT(zs_check_dim0_layout(src0.data(), nparams, world, total, L, ZS_F32));
  ZS_OK_OR_EXIT(zs_check_dim0_layout(dst0.data(), nparams, world, total, L, ZS_BF16));
  zs_dim0_desc* d_src0 = dev_copy(src0.data(), nparams);
  zs_dim0_desc* d_dst0 = dev_copy(dst0.data(), nparams);
  const int64_t wl = (int64_t)world * L;
  float* all_shards = dev_copy<float>(nullptr, (size_t)(wl > 0 ? wl : 1));
  float* zm = dev_copy<float>(nullptr, (size_t)(L > 0 ? L : 1));
  float* zv = dev_copy<float>(nullptr, (size_t)(L > 0 ? L : 1));
  for (int32_t r = 0; r < world; ++r)
    ZS_OK_OR_EXIT(zs_pack_shard_dim0(d_src0, nparams, ZS_F32, world, r, L, all_shards + (size_t)r * L,
                                     zm, zv, s));
  uint16_t* gathered0 = dev_copy<uint16_t>(nullptr, (size_t)(wl > 0 ? wl : 1));
  ZS_OK_OR_EXIT(zs_cast_for_gather(all_shards, wl, gathered0, s));
  ZS_OK_OR_EXIT(zs_copy_out_dim0(gathered0, wl, d_dst0, nparams, world, total, L, s));
  HIP_OK(hipStreamSynchronize(s));

  FILE* out = std::fopen(argv[2], "wb");
  if (!out) return 2;
  ok = put(out, host_copy(d_g, n).data(), n) && put(out, host_copy(d_sumsq, 1).data());
  for (const float* p : {d_th, d_m, d_v}) ok = ok && put(out, host_copy(p, n).data(), n);
  ok = ok && put(out, host_copy(d_out, n).data(), n);
  for (const float* p : {f_th, f_m, f_v}) ok = ok && put(out, host_copy(p, n).data(), n);
  ok = ok && put(out, host_copy(f_out, n).data(), n);
  for (int32_t i = 0; i < nparams; ++i) ok = ok && put(out, host_copy(outs[i], numel[i]).data(), numel[i]);
  ok = ok && put(out, host_copy(d_master, n).data(), n);
  ok = ok && put(out, host_copy(c_out, n).data(), n);
  ok = ok && put(out, host_copy(acc, n).data(), n) && put(out, host_copy(acc_ss, 1).data());
  ok = ok && put(out, host_copy(lacc, n).data(), n);
  ok = ok && put(out, host_copy(coef, 1).data()) && put(out, host_copy(norm, 1).data());
  ok = ok && put(out, &L);
  ok = ok && put(out, host_copy(all_shards + (size_t)(world - 1) * L, (size_t)L).data(), (size_t)L);
  for (int32_t i = 0; i < nparams; ++i) ok = ok && put(out, host_copy(outs0[i], numel[i]).data(), numel[i]);
  ok = std::fclose(out) == 0 && ok;
  if (!ok) return 2;

  for (const void* r : rows) HIP_OK(hipFree(const_cast<void*>(r)));
  for (void* p : {(void*)d_th, (void*)d_m, (void*)d_v, (void*)f_th, (void*)f_m, (void*)f_v,
                  (void*)d_g, (void*)d_out, (void*)f_out, (void*)d_sumsq, d_ws, (void*)d_out_desc,
                  (void*)d_src_desc, (void*)d_master, (void*)c_out, (void*)acc, (void*)acc_ss,
                  (void*)lacc, (void*)coef, (void*)norm, (void*)d_src0, (void*)d_dst0,
                  (void*)all_shards, (void*)zm, (void*)zv, (void*)gathered0})
    HIP_OK(hipFree(p));
  for (int32_t i = 0; i < nparams; ++i) {
    HIP_OK(hipFree(outs[i]));
    HIP_OK(hipFree(srcs[i]));
    HIP_OK(hipFree(outs0[i]));
  }
  HIP_OK(hipStreamDestroy(s));
  std::printf("zs_driver ok: world=%d dtype=%d n=%lld nparams=%d\n", world, dtype, (long long)n, nparams);
  return 0;
}
