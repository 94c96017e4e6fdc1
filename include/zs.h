/*
 * zs.h -- C ABI of one data-parallel rank's sharded ZeRO/FSDP update on
 * AMD Instinct MI355X (gfx950).
 *
 * The update of one rank, in the order the pages give it:
 *   1. pack     zs_flat_layout + zs_pack_shard: the rank's fp32 slice of a
 *               FlatParameter (all parameters of a unit laid end to end and
 *               padded at the tail to a multiple of N).
 *   2. reduce   zs_reduce_grads: the fp32 mean of N per-rank gradient
 *               contributions for that slice -- the arithmetic a
 *               reduce-scatter performs for this rank.
 *   3. AdamW    zs_adamw_step: the local AdamW update of the fp32 master, m
 *               and v slice, optionally writing the bf16 result straight
 *               into the rank's slot of the all-gather buffer.
 *   4. cast and copy-out
 *               zs_cast_for_gather: fp32 master -> bf16 slot of the gather
 *               buffer; zs_copy_out: a gathered flat buffer -> per-parameter
 *               tensors (the unshard copy-out).
 *   Fused       zs_sharded_step: steps 2-3 (and the cast) in one pass.
 *
 * Pages (title, address) cited below:
 *   [L5]  "Lesson 5: ZeRO and FSDP", hpc.payai.win/train/lesson05.html
 *   [ZvF] "ZeRO vs FSDP", muhenan.com/post/zero-vs-fsdp
 *   [FZ3] "03 - FSDP (ZeRO-3): per-layer all-gather and reshard",
 *         llm-infra-atlas.github.io/parallel/01_dp/03_fsdp/
 *   [LAF] "FSDP" (Latent Atlas), process-cxr.github.io/ai-library/training/
 *         distributed-training/fsdp
 *   [DPZ] "Data parallelism and ZeRO memory sharding", jefxiong.cn/index.php/
 *         archives/aigc-fundamentals-zero.html
 *
 * Conventions common to every entry point:
 *   - Ownership: the caller owns every buffer (device data, descriptor tables,
 *     workspace). The library allocates no memory and keeps no state between
 *     calls, so calls on different streams are independent.
 *   - Execution: device work is enqueued on `stream` (NULL = the legacy
 *     default stream) and is asynchronous; results are valid once the
 *     stream has completed. No call synchronises.
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     a failed check returns a negative ZS_ERR_* code and enqueues nothing.
 *     A HIP launch failure returns ZS_ERR_HIP. A HIP error already pending on
 *     the calling thread when a call that launches work begins (left by an
 *     earlier, unrelated HIP call) is also returned as ZS_ERR_HIP, before
 *     anything is enqueued, and is left pending for the caller to read and
 *     clear (hipGetLastError). zs_status_string() names every code.
 *   - Launch shapes: chosen per call from the sizes and world size. The
 *     environment variables ZS_ADAMW_V, ZS_ADAMW_LDS, ZS_RANK_CHUNK,
 *     ZS_FUSED_G, ZS_FUSED_LDS, ZS_FUSED_BS, ZS_ACCUM_SHAPE, ZS_REDUCE_G and
 *     ZS_GRID_CAP override them for measurement sweeps, and are read only when
 *     ZS_TUNING=1 is set, once per process, at the first call; they change
 *     speed, never results.
 *   - Sizes are element counts (int64_t); n == 0 is a valid no-op.
 *   - bf16 values are passed as uint16_t bit patterns (the top half of an
 *     IEEE fp32). fp32 -> bf16 is round-to-nearest-even; NaN stays a quiet
 *     NaN with its sign; overflow goes to infinity.
 *   - Alignment: any element-aligned pointer is accepted. Inputs and fp32
 *     state on 16-byte boundaries (8-byte for bf16 contributions) take the
 *     vector path, whatever the alignment of a bf16 output (its 4-element
 *     groups are stored as one 8-byte or two 4-byte writes, or, when the
 *     output is 2 or 6 bytes past an 8-byte boundary, as aligned 8-byte
 *     words that straddle neighbouring groups); others take an element-wise
 *     path with the same results.
 */
#ifndef ZS_H_
#define ZS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t zs_status;

#define ZS_OK 0
#define ZS_ERR_NULL (-1)      /* a required pointer is NULL                       */
#define ZS_ERR_SIZE (-2)      /* negative or inconsistent element count           */
#define ZS_ERR_WORLD (-3)     /* world size outside [1, ZS_MAX_WORLD]             */
#define ZS_ERR_RANK (-4)      /* rank outside [0, world)                          */
#define ZS_ERR_DTYPE (-5)     /* dtype code is not ZS_F32 or ZS_BF16              */
#define ZS_ERR_HPARAM (-6)    /* hyper-parameter not finite / out of range, step<1 */
#define ZS_ERR_SHARD (-7)     /* shard_numel != ceil(total / world)               */
#define ZS_ERR_WORKSPACE (-8) /* workspace missing or smaller than required       */
#define ZS_ERR_LAYOUT (-9)    /* descriptor table does not tile [0, total)        */
#define ZS_ERR_ALIGN (-10)    /* pointer not aligned to its element size          */
#define ZS_ERR_OVERLAP (-11)  /* an output buffer overlaps an input it may not     */
#define ZS_ERR_HIP (-100)     /* a HIP runtime call or kernel launch failed       */

/* Element types of gradient contributions and parameters. */
#define ZS_F32 0
#define ZS_BF16 1

/* Largest number of simulated ranks one reduce may combine. */
#define ZS_MAX_WORLD 256

/*
 * One parameter of a unit, as laid out in its FlatParameter ([L5] s7.1 point 1;
 * [ZvF] s3, difference 1; [LAF] s5.1). Tables of these live in DEVICE memory
 * when passed to zs_pack_shard / zs_copy_out, and in HOST memory when passed
 * to zs_check_layout.
 *   ptr          device address of the parameter's contiguous (C-order) storage
 *   flat_offset  element offset of the parameter inside the flat buffer
 *   numel        element count of the parameter
 * A valid table lists the parameters in flat order and tiles [0, total):
 * flat_offset[0] == 0 and flat_offset[i+1] == flat_offset[i] + numel[i].
 */
typedef struct zs_param_desc {
  void* ptr;
  int64_t flat_offset;
  int64_t numel;
} zs_param_desc;

/*
 * AdamW hyper-parameters ([LAF] s9.3 lists lr, beta1, beta2, epsilon,
 * weight_decay). Given in double; the kernels derive fp32 constants from
 * them on the host. `step` is the 1-based step count t used for bias
 * correction 1 - beta^t.
 */
typedef struct zs_adamw_hparams {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
  int64_t step;
} zs_adamw_hparams;

/*
 * zs_flat_layout -- FlatParameter layout of a unit (host only, no device work).
 * [L5] s7.1 points 1 and 3; [LAF] s5.1; [DPZ] s4.2 (contiguous split).
 *   numels[nparams]      element count of each parameter, in registration order
 *   world                data-parallel world size N (>= 1)
 *   align                S is rounded up to a multiple of `align` elements
 *                        (>= 1). 1 gives the pages' layout, P = ceil(T / N) * N.
 *                        64 puts every rank's slice of a bf16 gather buffer,
 *                        and every row of a bf16 [N, S] receive buffer, on a
 *                        128-byte line: slices and rows off it cost the single
 *                        pass up to 3% (slices, at n = 1,003,782,656, N = 8)
 *                        and 10% (rows, at n = 117,187,500, N = 64). The extra
 *                        padding is at the tail; parameter offsets do not move.
 *   offsets_out[nparams] receives flat_offset of each parameter (exclusive
 *                        prefix sum of numels); may be NULL
 *   total_out            receives T = sum(numels)
 *   padded_out           receives P = S * N (tail padding only)
 *   shard_out            receives S = ceil(T / N) rounded up to a multiple of
 *                        align, the per-rank slice length
 * All pointers are host pointers. Output pointers other than offsets_out may
 * be NULL. Errors: ZS_ERR_NULL (numels NULL with nparams > 0), ZS_ERR_SIZE
 * (nparams < 0, align < 1, a negative numel, or T or P overflowing int64),
 * ZS_ERR_WORLD.
 */
zs_status zs_flat_layout(const int64_t* numels, int32_t nparams, int32_t world, int64_t align,
                         int64_t* offsets_out, int64_t* total_out, int64_t* padded_out,
                         int64_t* shard_out);

/*
 * zs_check_layout -- verify on the host that a descriptor table (HOST memory)
 * tiles [0, total) in order and that every non-empty parameter has a non-NULL
 * pointer aligned to its element size (`dtype`: ZS_F32 sources 4 bytes, ZS_BF16
 * sources and copy-out destinations 2 bytes). Returns ZS_OK or ZS_ERR_NULL /
 * ZS_ERR_SIZE / ZS_ERR_LAYOUT / ZS_ERR_ALIGN / ZS_ERR_DTYPE. The pack and
 * copy-out kernels rely on these properties of the device table without
 * re-checking it, so callers build the device copy from a table that passed.
 */
zs_status zs_check_layout(const zs_param_desc* host_desc, int32_t nparams, int64_t total,
                          int32_t dtype);

/*
 * zs_pack_shard -- the rank's fp32 master slice of the padded FlatParameter.
 * [L5] s7.1 points 1 and 3; [LAF] s5.1; [L5] s2 (fp32 master, m, v per rank).
 *   d_desc[nparams]  DEVICE table describing the unit (see zs_param_desc);
 *                    parameters hold `src_dtype` elements (ZS_F32 or ZS_BF16)
 *   total_numel      T of the unit (the table must tile [0, T))
 *   world, rank      N and r
 *   align, shard_numel
 *                    the layout's rounding and S: shard_numel must equal the S
 *                    that zs_flat_layout gives for (T, N, align), otherwise
 *                    ZS_ERR_SHARD
 *   master[S]        receives flat[r*S + k] for k < S, as fp32 (bf16 sources
 *                    are widened exactly); positions at or past T are +0.0
 *   exp_avg[S], exp_avg_sq[S]
 *                    optional (NULL = untouched); set to +0.0 (fresh Adam state)
 * Device pointers: d_desc, master, exp_avg, exp_avg_sq and the table's ptrs.
 * master must not overlap any parameter. Errors: ZS_ERR_NULL, ZS_ERR_SIZE,
 * ZS_ERR_WORLD, ZS_ERR_RANK, ZS_ERR_DTYPE, ZS_ERR_SHARD, ZS_ERR_HIP.
 */
zs_status zs_pack_shard(const zs_param_desc* d_desc, int32_t nparams, int64_t total_numel,
                        int32_t src_dtype, int32_t world, int32_t rank, int64_t align,
                        int64_t shard_numel, float* master, float* exp_avg, float* exp_avg_sq,
                        hipStream_t stream);

/*
 * zs_reduce_grads -- mean of N gradient contributions for this rank's slice.
 * [DPZ] s3.1 (equations for g_r and g: the mean over ranks equals the
 * full-batch gradient); [L5] s3 ZeRO-1/2 step 1 (reduce-scatter keeps only
 * this rank's 1/N); [L5] s7.5 (reduce_dtype = float32).
 *   rows[world]   HOST array of `world` DEVICE pointers; rows[q] points at
 *                 contribution q for this slice, n elements of `dtype`
 *                 (ZS_BF16 or ZS_F32); unused (may be NULL) when n == 0.
 *                 The pointers travel by value in the kernel arguments, so a
 *                 launch captured into a HIP graph keeps them: a replay reads
 *                 the same row buffers.
 *                 Rows that start on 128-byte boundaries stream fastest: the
 *                 N rows of one [N, n] receive buffer whose row pitch is not a
 *                 multiple of 64 bytes start off the cache-line grid, and each
 *                 wave load then touches one line more (10% slower for the
 *                 single pass at n = 117,187,500, N = 64); pad the pitch.
 *                 A pitch that is a multiple of 2 MiB (what separate large
 *                 allocations give) measured fastest, 1-5% ahead of pitches
 *                 off it by 256 B to 64 KiB.
 *   grad_out[n]   DEVICE fp32 output: g[k] = (c_0[k] + c_1[k] + ... ) / N,
 *                 summed in fp32 in ascending q starting from c_0[k], then
 *                 one IEEE division by N (bit-identical for any launch shape)
 *   sumsq_out     optional DEVICE double: receives sum_k g[k]^2 (this
 *                 shard's partial of a global gradient norm, [DPZ] s6),
 *                 accumulated in fp64 in a fixed order: the same bits on
 *                 every call with the same n, N and dtype on devices with
 *                 the same number of compute units (the launch's tiles, and
 *                 so the order of the partial sums, follow the CU count)
 *   workspace     DEVICE scratch of at least zs_workspace_bytes(n) bytes,
 *                 required only when sumsq_out != NULL
 * grad_out may not overlap any row; sumsq_out and workspace may not overlap
 * each other, grad_out or a row (ZS_ERR_OVERLAP). Errors: ZS_ERR_NULL,
 * ZS_ERR_SIZE, ZS_ERR_WORLD, ZS_ERR_DTYPE, ZS_ERR_WORKSPACE, ZS_ERR_ALIGN,
 * ZS_ERR_OVERLAP, ZS_ERR_HIP.
 */
zs_status zs_reduce_grads(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                          float* grad_out, double* sumsq_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * zs_reduce_grads_noalloc -- zs_reduce_grads for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, results and errors without the
 * workspace. The sum of squares' partials live in the library's own scratch,
 * a static device array of ZS_NOALLOC_MAX_N / 256 + 256 doubles (8 MiB + 2 KiB)
 * that every device the library runs on holds until the process ends. The
 * call allocates nothing; its first call on a device looks up that device's
 * copy once.
 *   n > ZS_NOALLOC_MAX_N with sumsq_out != NULL: ZS_ERR_WORKSPACE (the scratch
 *   is too small); without a sum of squares any n is accepted.
 * All calls on one device share its scratch: two calls with a sum of squares
 * that overlap in time on one device (on different streams, or from different
 * threads) race and may return a wrong sum of squares. Serialise them. Nothing
 * in the scratch needs clearing: every call overwrites what it reads.
 */
#define ZS_NOALLOC_MAX_N (INT64_C(1) << 28)
zs_status zs_reduce_grads_noalloc(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                                  float* grad_out, double* sumsq_out, hipStream_t stream);

/* Bytes of workspace zs_reduce_grads / zs_accumulate_grads need for a sum of
 * squares over n elements: one fp64 partial per 256-element tile (at most
 * 2^24 - 1 of them) plus 256 second-level partials; 0 for n < 0. The contents
 * need no initialisation and are overwritten by every call that takes a sum of
 * squares. */
size_t zs_workspace_bytes(int64_t n);

/*
 * zs_adamw_step -- AdamW on the rank's fp32 slice, in place.
 * [L5] s3 (ZeRO-1/2 step 2; ZeRO-3 item 4: local update of the 1/N fp32
 * state, no communication); [DPZ] s4.2 (bias-corrected first step, eps
 * outside the root); [LAF] s8.2 step 6. Weight decay is decoupled.
 * Per element, with t = hp->step:
 *   m' = b1 m + (1 - b1) g;   v' = b2 v + (1 - b2) g^2
 *   theta' = theta (1 - lr wd) - (lr / (1 - b1^t)) m' / (sqrt(v' / (1 - b2^t)) + eps)
 *   master[n], exp_avg[n], exp_avg_sq[n]   DEVICE fp32, updated in place
 *   grad[n]                                DEVICE fp32 (e.g. zs_reduce_grads' output)
 *   hp                                     HOST pointer
 *   grad_scale    optional DEVICE fp32 scalar (NULL = 1): g is multiplied by
 *                 *grad_scale before the update (e.g. a gradient-clipping
 *                 coefficient computed on the device from sums of squares)
 *   bf16_out[n]   optional DEVICE bf16 output (NULL = skip): bf16(theta'),
 *                 typically the rank's slot of the all-gather buffer
 * No two of master, exp_avg, exp_avg_sq, grad and bf16_out may share bytes, and
 * grad_scale may not overlap an output (ZS_ERR_OVERLAP). Arrays that start on
 * 128-byte boundaries stream fastest: a wave's 1 KiB access to an array that
 * starts elsewhere straddles a partial cache line at each end, and a
 * partial-line write costs HBM a read-modify-write (a shard split into chunks
 * should split on multiples of 32 elements).
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE, ZS_ERR_HPARAM (non-finite values, lr, eps
 * or wd < 0, betas outside [0, 1), step < 1), ZS_ERR_ALIGN, ZS_ERR_OVERLAP,
 * ZS_ERR_HIP.
 */
zs_status zs_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, const float* grad,
                        int64_t n, const zs_adamw_hparams* hp, const float* grad_scale,
                        uint16_t* bf16_out, hipStream_t stream);

/*
 * zs_cast_for_gather -- bf16 copy of the rank's updated fp32 slice into its
 * slot of the all-gather buffer ([L5] s3 ZeRO-1/2 step 2 and Fig. 5-4: write
 * back the BF16 parameter shard; the slot of rank r starts at r*S).
 *   master[n]       DEVICE fp32 input
 *   gather_slot[n]  DEVICE bf16 output (the caller passes gather + r*S)
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE, ZS_ERR_ALIGN, ZS_ERR_HIP.
 */
zs_status zs_cast_for_gather(const float* master, int64_t n, uint16_t* gather_slot,
                             hipStream_t stream);

/*
 * zs_copy_out -- unshard copy-out: per-parameter tensors from a gathered flat
 * bf16 buffer ([L5] s7.1 point 1: contiguous slices of the gathered
 * FlatParameter become each submodule's parameter; [FZ3] s1 and s3: the
 * all-gather result is copied out before compute).
 *   gathered[gathered_numel]  DEVICE bf16 flat buffer (P elements; the tail
 *                             pad is ignored)
 *   d_desc[nparams]           DEVICE table of destinations (bf16 elements);
 *                             must tile [0, total_numel)
 *   total_numel               T of the unit; must be <= gathered_numel
 * param i receives gathered[flat_offset_i .. flat_offset_i + numel_i).
 * Destinations may not overlap `gathered` or each other. Errors: ZS_ERR_NULL,
 * ZS_ERR_SIZE, ZS_ERR_HIP.
 */
zs_status zs_copy_out(const uint16_t* gathered, int64_t gathered_numel, const zs_param_desc* d_desc,
                      int32_t nparams, int64_t total_numel, hipStream_t stream);

/*
 * zs_sharded_step -- reduce, AdamW and the bf16 cast in one pass over the
 * slice: the same arithmetic as zs_reduce_grads followed by zs_adamw_step
 * (bit-identical results), without writing or re-reading the fp32 gradient.
 *   rows, world, dtype, n      as zs_reduce_grads
 *   master, exp_avg, exp_avg_sq, hp, bf16_out
 *                              as zs_adamw_step (bf16_out may be NULL)
 *   grad_scale    optional DEVICE fp32 scalar (NULL = 1): the mean gradient is
 *                 multiplied by *grad_scale before the update (a clipping
 *                 coefficient computed from a prior sum of squares)
 * Errors: union of the two calls' errors.
 */
zs_status zs_sharded_step(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                          float* master, float* exp_avg, float* exp_avg_sq,
                          const zs_adamw_hparams* hp, const float* grad_scale,
                          uint16_t* bf16_out, hipStream_t stream);

/*
 * zs_accumulate_grads -- sharded (ZeRO-2) gradient accumulation over micro-
 * batches: reduce this micro-batch's N contributions and add the mean into the
 * rank's fp32 accumulator ([L5] s3: ZeRO-2 reduce-scatters every micro-batch
 * and keeps only its 1/N; [L5] s2: the fp32 buffer costs 4P/N).
 *   rows, world, dtype, n     as zs_reduce_grads
 *   acc[n]        DEVICE fp32 accumulator:
 *                   first != 0:  acc = scale * mean
 *                   first == 0:  acc = acc + scale * mean
 *                 mean as in zs_reduce_grads (bit-identical); the product with
 *                 scale is skipped when scale == 1 (e.g. scale = 1/K for a
 *                 mean over K micro-batches)
 *   sumsq_out, workspace, workspace_bytes
 *                 optional: sum of squares of the updated acc (fp64), as in
 *                 zs_reduce_grads -- on the last micro-batch this is the
 *                 shard's partial of the global gradient norm
 * Errors: those of zs_reduce_grads, ZS_ERR_HPARAM (scale not finite).
 */
zs_status zs_accumulate_grads(const void* const* rows, int32_t world, int32_t dtype, int64_t n,
                              float* acc, float scale, int32_t first, double* sumsq_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * zs_accumulate_local -- unsharded (ZeRO-1) accumulation of one micro-batch's
 * local gradient in fp32 ([L5] s3: ZeRO-1 sums the full local gradient and
 * reduce-scatters once after the last micro-batch; [L5] s2: 4P per rank).
 *   grad[n]   DEVICE gradient of `dtype` (ZS_BF16 or ZS_F32)
 *   acc[n]    DEVICE fp32: first != 0: acc = grad (widened exactly);
 *             first == 0: acc = acc + grad
 * The accumulators of all ranks then go through zs_accumulate_grads (first=1,
 * scale=1/K) or zs_reduce_grads as fp32 contributions.
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE, ZS_ERR_DTYPE, ZS_ERR_ALIGN, ZS_ERR_OVERLAP, ZS_ERR_HIP.
 */
zs_status zs_accumulate_local(const void* grad, int32_t dtype, int64_t n, float* acc,
                              int32_t first, hipStream_t stream);

/*
 * zs_clip_coefficient -- global-norm clipping factor from per-shard sums of
 * squares ([DPZ] s6: the global norm needs every shard's partial; the combine
 * across ranks is an all-reduce in a multi-GPU job).
 *   partials[count]  DEVICE fp64 sums of squares (e.g. each rank's sumsq_out),
 *                    added in index order
 *   max_norm         the clipping threshold (finite, > 0)
 *   coef_out         DEVICE fp32: min(1, max_norm / (sqrt(total) + 1e-6)),
 *                    NaN if the total is NaN; pass it as grad_scale to
 *                    zs_adamw_step
 *   norm_out         optional DEVICE fp64: sqrt(total)
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE (count < 1), ZS_ERR_HPARAM, ZS_ERR_ALIGN, ZS_ERR_HIP.
 */
zs_status zs_clip_coefficient(const double* partials, int32_t count, double max_norm,
                              float* coef_out, double* norm_out, hipStream_t stream);

/*
 * Per-parameter dim-0 sharding (FSDP2 Shard(0); [L5] s7.2 and Fig. 5-5: each
 * parameter keeps its shape and is split on dim 0, a rank holding [H/N, D];
 * [FZ3] s4: DTensor sharded on dim 0, batched all-gather). A parameter with d0
 * rows of `rowsize` elements gives each rank c = ceil(d0/N) rows, rank r
 * holding rows [r*c, min((r+1)*c, d0)) zero-padded to c rows. A rank's shard
 * of a unit (also the all-gather input) is its padded chunks concatenated in
 * registration order, L elements; the all-gather output is the N shards one
 * after the other (N * L elements).
 *
 *   ptr           device address of the full parameter (C order)
 *   flat_offset   offset of the parameter in the unsharded unit (prefix sum of numels)
 *   numel         elements of the parameter (d0 * rowsize)
 *   chunk         elements per rank: ceil(d0 / N) * rowsize
 *   local_offset  offset of the parameter's chunk inside a rank's shard
 */
typedef struct zs_dim0_desc {
  void* ptr;
  int64_t flat_offset;
  int64_t numel;
  int64_t chunk;
  int64_t local_offset;
} zs_dim0_desc;

/*
 * zs_dim0_layout -- per-parameter chunk sizes and the rank-shard layout (host only).
 *   dim0[nparams], rowsize[nparams]  HOST arrays (a 0-d parameter: dim0 = rowsize = 1)
 *   chunk_out[nparams]               receives ceil(dim0/N) * rowsize (may be NULL)
 *   local_offsets_out[nparams]       receives the chunk offsets in a rank's shard (may be NULL)
 *   local_total_out                  receives L (may be NULL)
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE (negative or overflowing sizes), ZS_ERR_WORLD.
 */
zs_status zs_dim0_layout(const int64_t* dim0, const int64_t* rowsize, int32_t nparams, int32_t world,
                         int64_t* chunk_out, int64_t* local_offsets_out, int64_t* local_total_out);

/*
 * zs_check_dim0_layout -- verify a HOST table: flat offsets tile [0, total),
 * local offsets tile [0, local_total) with the chunk sizes, numel <= world *
 * chunk, and non-empty parameters have storage aligned to the element size of
 * `dtype` (as zs_check_layout). Returns ZS_OK or ZS_ERR_NULL / ZS_ERR_SIZE /
 * ZS_ERR_WORLD / ZS_ERR_LAYOUT / ZS_ERR_ALIGN / ZS_ERR_DTYPE.
 */
zs_status zs_check_dim0_layout(const zs_dim0_desc* host_desc, int32_t nparams, int32_t world,
                               int64_t total, int64_t local_total, int32_t dtype);

/*
 * zs_pack_shard_dim0 -- rank r's fp32 master shard under dim-0 sharding
 * (padding rows +0.0), with optional zeroed Adam moments.
 *   d_desc[nparams]  DEVICE table (see zs_dim0_desc); parameters hold src_dtype
 *   local_total      L; master, exp_avg, exp_avg_sq hold L fp32 elements (DEVICE)
 * The AdamW, cast and fused-step entry points apply to the shard unchanged.
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE, ZS_ERR_WORLD, ZS_ERR_RANK, ZS_ERR_DTYPE,
 * ZS_ERR_ALIGN, ZS_ERR_OVERLAP, ZS_ERR_HIP.
 */
zs_status zs_pack_shard_dim0(const zs_dim0_desc* d_desc, int32_t nparams, int32_t src_dtype,
                             int32_t world, int32_t rank, int64_t local_total, float* master,
                             float* exp_avg, float* exp_avg_sq, hipStream_t stream);

/*
 * zs_copy_out_dim0 -- unshard under dim-0 sharding: every parameter's rows
 * from the N ranks' regions of the gathered bf16 buffer (padding rows
 * dropped). A real scatter: parameter i's rows [r*c, ...) come from
 * gathered[r*L + local_offset_i ...].
 *   gathered[gathered_numel]  DEVICE bf16, gathered_numel >= world * local_total
 *   d_desc[nparams]           DEVICE table of bf16 destinations
 *   total                     T of the unit (sum of numels)
 * Errors: ZS_ERR_NULL, ZS_ERR_SIZE, ZS_ERR_WORLD, ZS_ERR_ALIGN, ZS_ERR_HIP.
 */
zs_status zs_copy_out_dim0(const uint16_t* gathered, int64_t gathered_numel,
                           const zs_dim0_desc* d_desc, int32_t nparams, int32_t world,
                           int64_t total, int64_t local_total, hipStream_t stream);

/* Static, NUL-terminated name of a status code ("ZS_OK", "ZS_ERR_NULL", ...). */
const char* zs_status_string(zs_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t zs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H_ */
