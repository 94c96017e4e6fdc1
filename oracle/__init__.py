"""CPU oracle of one rank's sharded ZeRO/FSDP update: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy (fp64 unless stated) restatement of what
the update computes, written from the pages below. Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and shares no code with it.

Pages cited throughout (title, address):
  [L5]   "Lesson 5: ZeRO and FSDP (including the FSDP2 architecture evolution)",
         hpc.payai.win/train/lesson05.html
  [ZvF]  "ZeRO vs FSDP: memory accounting and communication breakdown of
         large-model distributed training", muhenan.com/post/zero-vs-fsdp
  [FZ3]  "03 - FSDP (ZeRO-3): per-layer all-gather and reshard",
         llm-infra-atlas.github.io/parallel/01_dp/03_fsdp/
  [LAF]  "FSDP" (Latent Atlas), process-cxr.github.io/ai-library/training/
         distributed-training/fsdp
  [DPZ]  "Data parallelism and ZeRO memory sharding",
         jefxiong.cn/index.php/archives/aigc-fundamentals-zero.html

Modules:
  layout  flatten / pad / shard / pack / copy-out      ([L5] s7.1, [LAF] s5.1)
  reduce  mean of per-rank gradient contributions      ([DPZ] s3.1, [L5] s7.5)
  adamw   decoupled-decay Adam on the fp32 shard       ([L5] s3, [DPZ] s4.2)
  bf16    fp32 -> bf16 round-to-nearest-even           ([L5] s3 step 2)
  step    the composed update: reduce, AdamW, cast
  accumulate  micro-batch accumulation (ZeRO-1 / ZeRO-2 orders), global-norm
          clipping                                     ([L5] s2-3, [DPZ] s6)
  dim0    per-parameter dim-0 sharding and copy-out     ([L5] s7.2, [FZ3] s4)
  ledger  per-rank state and communication formulas    ([L5] s2-3, [DPZ] s3.2-3.4)

Parity unpinned (no page value or closed form fixes it): the last-ulp fp32
result of AdamW under a different but algebraically equal arrangement, and the
association order of the sum of squares. Tests accept any result within the
stated tolerances for those.
"""
from . import accumulate, adamw, bf16, dim0, layout, ledger, reduce, step  # noqa: F401
