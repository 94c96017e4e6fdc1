"""One data-parallel rank's sharded ZeRO/FSDP update on AMD MI355X (gfx950).

The compute lives in libzs.so (hand-written HIP kernels behind the C ABI of
include/zs.h); this package is its thin Python binding. Importing the package
does not load the library; the first call does, and fails loudly if it has
not been built.
"""
from .api import (  # noqa: F401
    Dim0Table,
    ParamTable,
    ShardedStep,
    ZsArgumentError,
    ZsError,
    zs_accumulate_grads,
    zs_accumulate_local,
    zs_adamw_step,
    zs_cast_for_gather,
    zs_clip_coefficient,
    zs_copy_out,
    zs_copy_out_dim0,
    zs_dim0_layout,
    zs_flat_layout,
    zs_pack_shard,
    zs_pack_shard_dim0,
    zs_reduce_grads,
    zs_reduce_grads_noalloc,
    zs_sharded_step,
    zs_version,
    zs_workspace_bytes,
)
from ._lib import LIB_PATH, load  # noqa: F401
