"""Python binding of libzs: the C-ABI calls under the same names, taking torch tensors.

Argument marshalling only -- every step of the update runs in the HIP kernels
of libzs. PyTorch supplies device memory and the stream (by default the
current stream of the tensors' device); every call is asynchronous on it.

Errors from the library raise ZsArgumentError (a ValueError) for bad
arguments and ZsError (a RuntimeError) for HIP failures; tensors that are not
contiguous device tensors of the expected dtype raise ValueError before the
library is called.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L
from ._lib import ZS_BF16, ZS_F32, ZsArgumentError, ZsError  # noqa: F401

_DTYPES = {torch.float32: ZS_F32, torch.bfloat16: ZS_BF16}


def _lib():
    return L.load()


def _dev(t: torch.Tensor, name: str, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _hparams(lr, beta1, beta2, eps, weight_decay, step) -> L.AdamWHParams:
    return L.AdamWHParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                          int(step))


# ---------------------------------------------------------------- layout

def zs_flat_layout(numels, world: int, align: int = 1):
    """(offsets, total T, padded P, shard S) of a FlatParameter over `world`
    ranks, S rounded up to a multiple of `align` elements (1: no rounding)."""
    n = len(numels)
    arr = (C.c_int64 * max(n, 1))(*[int(x) for x in numels])
    offs = (C.c_int64 * max(n, 1))()
    total, padded, shard = C.c_int64(), C.c_int64(), C.c_int64()
    L.check("zs_flat_layout", _lib().zs_flat_layout(
        arr, n, int(world), int(align), offs, C.byref(total), C.byref(padded), C.byref(shard)))
    return list(offs[:n]), total.value, padded.value, shard.value


class ParamTable:
    """Descriptor table of one unit's parameters, in flat order.

    The host copy is checked by zs_check_layout; the device copy (24 bytes per
    parameter) is what the pack and copy-out kernels read. The tensors are
    kept referenced for the table's lifetime.
    """

    def __init__(self, tensors, device=None):
        if len(tensors) == 0:
            raise ValueError("a unit needs at least one parameter")
        dtype = tensors[0].dtype
        if dtype not in _DTYPES:
            raise ValueError(f"unsupported parameter dtype {dtype}")
        for i, t in enumerate(tensors):
            _dev(t, f"param[{i}]", dtype)
        self.tensors = list(tensors)
        self.dtype = dtype
        self.nparams = len(tensors)
        self.offsets, self.total, _, _ = zs_flat_layout([t.numel() for t in tensors], 1)
        host = (L.ParamDesc * self.nparams)()
        for i, (t, off) in enumerate(zip(self.tensors, self.offsets)):
            host[i].ptr = t.data_ptr()
            host[i].flat_offset = off
            host[i].numel = t.numel()
        L.check("zs_check_layout", _lib().zs_check_layout(host, self.nparams, self.total, _DTYPES[dtype]))
        device = device if device is not None else tensors[0].device
        raw = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8)
        self.device_table = raw.to(device)
        torch.cuda.current_stream(device).synchronize()  # the host staging copy is released

    @property
    def ptr(self):
        return C.c_void_p(self.device_table.data_ptr())


# ---------------------------------------------------------------- pack / copy-out

def zs_pack_shard(table: ParamTable, world: int, rank: int, master, exp_avg=None, exp_avg_sq=None,
                  stream=None, align: int = 1):
    _dev(master, "master", torch.float32)
    for name, t in (("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if t is not None:
            _dev(t, name, torch.float32)
            if t.numel() != master.numel():
                raise ValueError(f"{name} must have the master's size")
    L.check("zs_pack_shard", _lib().zs_pack_shard(
        table.ptr, table.nparams, table.total, _DTYPES[table.dtype], int(world), int(rank),
        int(align), master.numel(), _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq),
        _stream(stream, master.device)))


def zs_copy_out(gathered, table: ParamTable, stream=None):
    _dev(gathered, "gathered", torch.bfloat16)
    if table.dtype != torch.bfloat16:
        raise ValueError("copy-out destinations must be bf16")
    L.check("zs_copy_out", _lib().zs_copy_out(
        _ptr(gathered), gathered.numel(), table.ptr, table.nparams, table.total,
        _stream(stream, gathered.device)))


# ---------------------------------------------------------------- per-parameter dim-0 sharding

def zs_dim0_layout(shapes, world: int):
    """(chunks, local offsets, local total L) of per-parameter dim-0 sharding over `world` ranks.

    A 0-d parameter is one row of one element.
    """
    n = len(shapes)
    d0 = [int(s[0]) if len(s) else 1 for s in shapes]
    rs = []
    for s in shapes:
        r = 1
        for x in s[1:]:
            r *= int(x)
        rs.append(r)
    a = (C.c_int64 * max(n, 1))(*d0)
    b = (C.c_int64 * max(n, 1))(*rs)
    chunk = (C.c_int64 * max(n, 1))()
    loff = (C.c_int64 * max(n, 1))()
    lt = C.c_int64()
    L.check("zs_dim0_layout", _lib().zs_dim0_layout(a, b, n, int(world), chunk, loff, C.byref(lt)))
    return list(chunk[:n]), list(loff[:n]), lt.value


class Dim0Table:
    """Descriptor table of one unit's parameters under dim-0 sharding over `world` ranks.

    The host copy is checked by zs_check_dim0_layout; the device copy (40 bytes
    per parameter) is what the pack and copy-out kernels read. The tensors are
    kept referenced for the table's lifetime.
    """

    def __init__(self, tensors, world: int, device=None):
        if len(tensors) == 0:
            raise ValueError("a unit needs at least one parameter")
        dtype = tensors[0].dtype
        if dtype not in _DTYPES:
            raise ValueError(f"unsupported parameter dtype {dtype}")
        for i, t in enumerate(tensors):
            _dev(t, f"param[{i}]", dtype)
        self.tensors = list(tensors)
        self.dtype = dtype
        self.world = int(world)
        self.nparams = len(tensors)
        self.chunks, self.local_offsets, self.local_total = zs_dim0_layout(
            [tuple(t.shape) for t in tensors], self.world)
        self.offsets, self.total, _, _ = zs_flat_layout([t.numel() for t in tensors], 1)
        host = (L.Dim0Desc * self.nparams)()
        for i, t in enumerate(self.tensors):
            host[i].ptr = t.data_ptr()
            host[i].flat_offset = self.offsets[i]
            host[i].numel = t.numel()
            host[i].chunk = self.chunks[i]
            host[i].local_offset = self.local_offsets[i]
        L.check("zs_check_dim0_layout", _lib().zs_check_dim0_layout(
            host, self.nparams, self.world, self.total, self.local_total, _DTYPES[dtype]))
        device = device if device is not None else tensors[0].device
        raw = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8)
        self.device_table = raw.to(device)
        torch.cuda.current_stream(device).synchronize()  # the host staging copy is released

    @property
    def ptr(self):
        return C.c_void_p(self.device_table.data_ptr())


def zs_pack_shard_dim0(table: Dim0Table, rank: int, master, exp_avg=None, exp_avg_sq=None,
                       stream=None):
    _dev(master, "master", torch.float32)
    if master.numel() != table.local_total:
        raise ValueError(f"master must hold the rank's {table.local_total} elements")
    for name, t in (("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if t is not None:
            _dev(t, name, torch.float32)
            if t.numel() != master.numel():
                raise ValueError(f"{name} must have the master's size")
    L.check("zs_pack_shard_dim0", _lib().zs_pack_shard_dim0(
        table.ptr, table.nparams, _DTYPES[table.dtype], table.world, int(rank), table.local_total,
        _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq), _stream(stream, master.device)))


def zs_copy_out_dim0(gathered, table: Dim0Table, stream=None):
    _dev(gathered, "gathered", torch.bfloat16)
    if table.dtype != torch.bfloat16:
        raise ValueError("copy-out destinations must be bf16")
    L.check("zs_copy_out_dim0", _lib().zs_copy_out_dim0(
        _ptr(gathered), gathered.numel(), table.ptr, table.nparams, table.world, table.total,
        table.local_total, _stream(stream, gathered.device)))


# ---------------------------------------------------------------- reduce / AdamW / cast

def _rows(rows, n):
    if len(rows) == 0:
        raise ValueError("need at least one gradient contribution")
    dtype = rows[0].dtype
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported contribution dtype {dtype}")
    for i, r in enumerate(rows):
        _dev(r, f"rows[{i}]", dtype)
        if r.numel() != n:
            raise ValueError(f"rows[{i}] has {r.numel()} elements, expected {n}")
    arr = (C.c_void_p * len(rows))(*[r.data_ptr() for r in rows])
    return arr, len(rows), _DTYPES[dtype]


def zs_workspace_bytes(n: int) -> int:
    return int(_lib().zs_workspace_bytes(int(n)))


def zs_reduce_grads(rows, grad_out, sumsq_out=None, workspace=None, stream=None):
    _dev(grad_out, "grad_out", torch.float32)
    arr, world, dt = _rows(rows, grad_out.numel())
    ws_bytes = 0
    if sumsq_out is not None:
        _dev(sumsq_out, "sumsq_out", torch.float64)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    L.check("zs_reduce_grads", _lib().zs_reduce_grads(
        arr, world, dt, grad_out.numel(), _ptr(grad_out), _ptr(sumsq_out), _ptr(workspace),
        ws_bytes, _stream(stream, grad_out.device)))


def zs_reduce_grads_noalloc(rows, grad_out, sumsq_out=None, stream=None):
    """zs_reduce_grads without a workspace: the sum of squares uses the
    library's static scratch (no device allocation by the library)."""
    _dev(grad_out, "grad_out", torch.float32)
    arr, world, dt = _rows(rows, grad_out.numel())
    if sumsq_out is not None:
        _dev(sumsq_out, "sumsq_out", torch.float64)
    L.check("zs_reduce_grads_noalloc", _lib().zs_reduce_grads_noalloc(
        arr, world, dt, grad_out.numel(), _ptr(grad_out), _ptr(sumsq_out), _stream(stream, grad_out.device)))


def _state(master, exp_avg, exp_avg_sq):
    _dev(master, "master", torch.float32)
    _dev(exp_avg, "exp_avg", torch.float32)
    _dev(exp_avg_sq, "exp_avg_sq", torch.float32)
    n = master.numel()
    if exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError("master, exp_avg and exp_avg_sq must have the same size")
    return n


def _opt_out(bf16_out, grad_scale, n):
    if bf16_out is not None:
        _dev(bf16_out, "bf16_out", torch.bfloat16)
        if bf16_out.numel() != n:
            raise ValueError("bf16_out must have the master's size")
    if grad_scale is not None:
        _dev(grad_scale, "grad_scale", torch.float32)
        if grad_scale.numel() != 1:
            raise ValueError("grad_scale is a single fp32 value")


def zs_adamw_step(master, exp_avg, exp_avg_sq, grad, *, lr, beta1, beta2, eps, weight_decay, step,
                  grad_scale=None, bf16_out=None, stream=None):
    n = _state(master, exp_avg, exp_avg_sq)
    _dev(grad, "grad", torch.float32)
    if grad.numel() != n:
        raise ValueError("grad must have the master's size")
    _opt_out(bf16_out, grad_scale, n)
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, step)
    L.check("zs_adamw_step", _lib().zs_adamw_step(
        _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(grad), n, C.byref(hp),
        _ptr(grad_scale), _ptr(bf16_out), _stream(stream, master.device)))


def zs_cast_for_gather(master, gather_slot, stream=None):
    _dev(master, "master", torch.float32)
    _dev(gather_slot, "gather_slot", torch.bfloat16)
    if gather_slot.numel() != master.numel():
        raise ValueError("gather_slot must have the master's size")
    L.check("zs_cast_for_gather", _lib().zs_cast_for_gather(
        _ptr(master), master.numel(), _ptr(gather_slot), _stream(stream, master.device)))


def zs_sharded_step(rows, master, exp_avg, exp_avg_sq, *, lr, beta1, beta2, eps, weight_decay,
                    step, grad_scale=None, bf16_out=None, stream=None):
    n = _state(master, exp_avg, exp_avg_sq)
    arr, world, dt = _rows(rows, n)
    _opt_out(bf16_out, grad_scale, n)
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, step)
    L.check("zs_sharded_step", _lib().zs_sharded_step(
        arr, world, dt, n, _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq), C.byref(hp),
        _ptr(grad_scale), _ptr(bf16_out), _stream(stream, master.device)))


class ShardedStep:
    """zs_sharded_step with its arguments checked and marshalled once.

    Calling the object with a step number issues one C call with the prepared
    arguments: the per-step host cost is a single ctypes call, which is what a
    small (launch-bound) shard needs. The tensors are kept referenced. The
    stream is fixed when the object is made (default: the current stream of
    the master's device at that moment), so an object used under HIP graph
    capture must be made inside the capture. The library still validates
    every call.
    """

    def __init__(self, rows, master, exp_avg, exp_avg_sq, *, lr, beta1, beta2, eps, weight_decay,
                 grad_scale=None, bf16_out=None, stream=None):
        n = _state(master, exp_avg, exp_avg_sq)
        self._rows, self._world, self._dtype = _rows(rows, n)
        _opt_out(bf16_out, grad_scale, n)
        self._keep = (list(rows), master, exp_avg, exp_avg_sq, grad_scale, bf16_out)
        self._hp = _hparams(lr, beta1, beta2, eps, weight_decay, 1)
        self._fn = _lib().zs_sharded_step
        self._args = (self._rows, self._world, self._dtype, n, _ptr(master), _ptr(exp_avg),
                      _ptr(exp_avg_sq), C.byref(self._hp), _ptr(grad_scale), _ptr(bf16_out),
                      _stream(stream, master.device))

    def __call__(self, step: int) -> None:
        self._hp.step = int(step)
        st = self._fn(*self._args)
        if st != 0:
            L.check("zs_sharded_step", st)


def zs_accumulate_grads(rows, acc, *, scale=1.0, first=False, sumsq_out=None, workspace=None,
                        stream=None):
    _dev(acc, "acc", torch.float32)
    arr, world, dt = _rows(rows, acc.numel())
    ws_bytes = 0
    if sumsq_out is not None:
        _dev(sumsq_out, "sumsq_out", torch.float64)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    L.check("zs_accumulate_grads", _lib().zs_accumulate_grads(
        arr, world, dt, acc.numel(), _ptr(acc), float(scale), int(bool(first)), _ptr(sumsq_out),
        _ptr(workspace), ws_bytes, _stream(stream, acc.device)))


def zs_accumulate_local(grad, acc, *, first=False, stream=None):
    _dev(acc, "acc", torch.float32)
    _dev(grad, "grad")
    if grad.dtype not in _DTYPES:
        raise ValueError(f"unsupported gradient dtype {grad.dtype}")
    if grad.numel() != acc.numel():
        raise ValueError("grad and acc must have the same size")
    L.check("zs_accumulate_local", _lib().zs_accumulate_local(
        _ptr(grad), _DTYPES[grad.dtype], acc.numel(), _ptr(acc), int(bool(first)),
        _stream(stream, acc.device)))


def zs_clip_coefficient(partials, max_norm, coef_out, norm_out=None, stream=None):
    _dev(partials, "partials", torch.float64)
    _dev(coef_out, "coef_out", torch.float32)
    if coef_out.numel() != 1:
        raise ValueError("coef_out is a single fp32 value")
    if norm_out is not None:
        _dev(norm_out, "norm_out", torch.float64)
    L.check("zs_clip_coefficient", _lib().zs_clip_coefficient(
        _ptr(partials), partials.numel(), float(max_norm), _ptr(coef_out), _ptr(norm_out),
        _stream(stream, partials.device)))


def zs_version() -> int:
    return int(_lib().zs_version())
