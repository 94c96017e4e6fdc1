"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle routine (a dropped term, a
wrong sign, an off-by-one index, a reversed order, a different rounding rule),
swaps it into the oracle module for the duration of the case, and runs the pin
tests of that routine: at least one of them must fail. A pin set that passed a
mistaken oracle would not be pinning it.
"""
from fractions import Fraction

import numpy as np
import pytest

import test_oracle_accumulate as pins_accumulate
import test_oracle_adamw as pins_adamw
import test_oracle_bf16 as pins_bf16
import test_oracle_dim0 as pins_dim0
import test_oracle_layout as pins_layout
import test_oracle_ledger as pins_ledger
import test_oracle_reduce as pins_reduce
from oracle import accumulate, adamw, bf16, dim0, layout, ledger, reduce, step


def _fails(pins) -> bool:
    failed = False
    for pin in pins:
        try:
            pin()
        except Exception:  # an assertion, or the mistake breaking the pin's own arithmetic
            failed = True
    return failed


# ---- AdamW: one planted mistake each, otherwise the oracle's own arithmetic

def _adamw_variant(mistake):
    def step(theta, m, v, g, t, hp, state_dtype=np.float32):
        adamw.check_hparams(hp, t)
        th = np.asarray(theta, dtype=np.float64)
        m0 = np.asarray(m, dtype=np.float64)
        v0 = np.asarray(v, dtype=np.float64)
        gg = np.asarray(g, dtype=np.float64)
        b1, b2 = (hp.beta2, hp.beta1) if mistake == "swapped_betas" else (hp.beta1, hp.beta2)
        if mistake == "l2_decay":
            gg = gg + hp.weight_decay * th
        m1 = (b1 * m0 + (1.0 - b1) * gg).astype(state_dtype)
        v1 = (b2 * v0 + (1.0 - b2) * gg * gg).astype(state_dtype)
        bc1 = 1.0 if mistake in ("no_bias_correction", "bias_correction_v_only") else 1.0 - b1 ** t
        bc2 = 1.0 if mistake in ("no_bias_correction", "bias_correction_m_only") else 1.0 - b2 ** t
        if mistake == "step_off_by_one":
            bc1, bc2 = 1.0 - b1 ** (t + 1), 1.0 - b2 ** (t + 1)
        m_hat = m1.astype(np.float64) / bc1
        v_hat = v1.astype(np.float64) / bc2
        if mistake == "eps_inside_root":
            upd = hp.lr * m_hat / np.sqrt(v_hat + hp.eps)
        else:
            upd = hp.lr * m_hat / (np.sqrt(v_hat) + hp.eps)
        if mistake == "l2_decay":
            decay = 1.0
        elif mistake == "decay_sign":
            decay = 1.0 + hp.lr * hp.weight_decay
        else:
            decay = 1.0 - hp.lr * hp.weight_decay
        if mistake == "decay_after_update":
            return ((th - upd) * decay).astype(state_dtype), m1, v1
        return (th * decay - upd).astype(state_dtype), m1, v1
    return step


@pytest.mark.parametrize("mistake", ["no_bias_correction", "bias_correction_m_only",
                                     "bias_correction_v_only", "step_off_by_one", "l2_decay",
                                     "eps_inside_root", "decay_sign", "decay_after_update",
                                     "swapped_betas"])
def test_adamw_pins_catch(monkeypatch, mistake):
    monkeypatch.setattr(adamw, "adamw_step", _adamw_variant(mistake))
    assert _fails([pins_adamw.test_matches_torch_adamw_fp64_over_ten_steps,
                   pins_adamw.test_closed_form_first_step, pins_adamw.test_special_cases,
                   pins_adamw.test_worked_example_from_the_page]), mistake


def test_adamw_pins_pass_the_oracle_itself():
    assert not _fails([pins_adamw.test_matches_torch_adamw_fp64_over_ten_steps,
                       pins_adamw.test_closed_form_first_step, pins_adamw.test_special_cases,
                       pins_adamw.test_worked_example_from_the_page])


# ---- the mean over ranks

def _mean_exact_sum(rows):  # forgets the division by N
    return reduce.decode_rows(rows).astype(np.float64).sum(axis=0).astype(np.float32)


def _mean_exact_drops_last(rows):  # an off-by-one over the ranks
    c = reduce.decode_rows(rows).astype(np.float64)
    n = c.shape[0]
    return (c[: max(1, n - 1)].sum(axis=0) / n).astype(np.float32)


def _seq32_descending(rows):  # the fp32 running sum in the other order
    c = reduce.decode_rows(rows)
    s = c[-1].copy()
    for r in range(c.shape[0] - 2, -1, -1):
        s = (s + c[r]).astype(np.float32)
    return (s / np.float32(c.shape[0])).astype(np.float32)


def _seq32_divide_first(rows):  # each contribution divided by N before the fp32 sum
    c = reduce.decode_rows(rows)
    n = np.float32(c.shape[0])
    s = (c[0] / n).astype(np.float32)
    for r in range(1, c.shape[0]):
        s = (s + (c[r] / n).astype(np.float32)).astype(np.float32)
    return s


def _seq32_sum_in_fp64(rows):  # the running sum kept in fp64, rounded once
    c = reduce.decode_rows(rows).astype(np.float64)
    s = c[0].copy()
    for r in range(1, c.shape[0]):
        s = s + c[r]
    return (s / c.shape[0]).astype(np.float32)


REDUCE_PINS = [lambda: pins_reduce.test_mean_exact_is_rounded_once("bf16"),
               lambda: pins_reduce.test_mean_exact_is_rounded_once("f32"),
               pins_reduce.test_mean_seq32_order_is_ascending_from_rank0,
               lambda: pins_reduce.test_seq32_within_recursive_summation_bound("f32"),
               pins_reduce.test_single_rank_and_identical_contributions,
               pins_reduce.test_mean_of_rank_means_equals_full_batch_gradient_linear_loss,
               pins_reduce.test_mean_of_rank_means_equals_full_batch_gradient_least_squares]


@pytest.mark.parametrize("name,fn", [("mean_exact", _mean_exact_sum), ("mean_exact", _mean_exact_drops_last),
                                     ("mean_seq32", _seq32_descending),
                                     ("mean_seq32", _seq32_divide_first),
                                     ("mean_seq32", _seq32_sum_in_fp64)])
def test_reduce_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(reduce, name, fn)
    assert _fails(REDUCE_PINS), fn.__name__


def test_reduce_pins_pass_the_oracle_itself():
    assert not _fails(REDUCE_PINS)


def _abs_mean_no_division(rows):  # sum of magnitudes, not divided by N
    return np.abs(reduce.decode_rows(rows).astype(np.float64)).sum(axis=0)


def _abs_mean_of_sum(rows):  # |sum c_r| / N in place of sum |c_r| / N
    c = reduce.decode_rows(rows).astype(np.float64)
    return np.abs(c.sum(axis=0)) / c.shape[0]


ABS_MEAN_PINS = [pins_reduce.test_abs_mean_hand_values, pins_reduce.test_abs_mean_special_cases]


@pytest.mark.parametrize("fn", [_abs_mean_no_division, _abs_mean_of_sum])
def test_abs_mean_pins_catch(monkeypatch, fn):
    monkeypatch.setattr(reduce, "abs_mean", fn)
    assert _fails(ABS_MEAN_PINS), fn.__name__


def test_abs_mean_pins_pass_the_oracle_itself():
    assert not _fails(ABS_MEAN_PINS)


# ---- layout: flatten, pad, shard

def _shard_shifted(flat, world, rank):  # starts one element late
    s = flat.size // world
    out = np.zeros(s, dtype=flat.dtype)
    part = flat[rank * s + 1:(rank + 1) * s + 1]
    out[:part.size] = part
    return out


def _flatten_front_pad(params, world, dtype=None, align=1):  # the pad at the front
    lay = layout.flat_layout([np.asarray(p).size for p in params], world, align)
    if dtype is None:
        dtype = np.asarray(params[0]).dtype if params else np.float32
    flat = np.zeros(lay.padded, dtype=dtype)
    for off, p in zip(lay.offsets, params):
        a = np.asarray(p).ravel(order="C")
        flat[lay.pad + off:lay.pad + off + a.size] = a
    return flat


def _flatten_fortran(params, world, dtype=None, align=1):  # each tensor in column-major order
    lay = layout.flat_layout([np.asarray(p).size for p in params], world, align)
    if dtype is None:
        dtype = np.asarray(params[0]).dtype if params else np.float32
    flat = np.zeros(lay.padded, dtype=dtype)
    for off, p in zip(lay.offsets, params):
        a = np.asarray(p).ravel(order="F")
        flat[off:off + a.size] = a
    return flat


def _layout_with(shard_rule):
    def flat_layout(numels, world, align=1):
        offsets, t = [], 0
        for n in numels:
            offsets.append(t)
            t += int(n)
        s = shard_rule(t, world, align)
        return layout.Layout(tuple(offsets), t, s * world, s, s * world - t, world)
    flat_layout.__name__ = shard_rule.__name__
    return flat_layout


def _layout_floor(t, world, align):  # S = T / N rounded down instead of up
    return -(-(t // world) // align) * align


def _layout_align_floor(t, world, align):  # ceil(T / N) rounded down to a multiple of align
    return (-(-t // world) // align) * align


def _layout_align_total(t, world, align):  # T rounded up to a multiple of align, then split
    return -(-(-(-t // align) * align) // world)


LAYOUT_PINS = [pins_layout.test_brute_force_small, pins_layout.test_tiny_shard_is_param,
               pins_layout.test_tiny_ragged_layout_and_pad,
               pins_layout.test_contiguous_assignment_matches_illustration,
               pins_layout.test_flat_window_equals_slices_of_flatten,
               pins_layout.test_copy_out_shapes_and_pad_dropped,
               pins_layout.test_multidim_params_flatten_row_major,
               pins_layout.test_brute_force_small_with_aligned_slices,
               pins_layout.test_aligned_slices_by_hand]


@pytest.mark.parametrize("name,fn", [("shard_of", _shard_shifted), ("flatten", _flatten_front_pad),
                                     ("flatten", _flatten_fortran),
                                     ("flat_layout", _layout_with(_layout_floor)),
                                     ("flat_layout", _layout_with(_layout_align_floor)),
                                     ("flat_layout", _layout_with(_layout_align_total))])
def test_layout_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(layout, name, fn)
    assert _fails(LAYOUT_PINS), fn.__name__


def test_layout_pins_pass_the_oracle_itself():
    assert not _fails(LAYOUT_PINS)


# ---- fp32 -> bf16

def _bf16_truncate(x):
    return (bf16.f32_bits(x) >> np.uint32(16)).astype(np.uint16)


def _bf16_ties_away(x):
    u = bf16.f32_bits(x).astype(np.uint64)
    r = (u + np.uint64(0x8000)) >> np.uint64(16)
    nan = ((u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)) & ((u & np.uint64(0x7FFFFF)) != 0)
    return np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r).astype(np.uint16)


def _bf16_ties_down(x):  # ties always round down (toward zero in magnitude)
    u = bf16.f32_bits(x).astype(np.uint64)
    hi, lo = u >> np.uint64(16), u & np.uint64(0xFFFF)
    r = hi + (lo > np.uint64(0x8000)).astype(np.uint64)
    nan = ((u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)) & ((u & np.uint64(0x7FFFFF)) != 0)
    return np.where(nan, hi | np.uint64(0x40), r).astype(np.uint16)


def _bf16_nan_unquieted(x):  # NaN payload truncated without forcing the quiet bit
    u = bf16.f32_bits(x).astype(np.uint64)
    hi, lo = u >> np.uint64(16), u & np.uint64(0xFFFF)
    up = (lo > np.uint64(0x8000)) | ((lo == np.uint64(0x8000)) & ((hi & np.uint64(1)) == np.uint64(1)))
    r = hi + up.astype(np.uint64)
    nan = ((u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)) & ((u & np.uint64(0x7FFFFF)) != 0)
    return np.where(nan, hi, r).astype(np.uint16)


BF16_PINS = [pins_bf16.test_hand_worked_patterns, pins_bf16.test_against_torch_on_many_patterns,
             pins_bf16.test_nan_stays_quiet_nan]


@pytest.mark.parametrize("fn", [_bf16_truncate, _bf16_ties_away, _bf16_ties_down, _bf16_nan_unquieted])
def test_bf16_pins_catch(monkeypatch, fn):
    monkeypatch.setattr(bf16, "to_bf16_bits", fn)
    assert _fails(BF16_PINS), fn.__name__


def test_bf16_pins_pass_the_oracle_itself():
    assert not _fails(BF16_PINS)


# ---- micro-batch accumulation and clipping

def _zero2_no_scale(rows_per_microbatch, scale=1.0):
    acc = None
    for rows in rows_per_microbatch:
        u = reduce.mean_seq32(rows)
        acc = u.copy() if acc is None else (acc + u).astype(np.float32)
    return acc


def _zero2_keeps_last(rows_per_microbatch, scale=1.0):  # overwrites instead of adding
    acc = None
    for rows in rows_per_microbatch:
        acc = (reduce.mean_seq32(rows) * np.float32(scale)).astype(np.float32)
    return acc


def _zero1_scale_twice(rows_per_microbatch, scale=1.0):
    local = None
    for rows in rows_per_microbatch:
        c = reduce.decode_rows(rows) * np.float32(scale)
        local = c.copy() if local is None else (local + c).astype(np.float32)
    return (reduce.mean_seq32(local.astype(np.float32)) * np.float32(scale)).astype(np.float32)


def _clip_uncapped(partials, max_norm):
    norm = accumulate.global_norm(partials)
    return np.float32(max_norm / (norm + accumulate.CLIP_EPS)), norm


def _clip_no_root(partials, max_norm):  # the sum of squares taken for the norm
    norm = float(sum(float(p) for p in partials))
    c = min(1.0, max_norm / (norm + accumulate.CLIP_EPS))
    return np.float32(c), norm


ACCUM_PINS = [pins_accumulate.test_zero1_and_zero2_orders_equal_the_full_batch_gradient,
              pins_accumulate.test_single_microbatch_is_the_plain_reduce,
              lambda: pins_accumulate.test_both_orders_within_the_summation_bound("bf16"),
              pins_accumulate.test_clip_matches_torch_clip_grad_norm,
              pins_accumulate.test_clip_nonfinite_and_order]


@pytest.mark.parametrize("name,fn", [("zero2_accumulate", _zero2_no_scale),
                                     ("zero2_accumulate", _zero2_keeps_last),
                                     ("zero1_accumulate", _zero1_scale_twice),
                                     ("clip_coefficient", _clip_uncapped),
                                     ("clip_coefficient", _clip_no_root)])
def test_accumulate_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(accumulate, name, fn)
    assert _fails(ACCUM_PINS), fn.__name__


def test_accumulate_pins_pass_the_oracle_itself():
    assert not _fails(ACCUM_PINS)


# ---- FSDP2 dim-0 sharding

def _dim0_floor(shapes_, world):  # rows per rank rounded down
    rows, rs, chunk, loff = [], [], [], []
    t = 0
    for shp in shapes_:
        shp = tuple(int(x) for x in shp)
        d0 = shp[0] if len(shp) else 1
        r = int(np.prod(shp[1:])) if len(shp) > 1 else 1
        c = (d0 // world) * r
        rows.append(d0)
        rs.append(r)
        chunk.append(c)
        loff.append(t)
        t += c
    return dim0.Dim0Layout(tuple(rows), tuple(rs), tuple(chunk), tuple(loff), t, world)


def _copy_out_param_major(gathered, shapes_, world):  # reads the buffer as if parameter-major
    lay = dim0.dim0_layout(shapes_, world)
    outs = []
    for shp, c, lo in zip(shapes_, lay.chunk, lay.local_offsets):
        n = int(np.prod(shp)) if len(shp) else 1
        flat = np.empty(n, dtype=gathered.dtype)
        for r in range(world):
            v = dim0.valid(n, c, r)
            base = world * lo + r * c
            flat[r * c:r * c + v] = gathered[base:base + v]
        outs.append(flat.reshape(shp))
    return outs


DIM0_PINS = [pins_dim0.test_matches_torch_chunk_on_small_shapes,
             pins_dim0.test_multi_parameter_shard_and_roundtrip,
             pins_dim0.test_gpt2_token_embedding_at_eight_ranks, pins_dim0.test_tiny_ragged_layout,
             pins_dim0.test_llama_block_divides_evenly]


@pytest.mark.parametrize("name,fn", [("dim0_layout", _dim0_floor), ("copy_out_dim0", _copy_out_param_major)])
def test_dim0_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(dim0, name, fn)
    assert _fails(DIM0_PINS), fn.__name__


def test_dim0_pins_pass_the_oracle_itself():
    assert not _fails(DIM0_PINS)


# ---- the composed step

def _step_casts_input(rows, theta, m, v, t, hp, exact_mean=True):  # casts the old master
    g = reduce.mean_exact(rows) if exact_mean else reduce.mean_seq32(rows)
    th1, m1, v1 = adamw.adamw_step(theta, m, v, g, t, hp)
    return g, th1, m1, v1, bf16.to_bf16_bits(theta)


def _step_sum_not_mean(rows, theta, m, v, t, hp, exact_mean=True):
    g = reduce.decode_rows(rows).astype(np.float64).sum(axis=0).astype(np.float32)
    th1, m1, v1 = adamw.adamw_step(theta, m, v, g, t, hp)
    return g, th1, m1, v1, bf16.to_bf16_bits(th1)


@pytest.mark.parametrize("fn", [_step_casts_input, _step_sum_not_mean])
def test_step_pins_catch(monkeypatch, fn):
    monkeypatch.setattr(step, "sharded_step", fn)
    assert _fails([pins_adamw.test_worked_example_from_the_page,
                   pins_adamw.test_composed_step_matches_torch_over_steps]), fn.__name__


def test_step_pins_pass_the_oracle_itself():
    assert not _fails([pins_adamw.test_worked_example_from_the_page,
                       pins_adamw.test_composed_step_matches_torch_over_steps])


# ---- the memory and communication ledger

def _ledger_zero2_grads_whole(params, world, stage, k=12, fp32_grad_accum=False):
    p, n = Fraction(params), Fraction(world)
    base = {0: 4 * p + k * p, 1: 4 * p + k * p / n, 2: 4 * p + k * p / n, 3: (4 * p + k * p) / n}[stage]
    extra = (4 * p if stage <= 1 else 4 * p / n) if fp32_grad_accum else 0
    return base + extra


def _comm_zero3_like_zero2(params, stage):
    return 2 * Fraction(params)


def _ring_whole_buffer(buffer_size, world):
    return Fraction(buffer_size)



def _ledger_pins():
    fixtures = ["ledger_dpz_7p5b_n64.txt", "ledger_dpz_1p5b_n8.txt"]
    out = [pins_ledger.test_dpz_exact_zero3_value, pins_ledger.test_l5_7b_table_and_printout,
           pins_ledger.test_laf_7b_4gpu_table, pins_ledger.test_zvf_70b_context,
           pins_ledger.test_fp32_accumulation_extra, pins_ledger.test_n64_fractions_and_limits,
           pins_ledger.test_ring_phase_model]
    out += [lambda f=f: pins_ledger.test_dpz_printed_ledger(f) for f in fixtures]
    return out


@pytest.mark.parametrize("name,fn", [("state_bytes", _ledger_zero2_grads_whole),
                                     ("comm_elements", _comm_zero3_like_zero2),
                                     ("ring_phase", _ring_whole_buffer)])
def test_ledger_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(ledger, name, fn)
    assert _fails(_ledger_pins()), fn.__name__


def test_ledger_pins_pass_the_oracle_itself():
    assert not _fails(_ledger_pins())


# ---- the remaining helpers: sum of squares, windows, pack, copy-out, dim-0 counts

def _sumsq_abs(g):  # sum of magnitudes instead of squares
    return float(np.abs(np.asarray(g, dtype=np.float64)).sum())


def _sumsq_fp32(g):  # accumulated in fp32
    s = np.float32(0.0)
    for x in np.asarray(g, dtype=np.float32):
        s = np.float32(s + x * x)
    return float(s)


@pytest.mark.parametrize("fn", [_sumsq_abs, _sumsq_fp32])
def test_sumsq_pins_catch(monkeypatch, fn):
    monkeypatch.setattr(reduce, "sumsq", fn)
    assert _fails([pins_reduce.test_sumsq_matches_exact_sum,
                   pins_accumulate.test_clip_matches_torch_clip_grad_norm]), fn.__name__


def _window_shifted(fetch, numels, f0, f1, dtype=np.float32):  # reads one element late
    lay = layout.flat_layout(numels, 1)
    out = np.zeros(max(f1 - f0, 0), dtype=dtype)
    for i, (off, n) in enumerate(zip(lay.offsets, numels)):
        a, b = max(f0, off), min(f1, off + int(n))
        if a < b:
            src = fetch(i, min(a - off + 1, int(n)), min(b - off + 1, int(n)))
            out[a - f0:a - f0 + src.size] = src
    return out


def _pack_keeps_moments(params, world, rank):  # returns the master slice as m and v too
    master, _, _ = _orig_pack_shard(params, world, rank)
    return master, master.copy(), master.copy()


def _copy_out_drops_last(gathered, shapes_):
    sizes = [int(np.prod(s)) if len(s) else 1 for s in shapes_]
    lay = layout.flat_layout(sizes, 1)
    outs = []
    for off, n, shape in zip(lay.offsets, sizes, shapes_):
        a = gathered[off:off + n].copy()
        if n:
            a[-1] = 0
        outs.append(a.reshape(shape))
    return outs


_orig_pack_shard = layout.pack_shard


@pytest.mark.parametrize("name,fn", [("flat_window", _window_shifted), ("pack_shard", _pack_keeps_moments),
                                     ("copy_out", _copy_out_drops_last)])
def test_layout_helper_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(layout, name, fn)
    assert _fails(LAYOUT_PINS), fn.__name__


def _valid_off_by_one(numel, chunk, rank):  # counts one padding element as real
    return max(0, min(chunk, numel - rank * chunk + 1))


def test_dim0_valid_pins_catch(monkeypatch):
    monkeypatch.setattr(dim0, "valid", _valid_off_by_one)
    assert _fails(DIM0_PINS)


def _exact_mean_divides_by_ranks(rows_per_microbatch):  # forgets the micro-batch count
    tot, n = None, 0
    for rows in rows_per_microbatch:
        c = reduce.decode_rows(rows).astype(np.float64)
        tot = c.sum(axis=0) if tot is None else tot + c.sum(axis=0)
        n = c.shape[0]
    return (tot / n).astype(np.float32)


def _global_norm_max(partials):  # the largest shard's norm instead of the global one
    return float(np.sqrt(max(float(p) for p in partials)))


@pytest.mark.parametrize("name,fn", [("exact_mean_over_microbatches", _exact_mean_divides_by_ranks),
                                     ("global_norm", _global_norm_max)])
def test_accumulate_helper_pins_catch(monkeypatch, name, fn):
    monkeypatch.setattr(accumulate, name, fn)
    assert _fails(ACCUM_PINS + [pins_accumulate.test_exact_mean_over_microbatches_is_rounded_once]), fn.__name__
