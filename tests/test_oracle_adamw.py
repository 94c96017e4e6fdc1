"""Pins of the oracle's AdamW and of the composed step."""
import numpy as np
import pytest
import torch

from oracle import adamw, bf16, layout, reduce, step
from synth import gen
from _golden import all_of, first

HP = adamw.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_matches_torch_adamw_fp64_over_ten_steps():
    # torch.optim.AdamW implements decoupled decay + bias-corrected Adam; with the
    # oracle's state kept in fp64 the two must agree to fp64 rounding.
    n = 4096
    theta0 = gen.host_normal(1, n, 0.02).astype(np.float64)
    p = torch.nn.Parameter(torch.from_numpy(theta0.copy()))
    opt = torch.optim.AdamW([p], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                            weight_decay=HP.weight_decay, foreach=False, fused=False)
    th, m, v = theta0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 11):
        g = gen.host_normal(100 + t, n, 1e-3).astype(np.float64)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        th_prev, m_prev = th, m
        th, m, v = adamw.adamw_step(th, m, v, g, t, HP, state_dtype=np.float64)
        st = opt.state[p]
        # torch forms m' as m + (1-b1)(g - m), which cancels; compare on the scale
        # of the terms rather than of the result
        m_scale = HP.beta1 * np.abs(m_prev) + (1 - HP.beta1) * np.abs(g)
        th_scale = np.abs(th_prev) + HP.lr
        assert np.all(np.abs(st["exp_avg"].numpy() - m) <= 1e-12 * m_scale)
        assert np.all(np.abs(st["exp_avg_sq"].numpy() - v) <= 1e-13 * v)
        assert np.all(np.abs(p.detach().numpy() - th) <= 1e-12 * th_scale)


def test_closed_form_first_step():
    # from m = v = 0: m1 = (1-b1) g, v1 = (1-b2) g^2, m_hat = g, v_hat = g^2, so
    # theta1 = theta0 (1 - lr wd) - lr g / (|g| + eps)
    g = gen.host_normal(2, 1000, 1e-3)
    th0 = gen.host_normal(3, 1000, 0.02)
    z = np.zeros_like(g)
    th1, m1, v1 = adamw.adamw_step(th0, z, z, g, 1, HP, state_dtype=np.float64)
    g64, t64 = g.astype(np.float64), th0.astype(np.float64)
    assert np.allclose(m1, 0.1 * g64, rtol=1e-15)
    assert np.allclose(v1, 0.001 * g64 * g64, rtol=1e-12)
    want = t64 * (1 - 1e-3 * 0.01) - 1e-3 * g64 / (np.abs(g64) + 1e-8)
    assert np.allclose(th1, want, rtol=1e-12, atol=1e-18)
    # for |g| >> eps the step is lr * sign(g)
    assert np.allclose(th1, t64 * (1 - 1e-5) - 1e-3 * np.sign(g64), rtol=0, atol=1e-3 * 1e-8 / 1e-6 * 20)


def test_special_cases():
    th0 = gen.host_normal(4, 512, 0.02)
    m0 = gen.host_normal(5, 512, 1e-4)
    v0 = np.abs(gen.host_normal(6, 512, 1e-7))
    g = gen.host_normal(7, 512, 1e-3)
    # lr = 0 and wd = 0: theta unchanged bitwise, moments still advance
    th1, m1, v1 = adamw.adamw_step(th0, m0, v0, g, 3, adamw.HParams(lr=0.0, weight_decay=0.0))
    assert np.array_equal(th1, th0) and not np.array_equal(m1, m0)
    # g = 0 with zero moments: pure decay theta (1 - lr wd)
    z = np.zeros_like(th0)
    th1, m1, v1 = adamw.adamw_step(th0, z, z, z, 1, HP)
    assert np.array_equal(th1, (th0.astype(np.float64) * (1 - HP.lr * HP.weight_decay)).astype(np.float32))
    assert not m1.any() and not v1.any()
    # b1 = b2 = 0: theta - lr g / (|g| + eps), at every step t
    hp0 = adamw.HParams(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0)
    th1, _, _ = adamw.adamw_step(th0, m0, v0, g, 5, hp0, state_dtype=np.float64)
    g64 = g.astype(np.float64)
    assert np.allclose(th1, th0 - 1e-3 * g64 / (np.abs(g64) + 1e-8), rtol=1e-14, atol=1e-18)


def test_zero_padding_stays_zero_bitwise():
    z = np.zeros(8, np.float32)
    th, m, v = z.copy(), z.copy(), z.copy()
    for t in range(1, 20):
        th, m, v = adamw.adamw_step(th, m, v, z, t, adamw.HParams(weight_decay=0.1))
        for a in (th, m, v):
            assert not a.view(np.uint32).any()
        assert not bf16.to_bf16_bits(th).any()


def test_worked_example_from_the_page():
    f = "worked_example_dpz_4x8.txt"
    world = int(first(f, "world")[0])
    theta0 = np.array([float(x) for x in first(f, "theta0")], dtype=np.float32)
    grads = np.zeros((world, theta0.size), dtype=np.float32)
    for rec in all_of(f, "grad_hundredths"):
        grads[int(rec[0])] = [int(x) / 100.0 for x in rec[1:]]
    lr, b1, b2, eps, wd, t = (float(x) for x in first(f, "hparams"))
    hp = adamw.HParams(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    want_g = [float(x) for x in first(f, "mean_grad_4dp")]
    want_th = [float(x) for x in first(f, "updated_6dp")]

    # with fp32 contributions the mean matches the page at 4 decimals
    g = reduce.mean_exact(grads)
    assert [round(float(x), 4) for x in g] == want_g
    # unsharded update
    z = np.zeros_like(theta0)
    full, m_full, v_full = adamw.adamw_step(theta0, z, z, g, int(t), hp)
    assert [round(float(x), 6) for x in full] == want_th
    # sharded update: each rank updates its own two elements; gathered result is
    # identical (max_abs_diff = 0) and each rank holds 4 of the 16 m/v scalars
    lay = layout.flat_layout([theta0.size], world)
    parts, per_rank = [], []
    for r in range(world):
        sl = slice(r * lay.shard, (r + 1) * lay.shard)
        th_r, m_r, v_r = adamw.adamw_step(theta0[sl], z[sl], z[sl], g[sl], int(t), hp)
        parts.append(th_r)
        per_rank.append(m_r.size + v_r.size)
    gathered = np.concatenate(parts)
    assert float(np.max(np.abs(gathered - full))) == float(first(f, "max_abs_diff")[0])
    assert m_full.size + v_full.size == int(first(f, "mv_scalars_unsharded")[0])
    assert per_rank == [int(first(f, "mv_scalars_sharded")[0])] * world

    # with bf16 contributions (the build's input type) the updated parameters
    # still agree with the page at 6 decimals
    rows = bf16.to_bf16_bits(grads)
    _, th_b, _, _, _ = step.sharded_step(rows, theta0, z, z, int(t), hp)
    assert [round(float(x), 6) for x in th_b] == want_th


def test_composed_step_matches_torch_over_steps():
    # The rank's step -- mean of N bf16 contributions, AdamW on its fp32 slice,
    # bf16 of the new master -- against torch: the mean of the decoded rows in
    # fp64, torch.optim.AdamW in fp64 started each step from the oracle's fp32
    # state, and torch's own fp32 -> bf16 cast.
    world, n = 4, 2048
    theta = gen.host_normal(31, n, 0.02)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.zeros(n, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                            weight_decay=HP.weight_decay, foreach=False, fused=False)
    for t in range(1, 6):
        rows = gen.host_grad_rows(40 + t, world, n, "bf16")
        with torch.no_grad():
            p.copy_(torch.from_numpy(theta.astype(np.float64)))
            if t > 1:
                opt.state[p]["exp_avg"].copy_(torch.from_numpy(m.astype(np.float64)))
                opt.state[p]["exp_avg_sq"].copy_(torch.from_numpy(v.astype(np.float64)))
        g, theta, m, v, out = step.sharded_step(rows, theta, m, v, t, HP)
        rows_t = torch.from_numpy(rows.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
        want_g = rows_t.mean(dim=0).to(torch.float32)
        assert np.array_equal(g, want_g.numpy())
        p.grad = want_g.to(torch.float64)
        opt.step()
        want = p.detach().numpy()
        # the oracle rounds m and v to fp32 before it forms the update, torch
        # does not: half an ulp of theta plus 2^-22 of the update's size
        r = (np.abs(m.astype(np.float64)) / (1 - HP.beta1 ** t)
             / (np.sqrt(v.astype(np.float64) / (1 - HP.beta2 ** t)) + HP.eps))
        bound = 0.5 * np.spacing(np.abs(theta)).astype(np.float64) + 2.0 ** -22 * HP.lr * r
        assert np.all(np.abs(theta.astype(np.float64) - want) <= bound)
        # moments: one rounding of the same fp64 value up to the order of its two
        # terms (torch forms m + (1 - beta1)(g - m)); bf16-short gradients put
        # some of them on an exact fp32 tie, which that order may decide
        for mine, key in ((m, "exp_avg"), (v, "exp_avg_sq")):
            ref = opt.state[p][key].numpy()
            tie = (0.5 + 2.0 ** -20) * np.spacing(np.abs(mine)).astype(np.float64)
            assert np.all(np.abs(mine.astype(np.float64) - ref) <= tie)
        want_b = torch.from_numpy(theta).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
        assert np.array_equal(out, want_b)


def test_error_scales_bound_a_perturbed_update():
    # an fp32 re-evaluation of the same formula (a different rounding sequence)
    # stays well inside 1e-6 of the scales -- the tolerance is not vacuous and
    # not too tight for an fp32 kernel.
    n = 20000
    th = gen.host_normal(8, n, 0.02)
    m = gen.host_normal(9, n, 1e-4)
    v = np.abs(gen.host_normal(10, n, 1e-7))
    g = gen.host_normal(11, n, 1e-3)
    t = 7
    th1, m1, v1 = adamw.adamw_step(th, m, v, g, t, HP)
    f = np.float32
    bc1, bc2 = 1 - HP.beta1 ** t, 1 - HP.beta2 ** t
    mm = f(HP.beta1) * m + f(1 - HP.beta1) * g
    vv = f(HP.beta2) * v + f(1 - HP.beta2) * g * g
    den = np.sqrt(vv) * f(1 / np.sqrt(bc2)) + f(HP.eps)
    th32 = th * f(1 - HP.lr * HP.weight_decay) - f(HP.lr / bc1) * mm / den
    st, sm, sv = adamw.error_scales(th, m, g, t, HP, m1, v1)
    assert np.all(np.abs(th32.astype(np.float64) - th1) <= 1e-6 * st)
    assert np.all(np.abs(mm.astype(np.float64) - m1) <= 1e-6 * sm)
    assert np.all(np.abs(vv.astype(np.float64) - v1) <= 1e-6 * sv)
    # while a dropped bias correction (one plausible slip) is far outside
    th_bad = th * f(1 - HP.lr * HP.weight_decay) - f(HP.lr) * mm / (np.sqrt(vv) + f(HP.eps))
    assert np.any(np.abs(th_bad.astype(np.float64) - th1) > 1e-6 * st)


@pytest.mark.parametrize("bad", [dict(lr=float("nan")), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=-1.0)])
def test_bad_hparams(bad):
    z = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        adamw.adamw_step(z, z, z, z, 1, adamw.HParams(**bad))
    with pytest.raises(ValueError):
        adamw.adamw_step(z, z, z, z, 0, HP)
