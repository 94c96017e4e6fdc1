"""Pins of the oracle's memory/communication ledger against values the pages print."""
from fractions import Fraction

import pytest

from oracle import ledger
from _golden import all_of, first

STAGE_OF = {"DDP": 0, "ZeRO-1": 1, "ZeRO-2": 2, "ZeRO-3": 3}


@pytest.mark.parametrize("fixture", ["ledger_dpz_7p5b_n64.txt", "ledger_dpz_1p5b_n8.txt"])
def test_dpz_printed_ledger(fixture):
    params = int(first(fixture, "params")[0])
    world = int(first(fixture, "world")[0])
    for name, bpp, gb, saving, comm in all_of(fixture, "row"):
        st = STAGE_OF[name]
        assert ledger.fmt(ledger.bytes_per_param(world, st), 4) == bpp
        state = ledger.state_bytes(params, world, st)
        assert state == params * ledger.bytes_per_param(world, st)
        assert ledger.fmt(ledger.to_gb(state), 2) == gb
        assert ledger.fmt(ledger.saving_vs_ddp(world, st), 2) == saving
        assert ledger.fmt(ledger.to_gb(ledger.comm_bytes(params, st)), 2) == comm


def test_dpz_exact_zero3_value():
    params = int(first("ledger_dpz_7p5b_n64.txt", "params")[0])
    _, exact = first("ledger_dpz_7p5b_n64.txt", "exact_gb")
    assert ledger.to_gb(ledger.state_bytes(params, 64, 3)) == Fraction(exact)
    # every figure of that run exactly, as rationals
    assert ledger.to_gb(ledger.state_bytes(params, 64, 0)) == 120
    assert ledger.to_gb(ledger.state_bytes(params, 64, 1)) == Fraction("31.40625")
    assert ledger.to_gb(ledger.state_bytes(params, 64, 2)) == Fraction("16.640625")


def test_l5_7b_table_and_printout():
    f = "ledger_l5_7b.txt"
    params = int(first(f, "params")[0])
    for n, z0, z1, z2, z3 in all_of(f, "table"):
        n = int(n)
        for st, shown in zip(range(4), (z0, z1, z2, z3)):
            exact = ledger.to_gb(ledger.state_bytes(params, n, st))
            # a displayed table value is the exact value rounded at its last shown digit
            digits = len(shown.split(".")[1])
            assert abs(exact - Fraction(shown)) <= Fraction(1, 2 * 10 ** digits)
    for n, st, gb in all_of(f, "exact"):
        assert ledger.to_gb(ledger.state_bytes(params, int(n), int(st))) == Fraction(gb)
    for n, z1, z2, z3, comm in all_of(f, "printed"):
        n = int(n)
        got = [ledger.fmt(ledger.to_gb(ledger.state_bytes(params, n, st)), 1) for st in (1, 2, 3)]
        assert got == [z1, z2, z3]
        assert ledger.fmt(ledger.comm_elements(params, 3) / 10 ** 9, 1) == comm
    for st, val in all_of(f, "comm_elements"):
        assert ledger.comm_elements(params, int(st)) / 10 ** 9 == Fraction(val)
    for st, val in all_of(f, "comm_bytes"):
        assert ledger.to_gb(ledger.comm_bytes(params, int(st))) == Fraction(val)
    z3_70b = Fraction(first(f, "z3_70b_n64")[0])
    assert ledger.to_gb(ledger.state_bytes(70 * 10 ** 9, 64, 3)) == z3_70b


def test_laf_7b_4gpu_table():
    p = 7 * 10 ** 9
    for name, st, world, par, grad, opt, total in all_of("ledger_laf_7b_4gpu.txt", "row"):
        st, world = int(st), int(world)
        assert ledger.to_gb(ledger.state_bytes(p, world, st)) == Fraction(total)
        # components: params replicated below stage 3, grads sharded from stage 2
        par_exp = Fraction(2 * p, world if st == 3 else 1)
        grad_exp = Fraction(2 * p, world if st >= 2 else 1)
        opt_exp = Fraction(12 * p, world if st >= 1 else 1)
        assert ledger.to_gb(par_exp) == Fraction(par)
        assert ledger.to_gb(grad_exp) == Fraction(grad)
        assert ledger.to_gb(opt_exp) == Fraction(opt)
        assert par_exp + grad_exp + opt_exp == ledger.state_bytes(p, world, st)


def test_zvf_70b_context():
    f = "ledger_zvf_70b.txt"
    p = int(first(f, "params")[0])
    assert ledger.to_gb(ledger.state_bytes(p, 1, 0)) == Fraction(first(f, "total_gb")[0])
    assert ledger.to_gb(2 * p) == Fraction(first(f, "weights_gb")[0])
    assert ledger.to_gb(12 * p) == Fraction(first(f, "optimizer_gb")[0])
    assert ledger.to_gb(ledger.state_bytes(p, 64, 3)) == Fraction(first(f, "z3_n64_gb")[0])


def test_stages_equal_at_one_rank():
    # the calculator exercise's own cross-check: at dp = 1 stages 1..3 coincide
    for p in (1, 10 ** 6, 7 * 10 ** 9):
        vals = {ledger.state_bytes(p, 1, st) for st in (0, 1, 2, 3)}
        assert vals == {16 * p}


def test_fp32_accumulation_extra():
    p, n = 7 * 10 ** 9, 8
    for st in (0, 1):
        d = ledger.state_bytes(p, n, st, fp32_grad_accum=True) - ledger.state_bytes(p, n, st)
        assert d == 4 * p
    for st in (2, 3):
        d = ledger.state_bytes(p, n, st, fp32_grad_accum=True) - ledger.state_bytes(p, n, st)
        assert d == Fraction(4 * p, n)


def test_n64_fractions_and_limits():
    # Lesson 5 s2: at N=64 optimizer state 12P -> 0.1875P, totals ~4.19P (saves ~74%)
    # and ~2.22P (~86%); stage 2 saves 2P(1 - 1/N) of gradient memory over stage 1.
    p = 1
    assert Fraction(12, 64) == Fraction("0.1875")
    z1 = ledger.state_bytes(p, 64, 1)
    z2 = ledger.state_bytes(p, 64, 2)
    assert ledger.fmt(z1, 2) == "4.19" and ledger.fmt(z2, 2) == "2.22"
    assert round(float(1 - z1 / 16) * 100) == 74
    assert round(float(1 - z2 / 16) * 100) == 86
    for n in (2, 8, 64, 1024):
        assert ledger.state_bytes(10, n, 1) - ledger.state_bytes(10, n, 2) == 2 * 10 * (1 - Fraction(1, n))
    # limits N -> infinity: stage 1 -> 4P (at most 4x), stage 2 -> 2P (at most 8x)
    big = 10 ** 12
    assert abs(ledger.saving_vs_ddp(big, 1) - 4) < Fraction(1, 10 ** 9)
    assert abs(ledger.saving_vs_ddp(big, 2) - 8) < Fraction(1, 10 ** 9)
    assert ledger.saving_vs_ddp(64, 3) == 64


def test_ring_phase_model():
    # DP-and-ZeRO page s3.4: each ring phase moves (N-1)/N of the buffer; all-reduce = 2 phases
    g = 10 ** 9
    assert ledger.ring_phase(g, 1) == 0
    assert ledger.ring_phase(g, 4) == Fraction(3 * g, 4)
    assert 2 * ledger.ring_phase(g, 64) == Fraction(2 * 63 * g, 64)
    assert ledger.comm_elements(5, 0) == ledger.comm_elements(5, 1) == ledger.comm_elements(5, 2) == 10
    assert ledger.comm_elements(5, 3) == 15


@pytest.mark.parametrize("args", [(0, 8, 1), (-5, 8, 1), (10, 0, 1), (10, 8, 4), (10, 8, -1)])
def test_errors(args):
    with pytest.raises(ValueError):
        ledger.state_bytes(*args)
