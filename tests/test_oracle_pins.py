"""Pins of the CPU oracle against what mathematics fixes (no GPU).

* exact-rational brute force on tiny heads (logits, argmax with exact ties),
* high-precision logsumexp of the exact logits (mpmath),
* closed forms: zero row, one-hot row, identical columns, power-of-two scale,
* invariants: per-lane combine = global argmax, lane-count invariance,
  exp(log-probs) sums to 1,
* mutation checks: plausible mistakes planted in a copy of the oracle make at
  least one pin fail.
"""
import math

import mpmath
import numpy as np
import pytest

import oracle
from logit_source_projection_amd import inputs
from fractions import Fraction

from tests.exact import bf16_to_fraction, exact_argmax, exact_logits


def tiny_head(B, H, V, seed, sigma_w=0.5):
    x = inputs.draw_hidden(B, H, seed)
    w = inputs.draw_weight(H, V, sigma_w, seed)
    return x, w


# ----------------------------------------------------------------------------
# pin helpers (each raises AssertionError on a mismatch); the mutation tests
# run them against deliberately broken copies of the oracle.
# ----------------------------------------------------------------------------

def pin_logits_exact(logits_fn, x, w):
    z = logits_fn(x, w)
    ze = exact_logits(x, w)
    H = x.shape[1]
    for b in range(x.shape[0]):
        for v in range(w.shape[1]):
            # error bound of an fp64 sum of H exact products
            mag = sum(abs(bf16_to_fraction(x[b, h]) * bf16_to_fraction(w[h, v]))
                      for h in range(H))
            bound = float(mag) * H * 2.0 ** -52
            assert abs(z[b, v] - float(ze[b][v])) <= bound, (b, v)


def pin_ids_exact(logits_fn, project_fn, x, w, lane_off):
    z = logits_fn(x, w)
    r = project_fn(z, lane_off)
    ze = exact_logits(x, w)
    for b in range(x.shape[0]):
        assert int(r["ids"][b]) == exact_argmax(ze[b]), b


def pin_lanes_exact(logits_fn, project_fn, x, w, lane_off):
    """Per-lane results against the exact rationals: lane_arg is the lowest
    global index of the exact maximum inside the lane, lane_max that maximum
    (within the fp64 error of a sum of H exact products), and the lane
    sum-exp is sum exp(z - lane_max) over the lane."""
    z = logits_fn(x, w)
    r = project_fn(z, lane_off)
    ze = exact_logits(x, w)
    for b in range(x.shape[0]):
        tol = _fp64_bound(x, w, b) + 1e-300
        for i in range(len(lane_off) - 1):
            seg = ze[b][lane_off[i]:lane_off[i + 1]]
            best = max(seg)
            assert int(r["lane_arg"][b, i]) == lane_off[i] + seg.index(best), (b, i)
            assert abs(float(r["lane_max"][b, i]) - float(best)) <= tol, (b, i)
            se = math.fsum(math.exp(float(q - best)) for q in seg)
            assert abs(float(r["lane_sumexp"][b, i]) - se) <= 1e-12 * se, (b, i)


def _fp64_bound(x, w, b):
    """Largest error bound over row b of an fp64 sum of H exact products."""
    H = x.shape[1]
    xs = [abs(bf16_to_fraction(x[b, h])) for h in range(H)]
    worst = 0
    for v in range(w.shape[1]):
        mag = sum(xs[h] * abs(bf16_to_fraction(w[h, v])) for h in range(H))
        worst = max(worst, mag)
    return float(worst) * H * 2.0 ** -52


def pin_gap_exact(logits_fn, project_fn, x, w, lane_off):
    """top2_gap and near_tie on every row against the exact rationals: the gap
    is the largest exact logit minus the next largest (distinct indices), and
    the flag is gap < 2e-3 * max |z| unless the exact gap sits within the fp64
    error of the threshold."""
    z = logits_fn(x, w)
    r = project_fn(z, lane_off)
    ze = exact_logits(x, w)
    for b in range(x.shape[0]):
        srt = sorted(ze[b], reverse=True)
        gap = srt[0] - srt[1]
        tol = 2 * _fp64_bound(x, w, b) + 1e-300
        assert abs(float(r["gap"][b]) - float(gap)) <= tol, (b, r["gap"][b], float(gap))
        thr = Fraction(oracle.NEAR_TIE_REL) * max(abs(q) for q in ze[b])
        if abs(float(gap - thr)) > 2 * tol:
            assert bool(r["near_tie"][b]) == (gap < thr), (b, float(gap), float(thr))


def threshold_head():
    """One-hot rows (z[b, :] = W[h_b, :] exactly) whose top-2 gaps sit just
    below, exactly at and just above the near-tie threshold.  Column 7 holds
    -500 in every row, so max |z| = 500 and the threshold is 2e-3 * 500 = 1.0
    (exact in fp64); the rows' largest logits are 4.0.

      row 0: 4.0 vs 3.015625           gap 0.984375  -> near tie
      row 1: 4.0 vs 2.984375           gap 1.015625  -> not a near tie
      row 2: 4.0 vs 3.0                gap 1.0 (at)  -> not a near tie (strict)
      row 3: 4.0 vs 4.0                gap 0         -> near tie
      row 4: 500 vs 4.0 (no -500)      gap 496       -> not a near tie
    Rows 0-2 also hold a third value 2.5 (gap to the largest 1.5 > 1), so a
    gap taken to the third largest would misclassify row 0.
    Returns (x, w, off, expected gaps, expected flags)."""
    H, V = 8, 48
    rng = np.random.default_rng(77)
    w32 = (rng.standard_normal((H, V)) * 0.02).astype(np.float32)
    w = inputs.f32_to_bf16_bits(w32)
    x = np.zeros((5, H), dtype=np.uint16)
    def bits(v):
        return np.uint16(inputs.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])
    one = bits(1.0)
    top = [(3.015625, 2.5), (2.984375, 2.5), (3.0, 2.5), (4.0, None)]
    for b, (second, third) in enumerate(top):
        x[b, b] = one
        w[b, 7] = bits(-500.0)
        w[b, 11] = bits(4.0)
        w[b, 40] = bits(second)
        if third is not None:
            w[b, 25] = bits(third)
    x[4, 4] = one
    w[4, 30] = bits(500.0)
    w[4, 31] = bits(4.0)
    gaps = [0.984375, 1.015625, 1.0, 0.0, 496.0]
    flags = [True, False, False, True, False]
    return x, w, [0, 16, 48], gaps, flags


def pin_near_tie_threshold(logits_fn, project_fn):
    x, w, off, gaps, flags = threshold_head()
    z = logits_fn(x, w)
    r = project_fn(z, off)
    for b, (gp, fl) in enumerate(zip(gaps, flags)):
        assert float(r["gap"][b]) == gp, (b, r["gap"][b], gp)
        assert bool(r["near_tie"][b]) == fl, (b, r["near_tie"][b], fl)


def pin_lse_mp(logits_fn, project_fn, x, w, lane_off):
    z = logits_fn(x, w)
    r = project_fn(z, lane_off)
    ze = exact_logits(x, w)
    mpmath.mp.dps = 40
    for b in range(x.shape[0]):
        s = mpmath.fsum(mpmath.exp(mpmath.mpf(q.numerator) / q.denominator) for q in ze[b])
        lse = float(mpmath.log(s))
        assert abs(r["lse"][b] - lse) <= 1e-12 * max(1.0, abs(lse)), (b, r["lse"][b], lse)
        top = max(ze[b])
        sel = float(mpmath.mpf(top.numerator) / top.denominator - mpmath.log(s))
        assert abs(r["sel_lp"][b] - sel) <= 1e-12 * max(1.0, abs(sel)), b


TINY_CASES = [
    # B, H, V, lane offsets, seed
    (3, 16, 40, [0, 40], 1),
    (4, 32, 96, [0, 50, 96], 2),
    (2, 64, 130, [0, 33, 64, 130], 3),
    (4, 24, 512, [0, 200, 300, 512], 4),
]


@pytest.mark.parametrize("B,H,V,off,seed", TINY_CASES)
def test_logits_match_exact_rationals(B, H, V, off, seed):
    x, w = tiny_head(B, H, V, seed)
    pin_logits_exact(oracle.logits, x, w)


@pytest.mark.parametrize("B,H,V,off,seed", TINY_CASES)
def test_ids_match_exact_argmax(B, H, V, off, seed):
    x, w = tiny_head(B, H, V, seed)
    pin_ids_exact(oracle.logits, oracle.project, x, w, off)


@pytest.mark.parametrize("B,H,V,off,seed", TINY_CASES)
def test_top2_gap_and_near_tie_match_exact_rationals(B, H, V, off, seed):
    x, w = tiny_head(B, H, V, seed)
    pin_gap_exact(oracle.logits, oracle.project, x, w, off)


@pytest.mark.parametrize("B,H,V,off,seed", TINY_CASES)
def test_lane_results_match_exact_rationals(B, H, V, off, seed):
    x, w = tiny_head(B, H, V, seed)
    pin_lanes_exact(oracle.logits, oracle.project, x, w, off)


def test_lane_results_with_ties_inside_and_across_lanes():
    B, H, V = 3, 32, 64
    x, w = tiny_head(B, H, V, 7)
    off = [0, 20, 41, 64]
    inputs.plant_equal_columns(x, w, 2, (50, 30, 5), 40.0)  # one tied column per lane
    inputs.plant_equal_columns(x, w, 0, (39, 22), 40.0)     # a tie inside lane 1
    pin_lanes_exact(oracle.logits, oracle.project, x, w, off)


def test_near_tie_threshold_rows():
    pin_near_tie_threshold(oracle.logits, oracle.project)


def test_near_tie_gap_on_planted_ties_and_other_rows():
    """Exact ties (gap 0) and the other rows of the same head, every row
    against the exact rationals."""
    B, H, V = 4, 32, 64
    x, w = tiny_head(B, H, V, 7)
    inputs.plant_equal_columns(x, w, 2, (50, 30, 5), 40.0)
    inputs.plant_equal_columns(x, w, 0, (39, 22), 40.0)
    pin_gap_exact(oracle.logits, oracle.project, x, w, [0, 20, 41, 64])


@pytest.mark.parametrize("B,H,V,off,seed", TINY_CASES[:3])
def test_lse_matches_high_precision(B, H, V, off, seed):
    x, w = tiny_head(B, H, V, seed)
    pin_lse_mp(oracle.logits, oracle.project, x, w, off)


def test_exact_ties_go_to_lowest_index():
    B, H, V = 3, 32, 64
    x, w = tiny_head(B, H, V, 7)
    off = [0, 20, 41, 64]
    # columns 5, 30 and 50 identical and dominant for row 2 (three lanes)
    inputs.plant_equal_columns(x, w, 2, (50, 30, 5), 40.0)
    # row 0: dominant tie inside one lane, columns 22 and 39
    inputs.plant_equal_columns(x, w, 0, (39, 22), 40.0)
    z = oracle.logits(x, w)
    ze = exact_logits(x, w)
    r = oracle.project(z, off)
    assert ze[2][5] == ze[2][30] == ze[2][50] == max(ze[2])
    assert int(r["ids"][2]) == 5
    assert ze[0][22] == ze[0][39] == max(ze[0])
    assert int(r["ids"][0]) == 22
    assert r["gap"][2] == 0.0 and r["near_tie"][2]
    # lane view: every lane that holds one of the tied columns reports it
    assert list(r["lane_arg"][2]) == [5, 30, 50]


def test_zero_row_closed_form():
    B, H, V = 3, 48, 1000
    x, w = tiny_head(B, H, V, 11, sigma_w=0.02)
    x[1, :] = 0
    off = [0, 300, 1000]
    z = oracle.logits(x, w)
    assert np.all(z[1] == 0.0)
    r = oracle.project(z, off)
    assert r["ids"][1] == 0
    assert abs(r["lse"][1] - math.log(V)) <= 1e-13
    lp = oracle.logprobs(z, r["lse"])
    assert np.allclose(lp[1], -math.log(V), rtol=0, atol=1e-13)
    assert abs(r["sel_lp"][1] + math.log(V)) <= 1e-13


def test_one_hot_row_selects_weight_row():
    B, H, V = 4, 40, 777
    x, w = tiny_head(B, H, V, 12, sigma_w=0.02)
    one = np.uint16(inputs.f32_to_bf16_bits(np.array([1.0], dtype=np.float32))[0])
    for b, h in enumerate([0, 17, 39, 5]):
        x[b, :] = 0
        x[b, h] = one
    z = oracle.logits(x, w)
    for b, h in enumerate([0, 17, 39, 5]):
        wrow = np.array([float(bf16_to_fraction(v)) for v in w[h]])
        assert np.array_equal(z[b], wrow)
        r = oracle.project(z, [0, 100, 500, 777])
        assert int(r["ids"][b]) == int(np.argmax(wrow))


def test_power_of_two_scaling_is_exact():
    B, H, V = 4, 256, 2048
    x, w = tiny_head(B, H, V, 13, sigma_w=0.02)
    # doubling a bf16 value adds one to its exponent field (no overflow here)
    x2 = x.copy()
    nz = (x2 & 0x7FFF) != 0
    x2[nz] = x2[nz] + np.uint16(1 << 7)
    off = inputs.equal_lanes(V, 2)
    z, z2 = oracle.logits(x, w), oracle.logits(x2, w)
    assert np.array_equal(z2, 2.0 * z)
    r, r2 = oracle.project(z, off), oracle.project(z2, off)
    assert np.array_equal(r["ids"], r2["ids"])


@pytest.mark.parametrize("k", [2, 3, 4, 7])
def test_lane_count_invariance(k):
    B, H, V = 5, 128, 5003
    x, w = tiny_head(B, H, V, 21, sigma_w=0.05)
    z = oracle.logits(x, w)
    r1 = oracle.project(z, [0, V])
    rk = oracle.project(z, inputs.equal_lanes(V, k))
    assert np.array_equal(r1["ids"], rk["ids"])
    assert np.allclose(r1["lse"], rk["lse"], rtol=1e-12, atol=0)


def test_logprobs_exponentiate_to_one():
    B, H, V = 6, 256, 4096
    x, w = tiny_head(B, H, V, 22, sigma_w=0.05)
    z = oracle.logits(x, w)
    r = oracle.project(z, inputs.equal_lanes(V, 2))
    lp = oracle.logprobs(z, r["lse"])
    for b in range(B):
        assert abs(math.fsum(np.exp(lp[b])) - 1.0) <= 1e-6
        assert lp[b, r["ids"][b]] == lp[b].max()


def test_lane_results_match_global_view():
    B, H, V = 4, 64, 3001
    x, w = tiny_head(B, H, V, 23)
    off = [0, 1000, 1001, 2500, 3001]  # includes a one-column lane
    z = oracle.logits(x, w)
    r = oracle.project(z, off)
    for b in range(B):
        for i in range(4):
            seg = z[b, off[i]:off[i + 1]]
            assert r["lane_arg"][b, i] == off[i] + int(np.argmax(seg))
            assert r["lane_max"][b, i] == seg.max()
        assert r["ids"][b] == int(np.argmax(z[b]))


def test_sampled_rows_equal_full_evaluation():
    B, H, V = 9, 96, 1500
    x, w = tiny_head(B, H, V, 24)
    z = oracle.logits(x, w)
    zs = oracle.logits(x, w, rows=[8, 0, 3])
    assert np.array_equal(zs, z[[8, 0, 3]])


def test_tiny_workload_forced_tie():
    d = inputs.make_workload("tiny")
    z = oracle.logits(d["x"], d["w"])
    r = oracle.project(z, d["lane_off"])
    row, a, b = d["planted"][0]
    assert z[row, a] == z[row, b] == z[row].max()
    assert int(r["ids"][row]) == a == 1000
    assert r["near_tie"][row] and r["gap"][row] == 0.0


def test_rejects_bad_lanes():
    z = np.zeros((1, 10))
    for off in ([0, 5], [1, 10], [0, 5, 5, 10], [0, 7, 3, 10]):
        with pytest.raises(ValueError):
            oracle.project(z, off)


# ----------------------------------------------------------------------------
# Mutation checks: a broken copy of the oracle must fail at least one pin.
# ----------------------------------------------------------------------------

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


MUT_X, MUT_W = tiny_head(3, 16, 64, 31)
MUT_OFF = [0, 20, 64]


def test_mutation_dropped_term_is_caught():
    def bad_logits(x, w):
        z = oracle.logits(x, w)
        xl = oracle.bf16_bits_to_f64(x[:, -1])
        wl = oracle.bf16_bits_to_f64(w[-1, :])
        return z - np.outer(xl, wl)
    assert _fails(lambda: pin_logits_exact(bad_logits, MUT_X, MUT_W))


def test_mutation_transposed_operand_is_caught():
    xs, ws = tiny_head(3, 16, 16, 32)

    def bad_logits(x, w):
        return oracle.logits(x, np.ascontiguousarray(w.T))
    assert _fails(lambda: pin_logits_exact(bad_logits, xs, ws))


def test_mutation_wrong_sign_is_caught():
    def bad_logits(x, w):
        return -oracle.logits(x, w)
    assert _fails(lambda: pin_logits_exact(bad_logits, MUT_X, MUT_W))


def test_mutation_highest_index_tie_break_is_caught():
    x, w = MUT_X.copy(), MUT_W.copy()
    inputs.plant_equal_columns(x, w, 1, (3, 40), 40.0)

    def bad_project(z, off):
        r = oracle.project(z, off)
        zz = z[:, ::-1]
        last = z.shape[1] - 1 - np.argmax(zz, axis=1)
        r = dict(r)
        r["ids"] = last
        return r
    assert _fails(lambda: pin_ids_exact(oracle.logits, bad_project, x, w, MUT_OFF))


def test_mutation_lane_off_by_one_is_caught():
    x, w = MUT_X.copy(), MUT_W.copy()
    # the row maximum sits on the last column of lane 0
    inputs.plant_equal_columns(x, w, 0, (19,), 40.0)

    def bad_project(z, off):
        r = dict(oracle.project(z, off))
        M, A, S = oracle.lane_pairs(z, off)
        # off-by-one: lane 0 loses its last column
        for b in range(z.shape[0]):
            seg = z[b, off[0]:off[1] - 1]
            A[b, 0] = off[0] + int(np.argmax(seg))
            M[b, 0] = seg.max()
        ids, _ = oracle.combine(M, A, S)
        r["ids"] = ids
        return r
    assert _fails(lambda: pin_ids_exact(oracle.logits, bad_project, x, w, MUT_OFF))


def test_mutation_unscaled_lane_sum_is_caught():
    def bad_project(z, off):
        r = dict(oracle.project(z, off))
        M, A, S = oracle.lane_pairs(z, off)
        m = M.max(axis=1)
        r["lse"] = m + np.log(S.sum(axis=1))  # forgot exp(mf_i - m)
        r["sel_lp"] = z.max(axis=1) - r["lse"]
        return r
    assert _fails(lambda: pin_lse_mp(oracle.logits, bad_project, MUT_X, MUT_W, MUT_OFF))


# Planted mistakes in the top-2 gap and the near-tie flag.  Each replaces the
# oracle's gap / flag by a plausible wrong version and must fail a pin.
def _with_gap(gap_fn, flag_fn=None):
    def bad_project(z, off):
        r = dict(oracle.project(z, off))
        r["gap"] = gap_fn(z)
        r["near_tie"] = (flag_fn or oracle.near_tie)(z, r["gap"])
        return r
    return bad_project


def _gap_pins_fail(bad_project):
    x, w = tiny_head(4, 32, 96, 2)
    return (_fails(lambda: pin_near_tie_threshold(oracle.logits, bad_project)) and
            _fails(lambda: pin_gap_exact(oracle.logits, bad_project, x, w, [0, 50, 96])))


def test_mutation_swapped_gap_operands_is_caught():
    def swapped(z):
        top = np.partition(z, -2, axis=1)[:, -2:]
        return top[:, 0] - top[:, 1]
    assert _gap_pins_fail(_with_gap(swapped))


def test_mutation_gap_to_third_largest_is_caught():
    def third(z):
        top = np.partition(z, -3, axis=1)[:, -3:]
        return top[:, 2] - top[:, 0]
    assert _fails(lambda: pin_near_tie_threshold(oracle.logits, _with_gap(third)))


def test_mutation_threshold_without_abs_is_caught():
    def no_abs(z, gap):
        return gap < oracle.NEAR_TIE_REL * z.max(axis=1)
    bad = _with_gap(oracle.top2_gap, no_abs)
    assert _fails(lambda: pin_near_tie_threshold(oracle.logits, bad))


def test_mutation_non_strict_threshold_is_caught():
    def le(z, gap):
        return gap <= oracle.NEAR_TIE_REL * np.abs(z).max(axis=1)
    bad = _with_gap(oracle.top2_gap, le)
    assert _fails(lambda: pin_near_tie_threshold(oracle.logits, bad))


@pytest.mark.parametrize("factor", [2e-4, 2e-2])
def test_mutation_wrong_threshold_factor_is_caught(factor):
    def wrong(z, gap):
        return gap < factor * np.abs(z).max(axis=1)
    bad = _with_gap(oracle.top2_gap, wrong)
    assert _fails(lambda: pin_near_tie_threshold(oracle.logits, bad))


def test_mutation_lane_arg_highest_index_is_caught():
    x, w = tiny_head(3, 32, 64, 7)
    inputs.plant_equal_columns(x, w, 0, (39, 22), 40.0)

    def bad_project(z, off):
        r = dict(oracle.project(z, off))
        A = r["lane_arg"].copy()
        for i in range(len(off) - 1):
            seg = z[:, off[i]:off[i + 1]][:, ::-1]
            A[:, i] = off[i + 1] - 1 - np.argmax(seg, axis=1)
        r["lane_arg"] = A
        return r
    assert _fails(lambda: pin_lanes_exact(oracle.logits, bad_project, x, w, [0, 20, 41, 64]))


def test_mutation_lane_boundary_shift_is_caught():
    x, w = tiny_head(3, 32, 64, 8)
    # each row's largest logit on the first column of a lane
    inputs.plant_equal_columns(x, w, 0, (20,), 40.0)
    inputs.plant_equal_columns(x, w, 1, (41,), 40.0)

    def bad_project(z, off):
        shifted = [off[0]] + [o + 1 for o in off[1:-1]] + [off[-1]]
        r = dict(oracle.project(z, off))
        r2 = oracle.project(z, shifted)
        r["lane_arg"], r["lane_max"] = r2["lane_arg"], r2["lane_max"]
        return r
    assert _fails(lambda: pin_lanes_exact(oracle.logits, bad_project, x, w, [0, 20, 41, 64]))
