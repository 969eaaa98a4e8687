"""Pins of the oracle on non-finite logits (CPU).

The pages do not say what the argmax does with NaN or infinities.  The
reading taken is numpy's argmax order: a NaN ranks above every number (all
NaNs equal, so the first NaN wins), +inf above every finite value, -inf
below, and the lowest index among equal values.  Every row then has an ID
among its columns.  These tests pin the oracle's per-lane results, its fold
across lanes and its full-logit plan to

  * a brute-force argmax written from that definition (a sort key per
    column, compared with Python's max over the row's columns);
  * numpy's own argmax of the complete row;
  * the IEEE rules for NaN and infinities in the fp64 product
    (NaN * anything = NaN, 0 * inf = NaN, x * inf = +-inf by the sign of x).

A fold that takes the first lane equal to max_i M_i (NaN compares equal to
nothing) picks lane 0 on a row whose first NaN lies in a later lane; the
rows below put it in lanes 1 and 2 so that such a fold fails.
"""
import math

import numpy as np
import pytest

import oracle

NAN, INF = float("nan"), float("inf")


def brute_argmax(row):
    """Index of the largest entry in the order of the definition: the key
    (is NaN, value or 0 for NaN, -index) of every column, the largest key
    wins."""
    def key(i):
        v = row[i]
        return (math.isnan(v), 0.0 if math.isnan(v) else v, -i)
    return max(range(len(row)), key=key)


def rows_with_non_finite():
    """Rows of 12 columns (lanes [0, 5), [5, 8), [8, 12)) covering NaN in
    one lane, in several lanes, in a later lane only, +inf and -inf mixes,
    signed zeros and a row of all -inf."""
    base = np.array([0.5, -1.0, 2.0, 2.0, -3.0, 1.0, 0.25, 2.0, -0.5, 1.5, 2.0, 0.0])
    rows = [base.copy() for _ in range(12)]
    rows[0][9] = NAN                       # NaN in the last lane only
    rows[1][6] = NAN                       # NaN in the middle lane only
    rows[2][[6, 10]] = NAN                 # NaN in two later lanes: the first wins
    rows[3][[1, 7]] = NAN                  # NaN in the first and middle lanes
    rows[4][:] = NAN                       # all NaN: index 0
    rows[5][[4, 11]] = INF                 # +inf in two lanes: the first wins
    rows[6][[3, 8]] = [INF, NAN]           # NaN above +inf
    rows[7][:] = -INF                      # all -inf: index 0
    rows[8][[2, 3, 7, 10]] = -INF          # the largest finite value is then 1.5
    rows[9][:] = -INF
    rows[9][11] = -0.0                     # one finite column
    rows[10][:] = 0.0
    rows[10][[0, 5]] = -0.0                # -0 equals +0: index 0
    rows[11][[0, 1, 2, 3, 4]] = -INF       # the first lane all -inf
    rows[11][9] = INF
    return np.array(rows)


OFF = [0, 5, 8, 12]


def test_ids_follow_the_definition_and_numpy():
    z = rows_with_non_finite()
    r = oracle.project(z, OFF)
    for b, row in enumerate(z):
        assert r["ids"][b] == brute_argmax(list(row)), b
    assert np.array_equal(r["ids"], np.argmax(z, axis=1))
    # the rows written above, by hand
    assert list(r["ids"]) == [9, 6, 6, 1, 0, 4, 8, 0, 9, 11, 0, 9]


def test_ids_do_not_depend_on_the_lane_split():
    z = rows_with_non_finite()
    want = oracle.project(z, OFF)["ids"]
    for off in ([0, 12], [0, 1, 12], [0, 6, 7, 12], list(range(13))):
        assert np.array_equal(oracle.project(z, off)["ids"], want), off


def test_lane_results_follow_the_definition():
    z = rows_with_non_finite()
    r = oracle.project(z, OFF)
    for b, row in enumerate(z):
        for i in range(len(OFF) - 1):
            seg = list(row[OFF[i]:OFF[i + 1]])
            a = OFF[i] + brute_argmax(seg)
            assert r["lane_arg"][b, i] == a, (b, i)
            m = r["lane_max"][b, i]
            assert (math.isnan(m) and math.isnan(row[a])) or m == row[a], (b, i)


def test_log_probs_of_non_finite_rows():
    z = rows_with_non_finite()
    r = oracle.project(z, OFF)
    for b, row in enumerate(z):
        if np.isnan(row).any() or np.isposinf(row).any():
            # no value is defined there; the formulas give NaN
            assert math.isnan(r["lse"][b]), b
    # -inf columns drop out of the sum: row 8 and row 11 (no NaN, row 11's
    # +inf aside) have a finite lse over their finite columns
    row = z[8]
    fin = row[np.isfinite(row)]
    assert r["lse"][8] == pytest.approx(math.log(np.exp(fin).sum()), rel=1e-14)
    assert r["sel_lp"][8] == pytest.approx(1.5 - r["lse"][8], rel=1e-14)


def test_non_finite_rows_are_never_excused():
    # the near-tie flag excuses rows from the ID comparison; a row with a NaN
    # has a NaN gap and must stay compared
    z = rows_with_non_finite()
    r = oracle.project(z, OFF)
    for b in (0, 1, 2, 3, 4, 6):
        assert not r["near_tie"][b], b


def bf16(v):
    return np.array(v, dtype=np.float32).view(np.uint32) >> 16


def test_logits_propagate_nan_and_infinities():
    """IEEE products and sums in the fp64 logits: NaN in a hidden row makes
    its whole logit row NaN; +inf in a weight column gives +-inf by the sign
    of the hidden value, and NaN where that value is 0."""
    x = np.array([[1.0, 2.0, 0.5],
                  [1.0, NAN, 0.5],
                  [-1.0, 0.0, 0.5],
                  [0.0, 1.0, 2.0]], dtype=np.float32)
    w = np.array([[1.0, INF, 0.5, 1.0],
                  [0.5, 1.0, -1.0, 2.0],
                  [2.0, 1.0, 1.0, -INF]], dtype=np.float32)
    z = oracle.logits(bf16(x).astype(np.uint16), bf16(w).astype(np.uint16))
    assert np.isnan(z[1]).all()
    assert z[0, 1] == INF and z[2, 1] == -INF and np.isnan(z[3, 1])
    assert z[0, 3] == -INF and z[2, 3] == -INF and z[3, 3] == -INF
    assert z[0, 0] == 1.0 + 1.0 + 1.0 and z[2, 2] == -0.5 + 0.0 + 0.5
    ids = oracle.project(z, [0, 2, 4])["ids"]
    assert list(ids) == [1, 0, 0, 1]
