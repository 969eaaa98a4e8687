"""Pins of the partial-completion oracle (SemBridge paper, section 3.6 and
section 6.4): exact-rational brute force for every registered operator,
closed forms, invariants, and planted mistakes that must fail a pin."""
from fractions import Fraction

import numpy as np
import pytest

from logit_source_projection_amd import inputs
from oracle import partial
from tests.exact import bf16_to_fraction, exact_logits


def tiny_lanes(B, Ks, N, seed, sigma_x=1.0, sigma_w=0.5):
    xs = [inputs.draw_hidden(B, K, seed * 16 + i, sigma=sigma_x) for i, K in enumerate(Ks)]
    ws = [inputs.draw_weight(K, N, sigma_w, seed * 16 + i) for i, K in enumerate(Ks)]
    return xs, ws


def exact_complete(xs, ws, op):
    """The definition over exact rationals: partials, then the operator over
    the lanes (exact, so the order cannot matter)."""
    P = [exact_logits(x, w) for x, w in zip(xs, ws)]
    B, N = len(P[0]), len(P[0][0])
    out = []
    for b in range(B):
        row = []
        for n in range(N):
            vals = [p[b][n] for p in P]
            if op == "sum":
                v = sum(vals, Fraction(0))
            elif op == "prod":
                v = Fraction(1)
                for t in vals:
                    v *= t
            elif op == "min":
                v = min(vals)
            else:
                v = max(vals)
            row.append(v)
        out.append(row)
    return out, P


def pin_exact(complete_fn, xs, ws, op):
    got = complete_fn(xs, ws, op)
    ref, P = exact_complete(xs, ws, op)
    for b in range(len(ref)):
        for n in range(len(ref[0])):
            # each partial is an fp64 sum of exact products: relative error
            # below K * 2^-52 of the sum of magnitudes; the operator adds one
            # rounding per lane
            mags = []
            for x, w in zip(xs, ws):
                K = x.shape[1]
                mags.append(sum(abs(bf16_to_fraction(x[b, h]) * bf16_to_fraction(w[h, n]))
                                for h in range(K)) * K * Fraction(2) ** -52)
            if op == "prod":
                bound = Fraction(0)
                for i in range(len(P)):
                    term = mags[i]
                    for j in range(len(P)):
                        if j != i:
                            term *= abs(P[j][b][n]) + mags[j]
                    bound += term
                bound += abs(ref[b][n]) * len(P) * Fraction(2) ** -52
            else:
                bound = sum(mags, Fraction(0)) + abs(ref[b][n]) * len(P) * Fraction(2) ** -52
            assert abs(Fraction(got[b, n]) - ref[b][n]) <= bound, (op, b, n)


CASES = [
    # B, K per lane, N, seed
    (2, (7,), 5, 1),
    (3, (4, 9), 6, 2),
    (2, (5, 3, 8), 4, 3),
]


@pytest.mark.parametrize("op", partial.OPS)
@pytest.mark.parametrize("B,Ks,N,seed", CASES)
def test_every_operator_matches_exact_rationals(op, B, Ks, N, seed):
    xs, ws = tiny_lanes(B, Ks, N, seed)
    pin_exact(partial.partial_complete, xs, ws, op)


def test_single_lane_is_its_partial_for_every_operator():
    xs, ws = tiny_lanes(3, (12,), 7, 4)
    P = partial.partials(xs, ws)
    for op in partial.OPS:
        assert np.array_equal(partial.complete(P, op), P[0])


def test_identical_lanes_closed_forms():
    xs, ws = tiny_lanes(2, (10,), 6, 5)
    xs3, ws3 = xs * 3, ws * 3
    P = partial.partials(xs, ws)[0]
    assert np.array_equal(partial.partial_complete(xs3, ws3, "max"), P)
    assert np.array_equal(partial.partial_complete(xs3, ws3, "min"), P)
    # 3P and P^3 are exact in fp64 up to one rounding each step
    assert np.allclose(partial.partial_complete(xs3, ws3, "sum"), 3 * P, rtol=1e-15, atol=0)
    assert np.allclose(partial.partial_complete(xs3, ws3, "prod"), P ** 3, rtol=1e-15, atol=0)


def test_zero_lane_absorbs_product_and_leaves_sum():
    xs, ws = tiny_lanes(2, (6, 6), 5, 6)
    xz = [xs[0], np.zeros_like(xs[1])]      # bf16 bits 0 -> +0.0
    P0 = partial.partials([xs[0]], [ws[0]])[0]
    assert np.array_equal(partial.partial_complete(xz, ws, "sum"), P0)
    assert not np.any(partial.partial_complete(xz, ws, "prod"))
    assert np.array_equal(partial.partial_complete(xz, ws, "max"), np.maximum(P0, 0))
    assert np.array_equal(partial.partial_complete(xz, ws, "min"), np.minimum(P0, 0))


def test_lane_order_does_not_change_min_max_and_moves_sum_only_in_last_bits():
    xs, ws = tiny_lanes(3, (9, 5, 7), 8, 7)
    a = {op: partial.partial_complete(xs, ws, op) for op in partial.OPS}
    b = {op: partial.partial_complete(xs[::-1], ws[::-1], op) for op in partial.OPS}
    assert np.array_equal(a["min"], b["min"]) and np.array_equal(a["max"], b["max"])
    assert np.allclose(a["sum"], b["sum"], rtol=1e-14, atol=1e-14)
    assert np.allclose(a["prod"], b["prod"], rtol=1e-14, atol=0)


def test_nan_partial_propagates_through_every_operator():
    """A NaN hidden value in lane 1's shard at row 2 makes that lane's
    partial NaN across row 2 (IEEE: NaN times anything is NaN).  Sum and
    product then give NaN there by IEEE arithmetic; minimum and maximum
    by the reading taken for them (numpy's np.minimum / np.maximum, not
    np.fmin / np.fmax, which would drop the NaN).  Every other row is
    independent of row 2 and equals the completion without the NaN."""
    xs, ws = tiny_lanes(4, (6, 7, 5), 9, 11)
    xn = [x.copy() for x in xs]
    xn[1][2, 3] = 0x7FC0                    # bf16 quiet NaN
    rows = [0, 1, 3]
    for op in partial.OPS:
        clean = partial.partial_complete(xs, ws, op)
        got = partial.partial_complete(xn, ws, op)
        assert np.isnan(got[2]).all(), op
        assert np.array_equal(got[rows], clean[rows]), op
        assert not np.isnan(got[rows]).any(), op


def test_rejects_bad_inputs():
    xs, ws = tiny_lanes(2, (4, 4), 3, 8)
    with pytest.raises(ValueError):
        partial.partial_complete(xs, ws, "mean")
    with pytest.raises(ValueError):
        partial.partials(xs, ws[:1])
    with pytest.raises(ValueError):
        partial.partials(xs, [ws[0], ws[1][:, :2]])


# planted mistakes: each broken oracle must fail the exact pin
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


MX, MW = tiny_lanes(2, (6, 5), 4, 9)


def test_mutation_dropped_lane_is_caught():
    def bad(xs, ws, op):
        return partial.complete(partial.partials(xs, ws)[:-1], op)
    for op in partial.OPS:
        assert _fails(lambda: pin_exact(bad, MX, MW, op)), op


def test_mutation_swapped_operator_is_caught():
    swap = {"sum": "prod", "prod": "sum", "min": "max", "max": "min"}

    def bad(xs, ws, op):
        return partial.partial_complete(xs, ws, swap[op])
    for op in partial.OPS:
        assert _fails(lambda: pin_exact(bad, MX, MW, op)), op


def test_mutation_reduction_over_rows_instead_of_lanes_is_caught():
    def bad(xs, ws, op):
        P = partial.partials(xs, ws)
        return partial.complete(np.swapaxes(P, 0, 1), op)[: P.shape[1]]
    assert _fails(lambda: pin_exact(bad, MX, MW, "sum"))


def test_mutation_transposed_weight_is_caught():
    xs, ws = tiny_lanes(2, (5, 5), 5, 10)

    def bad(xs_, ws_, op):
        return partial.partial_complete(xs_, [np.ascontiguousarray(w.T) for w in ws_], op)
    assert _fails(lambda: pin_exact(bad, xs, ws, "sum"))
