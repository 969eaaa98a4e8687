"""GPU parity of the partial-completion call (sb_partial_complete) against the
oracle, through the C ABI.

Acceptance (per output row b, k lanes, rs_i(b) = max_n |P_i[b][n]| of the
oracle's partials):
  * sum, min, max: |g - o| <= PART_REL * k * max_i rs_i(b)
  * prod:          |g - o| <= PART_REL * k * prod_i rs_i(b)
Each GPU partial is an fp32 sum of exact bf16 x bf16 products over at most a
few thousand terms: its error is of order sqrt(K) * 2^-24 of the sum of
magnitudes, about 1e-5 of rs; PART_REL = 1e-3 leaves a wide margin and still
catches a dropped chunk, lane or operator.  Min and max select one partial,
so their error is at most one partial's; a product's error is bounded by the
sum over lanes of one partial's error times the others' magnitudes.
"""
import numpy as np
import pytest
import torch

from logit_source_projection_amd import inputs, sb
from oracle import partial as opart

pytestmark = pytest.mark.gpu

PART_REL = 1e-3


def upload(xs, ws, pad_x=0, pad_w=0, pad_bits=0x7FC0, device="cuda"):
    """Lane tensors with one common row stride each (padded with NaN bits
    that must never be read)."""
    B = xs[0].shape[0]
    N = ws[0].shape[1]
    ldx = ((max(x.shape[1] for x in xs) + 7) // 8) * 8 + pad_x
    ldw = ((N + 7) // 8) * 8 + pad_w
    xt, wt = [], []
    for x, w in zip(xs, ws):
        K = x.shape[1]
        xp = np.full((B, ldx), pad_bits, dtype=np.uint16)
        xp[:, :K] = x
        wp = np.full((K, ldw), pad_bits, dtype=np.uint16)
        wp[:, :N] = w
        xt.append(sb.to_device_bf16(xp, device)[:, :K])
        wt.append(sb.to_device_bf16(wp, device)[:, :N])
    return sb.Partial(xt, wt)


def run(part, op):
    B, N = part.B, part.N
    ldo = (N + 3) // 4 * 4
    out = torch.full((B, ldo), float("nan"), dtype=torch.float32, device="cuda")[:, :N]
    sb.sb_partial_complete(part, op, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(g, P, op):
    o = opart.complete(P, op)
    k = P.shape[0]
    rs = np.abs(P).max(axis=2)  # [k, B]
    scale = rs.prod(axis=0) if op == "prod" else rs.max(axis=0)
    err = np.abs(g.astype(np.float64) - o).max(axis=1)
    bad = err > PART_REL * k * np.maximum(scale, 1e-30)
    assert not bad.any(), (op, np.nonzero(bad)[0][:5], err[bad][:5], scale[bad][:5])
    return err / np.maximum(scale, 1e-30)


CASES = [
    # B, K per lane, N
    (1, (100,), 130),
    (16, (600, 1000), 300),
    (17, (512, 513), 256),
    (33, (1024,), 100),
    (64, (777, 31, 1500), 520),
    (65, (512,), 64),
    (300, (700, 700), 200),
    (3, (1, 9), 1),       # one output column, a one-row shard
    (2, (31,), 8),
    (70000, (300, 200), 40),  # the lane reduction over two 65535-row launches
]


@pytest.mark.parametrize("B,Ks,N", CASES)
def test_partial_completion_small(require_gpu, B, Ks, N):
    print(f"partial B={B} Ks={Ks} N={N}", flush=True)
    xs, ws = inputs.draw_partial(B, N, Ks, seed=B + N, sigma_w=0.05)
    P = opart.partials(xs, ws)
    part = upload(xs, ws, pad_x=8, pad_w=16)
    for op in opart.OPS:
        check(run(part, op), P, op)


def test_single_lane_operators_agree_bitwise(require_gpu):
    # with one lane every operator returns the lane's partial itself
    xs, ws = inputs.draw_partial(20, 264, (900,), seed=5)
    part = upload(xs, ws)
    outs = [run(part, op) for op in opart.OPS]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    check(outs[0], opart.partials(xs, ws), "sum")


def test_identical_lanes(require_gpu):
    # the same shard and weight in two lanes: max == min == the partial,
    # sum == 2 * partial exactly (doubling is exact in fp32)
    xs, ws = inputs.draw_partial(8, 136, (700,), seed=6)
    part1 = upload(xs, ws)
    part2 = upload(xs * 2, ws * 2)
    p = run(part1, "sum")
    assert np.array_equal(run(part2, "max"), p)
    assert np.array_equal(run(part2, "min"), p)
    assert np.array_equal(run(part2, "sum"), 2 * p)


def test_repeated_calls_are_bitwise_identical(require_gpu):
    xs, ws = inputs.draw_partial(24, 520, (1300, 900), seed=7)
    part = upload(xs, ws)
    for op in opart.OPS:
        a = run(part, op)
        assert np.array_equal(a, run(part, op)), op


@pytest.mark.parametrize("B", [3, 40, 100])
def test_nan_partial_propagates(require_gpu, B):
    """A NaN hidden value in one lane's shard makes that lane's partial NaN
    across its row; every operator, minimum and maximum included, then gives
    NaN across that row (as the oracle's np.minimum / np.maximum do), and
    the other rows match the oracle as usual."""
    xs, ws = inputs.draw_partial(B, 300, (700, 500, 90), seed=900 + B, sigma_w=0.05)
    xs[1][B // 2, 17] = 0x7FC0
    P = opart.partials(xs, ws)
    part = upload(xs, ws)
    others = np.array([b for b in range(B) if b != B // 2])
    for op in opart.OPS:
        g = run(part, op)
        assert np.isnan(g[B // 2]).all(), op
        assert not np.isnan(g[others]).any(), op
        check(g[others], P[:, others], op)


def test_empty_batch(require_gpu):
    xs, ws = inputs.draw_partial(1, 64, (64,), seed=8)
    part = upload(xs, ws)
    part.desc.B = 0
    out = torch.empty(0, 64, dtype=torch.float32, device="cuda")
    sb.sb_partial_complete(part, "sum", out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("B", [16, 64])
def test_mlp_down_workload(require_gpu, B):
    """The full Qwen3-14B-shaped down projection: N = 5120, two lanes of 8704."""
    d = inputs.make_partial("mlp_down", B=B)
    print(f"mlp_down B={B}", flush=True)
    P = opart.partials(d["xs"], d["ws"])
    part = upload(d["xs"], d["ws"])
    worst = {}
    for op in opart.OPS:
        worst[op] = float(check(run(part, op), P, op).max())
    print("worst relative error per operator:", worst, flush=True)


def draw_partial_case(i):
    """Sweep case i: rows weighted to the dispatch boundaries, 1-6 lanes of
    ragged K (down to one row), ragged N, weight scale and row padding."""
    rng = np.random.default_rng([2025, i])
    B = int(rng.choice([1, 2, 15, 16, 17, 31, 32, 33, 64, 65, 128, 129, 300]))
    k = int(rng.integers(1, 7))
    Ks = tuple(int(rng.integers(1, 2500)) if rng.random() < 0.9 else int(rng.integers(1, 9))
               for _ in range(k))
    nmax = max(1, min(1500, int(1e8 // (B * sum(Ks)))))
    N = int(rng.integers(1, nmax + 1))
    sigma_w = float(rng.choice([0.005, 0.05, 0.5]))
    pad_x, pad_w = 8 * int(rng.integers(0, 3)), 8 * int(rng.integers(0, 3))
    return B, Ks, N, sigma_w, pad_x, pad_w


@pytest.mark.parametrize("i", range(60))
def test_partial_completion_sweep(require_gpu, i):
    B, Ks, N, sigma_w, pad_x, pad_w = draw_partial_case(i)
    print(f"partial sweep case {i}: B={B} Ks={Ks} N={N} sigma_w={sigma_w} "
          f"pad=({pad_x}, {pad_w})", flush=True)
    xs, ws = inputs.draw_partial(B, N, Ks, seed=4000 + i, sigma_w=sigma_w)
    P = opart.partials(xs, ws)
    part = upload(xs, ws, pad_x=pad_x, pad_w=pad_w)
    for op in opart.OPS:
        check(run(part, op), P, op)
