"""GPU parity over a seeded random sweep of head shapes, through the C ABI.

Each case draws its own shape and layout from a generator seeded by the case
number, so that a failure names a reproducible case:
  * B from a list weighted towards the batch boundaries of the dispatch
    (16, 32, 64 and 128 rows, 129 and 256 for the large-batch kernel);
  * H from 1 to 2111 (ragged K tails; from 1024 up, heads of few tiles split
    every tile's hidden sum into K slices);
  * V, k (1 to 64 lanes) and ragged lane widths, one weight allocation (lane
    offsets on multiples of 8) or one allocation per lane, each shard
    starting at a random 16-byte offset inside its cache line;
  * row strides of x and W padded by 0 to 16 elements of NaN bits past the
    next multiple of 8;
  * the scale of x and W (largest logits from about 0.01 to about 100);
  * in half of the cases two identical weight columns, made the maximum of
    one row, so that every row holds an exact tie between them.
V is capped so that the oracle finishes each case in well under a second.

Every case runs the token, per-lane, log-prob (with complete log-probs) and
full-logit calls and checks:
  * the surfaces against each other, bit for bit (IDs, log-probs = logits -
    lse, sel_lp);
  * the oracle under the acceptance rules (logits, lse, IDs off the near-tie
    rows, sel_lp, complete log-probs);
  * each lane's (max, lowest index) against the GPU's own logits, bit for bit;
  * every row whose maximum is the planted tie (by a clear margin) reports
    the lower column.
"""
import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from tests.gpu_common import (LOGIT_REL, check_against_oracle, check_internal, run_surfaces,
                              upload)

pytestmark = pytest.mark.gpu

N_CASES = 160
B_CHOICES = [1, 2, 7, 15, 16, 17, 31, 32, 33, 40, 63, 64, 65, 100, 127, 128, 129, 200, 255,
             256, 257, 300]
ORACLE_BUDGET = 1.5e8  # B * H * V multiply-adds per case


def draw_case(i):
    """Shape, lanes, layout and scales of sweep case i."""
    rng = np.random.default_rng([2024, i])
    B = int(rng.choice(B_CHOICES))
    band = int(rng.integers(0, 3))
    H = int(rng.integers(*[(1, 96), (96, 700), (700, 2112)][band]))
    sep = bool(rng.integers(0, 2))
    k = int(rng.integers(1, 9)) if rng.random() < 0.85 else int(rng.integers(9, 65))
    vmin = k if sep else 8 * k
    vmax = max(vmin, min(6000, int(ORACLE_BUDGET // (B * H))))
    V = int(rng.integers(vmin, vmax + 1))
    if sep:
        cuts = rng.choice(np.arange(1, V), k - 1, replace=False) if k > 1 else []
    else:
        cuts = 8 * rng.choice(np.arange(1, (V - 1) // 8 + 1), k - 1, replace=False) if k > 1 else []
    off = [0] + sorted(int(c) for c in cuts) + [V]
    bases = None
    if sep and rng.random() < 0.5:
        bases = [16 * int(rng.integers(0, 8)) for _ in range(k)]
    sigma_x = float(rng.choice([0.1, 1.0, 4.0]))
    sigma_w = float(rng.choice([0.002, 0.02, 0.2]))
    tie = None
    if B >= 2 and V >= 2 and rng.random() < 0.5:
        a, b = sorted(int(c) for c in rng.choice(V, 2, replace=False))
        tie = (int(rng.integers(0, B)), a, b)
    pad = 8 * int(rng.integers(0, 3))
    return dict(B=B, H=H, V=V, off=off, sep=sep, bases=bases, sigma_x=sigma_x,
                sigma_w=sigma_w, tie=tie, pad=pad, seed=3000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_head(require_gpu, i):
    c = draw_case(i)
    print(f"sweep case {i}: B={c['B']} H={c['H']} V={c['V']} k={len(c['off']) - 1} "
          f"separate={c['sep']} bases={c['bases']} sigma=({c['sigma_x']}, {c['sigma_w']}) "
          f"tie={c['tie']} pad={c['pad']}", flush=True)
    d = inputs.make_random(c["B"], c["H"], c["V"], c["off"], seed=c["seed"],
                           sigma_x=c["sigma_x"], sigma_w=c["sigma_w"])
    if c["tie"]:
        row, a, b = c["tie"]
        # large enough to be the row's maximum at every scale drawn here
        inputs.plant_equal_columns(d["x"], d["w"], row, (a, b), 60.0)
    # row strides: multiples of 8 plus c["pad"] more, the padding NaN bits
    # that no kernel may read
    pad_x = (8 - c["H"] % 8) % 8 + c["pad"]
    head = upload(d, lanes_separate=c["sep"], lane_base_bytes=c["bases"], pad_x=pad_x,
                  pad_w=c["pad"])
    g = run_surfaces(head)
    check_internal(g)
    z = oracle.logits(d["x"], d["w"])
    check_against_oracle(g, z, d["lane_off"])

    B, k, off = c["B"], len(c["off"]) - 1, c["off"]
    ids = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lane_ids = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
    lane_max = torch.full((B, k), float("nan"), dtype=torch.float32, device="cuda")
    sb.sb_project_lane_results(head, ids, lane_ids, lane_max)
    torch.cuda.synchronize()
    li, lm = lane_ids.cpu().numpy(), lane_max.cpu().numpy()
    lg = g["logits"]
    assert np.array_equal(ids.cpu().numpy(), g["ids_tok"])
    for j in range(k):
        seg = lg[:, off[j]:off[j + 1]]
        assert np.array_equal(li[:, j], off[j] + np.argmax(seg, axis=1)), j
        assert np.array_equal(lm[:, j], seg.max(axis=1)), j

    if c["tie"]:
        # the two columns are identical, so every row holds an exact tie
        # between them; where it is the row's maximum by more than twice the
        # logit tolerance, the GPU's own maximum is that tie too, and the ID
        # must be the lower column
        row, a, b = c["tie"]
        assert np.array_equal(lg[:, a], lg[:, b]), "identical columns give identical logits"
        others = np.delete(z, [a, b], axis=1)
        top = others.max(axis=1) if others.shape[1] else np.full(B, -np.inf)
        clear = z[:, a] - top > 2 * LOGIT_REL * np.abs(z).max(axis=1)
        assert np.all(g["ids_tok"][clear] == a), "a tie at the row maximum goes to the lower column"
        print(f"  rows whose maximum is the planted tie: {int(clear.sum())} of {B}", flush=True)
