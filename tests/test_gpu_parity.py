"""GPU parity: libsb's HIP path against the CPU oracle, through the C ABI.

Small cases run the oracle on every output; they span several 128-column
tiles, ragged lane widths, ragged hidden sizes and more than one 64-row
group.  Edge cases: empty hidden size, zero rows, one-hot rows, exact ties,
power-of-two scaling, non-finite padding that must never be read, lane-count
invariance, run-to-run determinism.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from tests.gpu_common import check_against_oracle, check_internal, run_surfaces, upload

pytestmark = pytest.mark.gpu


def _case(d, full_logprobs=True, **up):
    print(f"case {d['name']} B={d['B']} H={d['H']} V={d['V']} k={d['k']} {up}", flush=True)
    head = upload(d, **up)
    g = run_surfaces(head, full_logprobs=full_logprobs)
    check_internal(g)
    z = oracle.logits(d["x"], d["w"])
    r = check_against_oracle(g, z, d["lane_off"])
    return g, z, r


def test_tiny_workload_with_forced_tie(require_gpu):
    d = inputs.make_workload("tiny")
    g, z, r = _case(d)
    row, a, b = d["planted"][0]
    # identical columns give bit-identical fp32 logits: a true tie on the GPU
    assert g["logits"][row, a] == g["logits"][row, b]
    assert g["ids_tok"][row] == a == 1000
    assert np.array_equal(g["ids_tok"], r["ids"])


SMALL = [
    # B, H, V, lane offsets, separate lane allocations
    (16, 512, 3000, [0, 1000, 1001, 2999, 3000], True),
    (1, 256, 4096, [0, 4096], False),
    (7, 200, 1288, [0, 640, 1288], False),
    (17, 96, 2056, [0, 1024, 2056], False),
    (33, 1000, 777, [0, 300, 777], True),
    (64, 4096, 2048, [0, 1024, 2048], False),
    (65, 128, 1000, [0, 13, 500, 1000], True),
    (48, 136, 2000, [0, 1000, 2000], False),
    (100, 40, 1000, [0, 504, 1000], True),
    (130, 72, 1536, [0, 512, 1024, 1536], False),
    (5, 8, 100, [0, 50, 100], True),
    (3, 40, 129, [0, 129], True),
    # large-batch kernel (256-row x 256-column blocks)
    (256, 96, 1536, [0, 512, 1024, 1536], False),
    (300, 200, 3000, [0, 1000, 1001, 2999, 3000], True),
    (513, 72, 777, [0, 300, 777], True),
    (1000, 40, 1400, [0, 704, 1400], False),   # four m-blocks: super-tiles of 4 x 8
    (2100, 40, 520, [0, 256, 520], False),
]


@pytest.mark.parametrize("B,H,V,off,sep", SMALL)
def test_small_heads(require_gpu, B, H, V, off, sep):
    d = inputs.make_random(B, H, V, off, seed=B * 7 + H)
    _case(d, lanes_separate=sep)


@pytest.mark.parametrize("B", [9, 100, 260])
def test_non_finite_padding_is_never_read(require_gpu, B):
    H, V = 100, 700
    off = [0, 200, 433, 700]
    d = inputs.make_random(B, H, V, off, seed=5)
    g, _, _ = _case(d, lanes_separate=True, pad_w=24, pad_x=28)
    g2 = run_surfaces(upload(d, lanes_separate=True, pad_w=24, pad_x=28, pad_bits=0))
    assert np.array_equal(g["logits"], g2["logits"])


@pytest.mark.parametrize("B", [16, 40, 100, 300])
def test_lane_base_alignment(require_gpu, B):
    """Shards that start at 16-byte positions inside a 128-byte cache line
    (each lane's tile grid then starts up to 56 columns before its first
    column; a lane of 8 or 100 columns gains a tile): IDs and logits
    bit-identical to line-aligned shards (each logit's sum order depends on H
    only), lse within a few ulp (its per-tile partial sums group the columns
    differently), and everything equal to the oracle."""
    H, V = 136, 3000
    off = [0, 712, 720, 820, 3000]
    d = inputs.make_random(B, H, V, off, seed=11 + B)
    ref = run_surfaces(upload(d, lanes_separate=True, lane_base_bytes=[0, 0, 0, 0]))
    for bases in ([16, 48, 64, 112], [96, 112, 112, 0], [112, 16, 80, 48]):
        g, _, _ = _case(d, lanes_separate=True, lane_base_bytes=bases)
        for key in ("ids_tok", "ids_lp", "ids_r0", "logits"):
            assert np.array_equal(g[key], ref[key]), (bases, key)
        np.testing.assert_allclose(g["lse"], ref["lse"], rtol=4e-7, atol=0)


@pytest.mark.parametrize("B", [16, 17, 32, 33, 64, 65, 128, 129, 255, 256, 257])
def test_batch_boundaries(require_gpu, B):
    """Both sides of every switch on the batch size: one, two and four row
    blocks per workgroup, several row groups, the large-batch kernel."""
    d = inputs.make_random(B, 72, 1000, [0, 504, 1000], seed=1000 + B)
    _case(d, lanes_separate=(B % 2 == 1))


@pytest.mark.parametrize("B,sep", [(16, False), (40, True), (100, True), (300, False)])
def test_maximum_lane_count(require_gpu, B, sep):
    """k = 64 lanes (the ABI's maximum), widths from 8 to 1000 columns."""
    widths = [(8, 16, 136, 264, 1000, 24, 128, 504)[i % 8] for i in range(64)]
    off = [0]
    for wdt in widths:
        off.append(off[-1] + wdt)
    d = inputs.make_random(B, 64, off[-1], off, seed=2000 + B)
    _case(d, lanes_separate=sep)


@pytest.mark.parametrize("B,H,V,off", [
    (3, 64, 1, [0, 1]),              # a single vocabulary column
    (5, 32, 8, list(range(9))),      # eight lanes of one column each
    (40, 1, 300, [0, 100, 300]),     # H = 1: one product per logit
    (70, 1, 300, [0, 100, 300]),     # ... with 128-row large-batch blocks
    (200, 1, 300, [0, 100, 300]),    # ... with 256-row large-batch blocks
    (300, 64, 1, [0, 1]),            # one column, two 256-row blocks
    (100, 40, 9, [0, 1, 2, 9]),      # one-column lanes in 128-row blocks
])
def test_degenerate_heads(require_gpu, B, H, V, off):
    """Smallest vocabularies, one-column lanes and a one-element hidden size
    (the hidden rows padded to the 8-element stride with non-finite bits)."""
    d = inputs.make_random(B, H, V, off, seed=B + V)
    _case(d, lanes_separate=True, pad_x=(8 - H % 8) % 8)


@pytest.mark.parametrize("B", [65535, 70000])
def test_batches_up_to_and_past_one_launch_of_rows(require_gpu, B):
    """A launch has at most 65535 workgroups in y: the launches with one row
    per y index (normalize, reconstruct, the full-logit argmax) run over
    70000 rows as two slices (65535 rows, then 4465).  Every surface,
    complete log-probs included, against the oracle on every row; 256 and
    274 row blocks of the large-batch kernel."""
    d = inputs.make_random(B, 40, 520, [0, 256, 520], seed=3000 + B % 7)
    _case(d)


@pytest.mark.parametrize("B", [3, 40, 70])
def test_million_column_vocabulary(require_gpu, B):
    """V = 1,048,583 (2^20 + 7) in three ragged lanes: about 8200 tiles per
    row for the combine, the lse fold and the full-logit argmax (128 chunks),
    through the decode kernel (3 rows; 40 rows with packed hidden rows) and
    the large-batch kernel (70 rows, one 128-row block)."""
    V = (1 << 20) + 7
    off = [0, 300_001, 700_000, V]
    d = inputs.make_random(B, 24, V, off, seed=4100 + B)
    _case(d, lanes_separate=True)


def test_empty_hidden_size(require_gpu):
    B, V = 3, 1000
    x = torch.empty((B, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((0, V), dtype=torch.bfloat16, device="cuda")
    head = sb.Head(x, w, [0, 504, 1000], ldx=8, ldw=1000)
    g = run_surfaces(head)
    check_internal(g)
    assert np.all(g["logits"] == 0.0)
    assert np.all(g["ids_tok"] == 0)
    assert np.allclose(g["lse"], math.log(V), rtol=1e-6)


def test_empty_batch(require_gpu):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    head = sb.Head(x, w, [0, 256])
    ids = torch.empty((0,), dtype=torch.int32, device="cuda")
    sb.sb_project_tokens(head, ids)
    torch.cuda.synchronize()


def test_zero_and_one_hot_rows(require_gpu):
    B, H, V = 6, 320, 5000
    off = [0, 2504, 5000]
    d = inputs.make_random(B, H, V, off, seed=9)
    x = d["x"]
    x[0, :] = 0
    one = np.uint16(inputs.f32_to_bf16_bits(np.float32(1.0)))
    for b, h in [(1, 0), (2, 177), (3, 319)]:
        x[b, :] = 0
        x[b, h] = one
    g, z, r = _case(d)
    assert np.all(g["logits"][0] == 0.0) and g["ids_tok"][0] == 0
    assert abs(float(g["lse"][0]) - math.log(V)) <= 1e-5
    for b, h in [(1, 0), (2, 177), (3, 319)]:
        wrow = inputs.bf16_bits_to_f32(d["w"][h])
        assert np.array_equal(g["logits"][b], wrow), (b, h)


def test_power_of_two_scaling(require_gpu):
    B, H, V = 8, 512, 3072
    off = [0, 1024, 3072]
    d = inputs.make_random(B, H, V, off, seed=10)
    g1 = run_surfaces(upload(d))
    x2 = d["x"].copy()
    nz = (x2 & 0x7FFF) != 0
    x2[nz] += np.uint16(1 << 7)
    d2 = dict(d, x=x2)
    g2 = run_surfaces(upload(d2))
    assert np.array_equal(g2["logits"], 2.0 * g1["logits"])
    assert np.array_equal(g2["ids_tok"], g1["ids_tok"])


def test_exact_ties_across_and_within_lanes(require_gpu):
    B, H, V = 4, 256, 4096
    off = [0, 1024, 2048, 3072, 4096]
    d = inputs.make_random(B, H, V, off, seed=11)
    inputs.plant_equal_columns(d["x"], d["w"], 0, (3500, 2500, 700), 9.0)
    inputs.plant_equal_columns(d["x"], d["w"], 2, (1500, 1030), 9.0)
    inputs.plant_equal_columns(d["x"], d["w"], 3, (1023, 1024), 9.0)  # lane boundary
    g, z, r = _case(d)
    assert list(g["ids_tok"][[0, 2, 3]]) == [700, 1030, 1023]


@pytest.mark.parametrize("B", [16, 300])
def test_lane_count_invariance(require_gpu, B):
    H, V = 1024, 8192
    d = inputs.make_random(B, H, V, [0, V], seed=12)
    outs = []
    for k in (1, 2, 4, 8):
        d["lane_off"] = inputs.equal_lanes(V, k)
        outs.append(run_surfaces(upload(d)))
    for o in outs[1:]:
        assert np.array_equal(o["logits"], outs[0]["logits"])
        assert np.array_equal(o["ids_tok"], outs[0]["ids_tok"])


def test_repeated_calls_are_bitwise_identical(require_gpu):
    d = inputs.make_random(24, 640, 6000, [0, 3000, 6000], seed=13)
    head = upload(d)
    first = run_surfaces(head)
    for _ in range(3):
        again = run_surfaces(head)
        for key in ("ids_tok", "ids_lp", "ids_r0", "lse", "sel_lp", "logits", "logprobs"):
            assert np.array_equal(first[key], again[key]), key


def test_workspace_reuse_across_shapes(require_gpu):
    # one workspace, a large call then a small one on the same stream
    big = inputs.make_random(40, 256, 9008, [0, 4504, 9008], seed=14)
    small = inputs.make_random(3, 256, 1000, [0, 1000], seed=15)
    hb, hs = upload(big), upload(small)
    n = sb.sb_workspace_bytes(hb, sb.SB_SURF_LOGPROBS)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for d, h in ((big, hb), (small, hs)):
        ids = torch.empty(d["B"], dtype=torch.int32, device="cuda")
        lse = torch.empty(d["B"], dtype=torch.float32, device="cuda")
        sb.sb_project_logprobs(h, ids, lse, ws=ws)
        torch.cuda.synchronize()
        z = oracle.logits(d["x"], d["w"])
        r = oracle.project(z, d["lane_off"])
        ok = ~r["near_tie"]
        assert np.array_equal(ids.cpu().numpy()[ok], r["ids"][ok])
        assert np.allclose(lse.cpu().numpy(), r["lse"], rtol=1e-4)


@pytest.mark.parametrize("B,H,V,k", [
    (1, 32768, 4096, 2),     # one row, 8 K slices of 128 steps
    (4, 20000, 1500, 2),     # ragged K tail, 8 slices
    (64, 16384, 3000, 2),    # packed hidden rows (2 MB) and K slices
    (200, 12288, 600, 3),    # large-batch kernel, 192 K stages
])
def test_long_hidden_sums(require_gpu, B, H, V, k):
    """Hidden sizes of 12k-32k: every slice, stage and fold of a long sum,
    against the oracle within the row-max-relative logit tolerance."""
    d = inputs.make_random(B, H, V, inputs.equal_lanes(V, k), seed=H + B, sigma_w=0.01)
    _case(d, lanes_separate=True)
