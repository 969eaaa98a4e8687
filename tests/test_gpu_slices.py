"""GPU parity of heads whose tiles are split into K slices, and of one
workspace shared by calls of different shapes, surfaces and entry points.

A head with fewer 128-column tiles than the GPU holds head workgroups (for
instance one GPU's lane of a tensor-parallel head) splits every tile's hidden
steps into slices, one workgroup each; the workgroup that finishes a tile's
last slice adds the partial tiles in slice order.  The split depends on
(B, H, V) only, so the acceptance rules of the other parity tests apply
unchanged: every surface bit-identical, lane splits bit-identical, and all of
it equal to the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from oracle import partial as opart
from tests.gpu_common import check_against_oracle, check_internal, run_surfaces, upload
from tests.test_gpu_partial import upload as upload_partial

pytestmark = pytest.mark.gpu

# Workspace bytes every call reserves up front (the slice counters).
ZERO = 8192


def slices_of(head, B, H):
    """K slices of a head, read back from its token workspace size: past the
    counter region (and, for 33-64 rows, the hidden rows packed per 32-deep
    step, 4 KB per step), each slice holds one fp32 partial tile (rows per
    group x 128 columns) per tile of the tile capacity (lanes sized for the
    largest cache-line shift of 56 columns); last come the (row, tile) pairs
    of the combine launch."""
    rpg = 16 if B <= 16 else (32 if B <= 32 else 64)
    T = sum((head.lane_off[i + 1] - head.lane_off[i] + 56 + 127) // 128
            for i in range(len(head.lane_off) - 1))
    packed = (H + 31) // 32 * 4096 if 32 < B <= 64 else 0
    pairs = (B * T * 8 + 255) // 256 * 256
    extra = sb.sb_workspace_bytes(head, sb.SB_SURF_TOKENS) - ZERO - packed - pairs
    assert extra % (T * rpg * 128 * 4) == 0
    return max(1, extra // (T * rpg * 128 * 4))


SPLIT = [
    # B, H, V, lane offsets, separate lane allocations, K slices
    (16, 5120, 8192, [0, 8192], False, 4),            # 64 tiles: 4 slices of 40 steps
    (64, 5120, 16256, [0, 8000, 16256], False, 3),    # 127 tiles: slices of 56, 56, 48 steps
    (1, 2048, 1000, [0, 500, 1000], True, 4),
    (20, 1000, 3000, [0, 1500, 3000], True, 2),       # two row blocks; K tail in the last slice
    (40, 2056, 777, [0, 300, 777], True, 4),          # four row blocks; slices of 20, 20, 20, 5 steps
    (64, 4096, 2048, [0, 1024, 2048], False, 8),
    (7, 3000, 5000, [0, 2500, 5000], True, 5),        # 94 steps: 20, 20, 20, 20, 14
    (16, 2048, 8192, list(range(0, 8193, 128)), True, 4),  # 64 lanes of one or two tiles each
    (64, 8192, 2000, [0, 1000, 2000], True, 8),       # 256 steps: 8 slices of 32
    # just past one tile per CU at 16 rows: two slices
    (16, 5120, 37984, [0, 37984], False, 2),          # one GPU's lane of the dense head
    (9, 4100, 40000, [0, 20000, 40000], True, 2),     # 313 tiles; 129 steps: 68 + 61, K tail
    (16, 4096, 45056, [0, 45056], False, 2),          # 352 tiles
    (16, 4096, 45184, [0, 45184], False, 1),          # 353 tiles: not split
    (17, 5120, 37984, [0, 37984], False, 1),          # two row blocks: not split
]


@pytest.mark.parametrize("B,H,V,off,sep,S", SPLIT)
def test_split_heads(require_gpu, B, H, V, off, sep, S):
    print(f"split B={B} H={H} V={V} off={off} S={S}", flush=True)
    d = inputs.make_random(B, H, V, off, seed=B + H + V)
    head = upload(d, lanes_separate=sep, pad_x=(8 - H % 8) % 8 + 8)
    assert slices_of(head, B, H) == S
    g = run_surfaces(head)
    check_internal(g)
    check_against_oracle(g, oracle.logits(d["x"], d["w"]), d["lane_off"])


def test_split_head_lane_splits_are_bitwise_identical(require_gpu):
    """A split head (64 tiles, 4 slices) cut into 1 to 4 lanes (offsets on
    16-byte boundaries of the one weight allocation): the slices depend on
    (B, H, V) only, so every logit is summed in the same order."""
    B, H, V = 16, 5120, 8192
    d = inputs.make_random(B, H, V, [0, V], seed=21)
    outs = []
    for off in ([0, V], inputs.equal_lanes(V, 2), inputs.equal_lanes(V, 4), [0, 1000, V],
                [0, 800, 5000, V]):
        d["lane_off"] = list(off)
        outs.append(run_surfaces(upload(d)))
    for o in outs[1:]:
        for key in ("logits", "ids_tok", "ids_lp", "ids_r0"):
            assert np.array_equal(o[key], outs[0][key]), key
        # lse sums per-tile pairs, and lanes start their own tile grids
        np.testing.assert_allclose(o["lse"], outs[0]["lse"], rtol=4e-7, atol=0)


def test_split_head_repeated_calls_are_bitwise_identical(require_gpu):
    """The slice that folds a tile is whichever finishes last; the fold order
    is fixed, so repeated calls agree bit for bit."""
    d = inputs.make_random(40, 4096, 3000, [0, 1000, 3000], seed=22)
    head = upload(d)
    first = run_surfaces(head)
    for _ in range(4):
        again = run_surfaces(head)
        for key in ("ids_tok", "lse", "sel_lp", "logits", "logprobs"):
            assert np.array_equal(first[key], again[key]), key


def _ids_and_lse(d, head, surface, ws):
    B = d["B"]
    ids = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lse = None
    if surface == "tokens":
        sb.sb_project_tokens(head, ids, ws=ws)
    elif surface == "logprobs":
        lse = torch.empty(B, dtype=torch.float32, device="cuda")
        sb.sb_project_logprobs(head, ids, lse, ws=ws)
    else:
        ldv = (d["V"] + 3) // 4 * 4
        logits = torch.empty((B, ldv), dtype=torch.float32, device="cuda")[:, :d["V"]]
        sb.sb_full_logits(head, logits, ids, ws=ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), None if lse is None else lse.cpu().numpy()


def test_one_workspace_for_every_shape_surface_and_entry_point(require_gpu):
    """One workspace serves a sequence of calls whose
    regions grow and shrink: small and large batches, few and many lanes,
    split and unsplit heads, the full-logit plan (which fills most of the
    workspace with shards) and partial completion in between."""
    calls = [
        ("tokens", 3, 256, 1000, 1),
        ("full", 40, 512, 6000, 8),
        ("logprobs", 128, 512, 3000, 5),  # one 128-row large-batch block
        ("tokens", 64, 2048, 3000, 16),   # split, 16 lanes
        ("logprobs", 20, 640, 9000, 3),
        ("partial", 16, 0, 520, 2),
        ("tokens", 255, 136, 4000, 64),   # large-batch kernel, 64 lanes
        ("logprobs", 64, 4096, 2048, 2),  # split
        ("tokens", 1, 5120, 9000, 1),     # split
        ("full", 300, 72, 1000, 4),       # large-batch kernel
        ("tokens", 3, 256, 1000, 1),
    ]
    heads = []
    need = 0
    for i, (surf, B, H, V, k) in enumerate(calls):
        if surf == "partial":
            xs, wts = inputs.draw_partial(B, V, (700, 300), seed=30 + i)
            part = upload_partial(xs, wts)
            heads.append((xs, wts, part))
            need = max(need, sb.sb_partial_workspace_bytes(part))
            continue
        d = inputs.make_random(B, H, V, inputs.equal_lanes(V, k), seed=30 + i)
        head = upload(d, lanes_separate=True)
        heads.append((d, head))
        s = {"tokens": sb.SB_SURF_TOKENS, "logprobs": sb.SB_SURF_LOGPROBS,
             "full": sb.SB_SURF_FULL_LOGITS}[surf]
        need = max(need, sb.sb_workspace_bytes(head, s))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for (surf, B, H, V, k), h in zip(calls, heads):
        print(f"shared workspace: {surf} B={B} H={H} V={V} k={k}", flush=True)
        if surf == "partial":
            xs, wts, part = h
            out = torch.empty((B, V), dtype=torch.float32, device="cuda")
            sb.sb_partial_complete(part, "sum", out, ws=ws)
            torch.cuda.synchronize()
            o = opart.complete(opart.partials(xs, wts), "sum")
            scale = np.abs(opart.partials(xs, wts)).max(axis=(0, 2))
            assert np.all(np.abs(out.cpu().numpy() - o).max(axis=1) <= 2e-3 * scale)
            continue
        d, head = h
        ids, lse = _ids_and_lse(d, head, surf, ws)
        r = oracle.project(oracle.logits(d["x"], d["w"]), d["lane_off"])
        ok = ~r["near_tie"]
        assert np.array_equal(ids[ok], r["ids"][ok])
        if lse is not None:
            assert np.all(np.abs(lse - r["lse"]) <= 1e-4 * np.maximum(np.abs(r["lse"]), 1.0))
