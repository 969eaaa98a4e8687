"""GPU test of sb_project_tokens_static, the token call that allocates
nothing (its workspace is the library's static device array): through the C
ABI, its IDs must equal sb_project_tokens' bit for bit, on two calls in a
row (the second on a smaller head, which finds the first call's leftovers in
the array), and a call that needs more than the array is refused before
anything is launched."""
import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from tests.gpu_common import upload

pytestmark = pytest.mark.gpu


def _both(d):
    head = upload(d, lanes_separate=True)
    B = d["B"]
    ref = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    got = torch.full((B,), -2, dtype=torch.int32, device="cuda")
    sb.sb_project_tokens(head, ref)
    sb.sb_project_tokens_static(head, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # (B, H, V, k): a larger call, then a smaller one on the same array
    ((64, 4096, 50000, 4), (5, 512, 9000, 2)),       # packed rows, then one row block
    ((16, 4160, 37984, 1), (3, 256, 1000, 3)),       # two K slices, then a small head
    ((300, 512, 20000, 3), (100, 256, 8000, 2)),     # 256-row, then 128-row blocks
])
def test_static_scratch_matches_the_workspace_call(require_gpu, first, second):
    for i, (B, H, V, k) in enumerate((first, second)):
        print(f"static scratch call {i}: B={B} H={H} V={V} k={k}", flush=True)
        d = inputs.make_random(B, H, V, inputs.equal_lanes(V, k), seed=90 + B + i)
        ref, got = _both(d)
        assert np.array_equal(ref, got), (B, H, V, k)
        r = oracle.project(oracle.logits(d["x"], d["w"]), d["lane_off"])
        ok = ~r["near_tie"]
        assert np.array_equal(got[ok], r["ids"][ok])


def test_static_scratch_rejects_calls_that_do_not_fit(require_gpu):
    # 4096 rows of a 151936-column head need about 39 MB of (row, tile) pairs
    x = torch.zeros((4096, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 151936), dtype=torch.bfloat16, device="cuda")
    head = sb.Head(x, w, inputs.equal_lanes(151936, 4))
    assert sb.sb_workspace_bytes(head, sb.SB_SURF_TOKENS) > sb.SB_STATIC_SCRATCH_BYTES
    ids = torch.full((4096,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(sb.SbError) as e:
        sb.sb_project_tokens_static(head, ids)
    assert e.value.status == sb.SB_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((ids == -7).all())  # nothing was enqueued
