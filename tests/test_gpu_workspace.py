"""GPU tests of the workspace contract: its contents on entry do not matter.

The head kernels write every per-(row, tile) pair and every partial tile
before the combine and fold steps read them, and the only state a call
carries between workgroups -- the K-slice counters -- is cleared by the
call itself before its head kernel runs.  So a workspace full of garbage
(a caller's mistake, memory reused from other work, or a call that failed
after part of its work was enqueued) must give the same results, bit for
bit, as a freshly allocated one.  No kernel waits on a counter, so garbage
cannot stall a launch; at worst a stale counter would misplace a fold,
which these tests would see as wrong or unwritten outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from tests.gpu_common import check_against_oracle, upload

pytestmark = pytest.mark.gpu

# One head per dispatch path: one, two and four 16-row blocks (the last with
# the packed hidden rows), split heads (8 and 2 K slices), and the
# large-batch kernel with 128-row (B = 100) and 256-row (B = 200) blocks.
HEADS = [
    # B, H, V, k
    (5, 512, 20000, 3),
    (24, 640, 9000, 2),
    (48, 1024, 30000, 4),
    (16, 2048, 4096, 2),      # 32 tiles: 8 slices
    (16, 4160, 37984, 1),     # 297 tiles, 130 steps: 2 slices
    (100, 512, 20000, 5),
    (200, 256, 9000, 3),
]


def _surfaces(head, B, V, ws, fill=0xFF):
    ids_t = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    ids_l = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    ids_f = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lane_ids = torch.full((B, head.desc.k), -1, dtype=torch.int32, device="cuda")
    lse = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    ldv = (V + 3) // 4 * 4
    lp = torch.full((B, ldv), float("nan"), dtype=torch.float32, device="cuda")[:, :V]
    lg = torch.full((B, ldv), float("nan"), dtype=torch.float32, device="cuda")[:, :V]
    for call in (
            lambda: sb.sb_project_tokens(head, ids_t, ws=ws),
            lambda: sb.sb_project_lane_results(head, ids_t, lane_ids, ws=ws),
            lambda: sb.sb_project_logprobs(head, ids_l, lse, sel, lp, ws=ws),
            lambda: sb.sb_full_logits(head, lg, ids_f, ws=ws)):
        if ws is not None:
            ws.fill_(fill)  # garbage before every call
        call()
        torch.cuda.synchronize()
    return dict(ids_t=ids_t.cpu().numpy(), ids_l=ids_l.cpu().numpy(),
                ids_f=ids_f.cpu().numpy(), lane_ids=lane_ids.cpu().numpy(),
                lse=lse.cpu().numpy(), sel=sel.cpu().numpy(), lp=lp.cpu().numpy(),
                lg=lg.cpu().numpy())


@pytest.mark.parametrize("B,H,V,k", HEADS)
def test_garbage_workspace_gives_identical_results(require_gpu, B, H, V, k):
    print(f"garbage workspace B={B} H={H} V={V} k={k}", flush=True)
    d = inputs.make_random(B, H, V, inputs.equal_lanes(V, k), seed=B + H + k)
    head = upload(d, lanes_separate=True)
    clean = _surfaces(head, B, V, None)  # fresh temporary workspaces
    need = max(sb.sb_workspace_bytes(head, s) for s in
               (sb.SB_SURF_TOKENS, sb.SB_SURF_LOGPROBS_FULL, sb.SB_SURF_FULL_LOGITS))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for fill in (0xFF, 0x5A):
        dirty = _surfaces(head, B, V, ws, fill)
        for key in clean:
            assert np.array_equal(clean[key], dirty[key], equal_nan=True), (fill, key)
    assert np.all(clean["ids_t"] >= 0)
    z = oracle.logits(d["x"], d["w"])
    g = dict(ids_tok=clean["ids_t"], ids_lp=clean["ids_l"], ids_r0=clean["ids_f"],
             lse=clean["lse"], sel_lp=clean["sel"], logits=clean["lg"], logprobs=clean["lp"])
    check_against_oracle(g, z, d["lane_off"])


def test_random_garbage_between_calls_of_one_workspace(require_gpu):
    """Random bytes written over the whole workspace before each of a run
    of calls of different shapes."""
    rng = np.random.default_rng(5)
    heads = []
    need = 0
    for i, (B, H, V, k) in enumerate(HEADS):
        d = inputs.make_random(B, H, V, inputs.equal_lanes(V, k), seed=50 + i)
        h = upload(d, lanes_separate=True)
        heads.append((d, h))
        need = max(need, sb.sb_workspace_bytes(h, sb.SB_SURF_LOGPROBS))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for d, h in heads + heads[::-1]:
        junk = torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)).to("cuda")
        ws.copy_(junk)
        ids = torch.full((d["B"],), -1, dtype=torch.int32, device="cuda")
        lse = torch.empty(d["B"], dtype=torch.float32, device="cuda")
        sb.sb_project_logprobs(h, ids, lse, ws=ws)
        torch.cuda.synchronize()
        r = oracle.project(oracle.logits(d["x"], d["w"]), d["lane_off"])
        ok = ~r["near_tie"]
        assert np.array_equal(ids.cpu().numpy()[ok], r["ids"][ok]), (d["B"], d["V"])
        assert np.allclose(lse.cpu().numpy(), r["lse"], rtol=1e-4, atol=0)


def test_side_stream_without_a_workspace(require_gpu):
    """A call on a non-current stream with no workspace: the binding
    allocates the temporary on that stream and records it there, so the
    caching allocator cannot reuse it while the kernels run."""
    d = inputs.make_random(48, 1024, 30000, inputs.equal_lanes(30000, 3), seed=61)
    head = upload(d)
    r = oracle.project(oracle.logits(d["x"], d["w"]), d["lane_off"])
    ok = ~r["near_tie"]
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        ids = torch.full((48,), -1, dtype=torch.int32, device="cuda")
        lse = torch.empty(48, dtype=torch.float32, device="cuda")
        side.wait_stream(torch.cuda.current_stream())
        sb.sb_project_logprobs(head, ids, lse, stream=side)
        sb.sb_project_tokens(head, ids, stream=side)
        # the current stream allocates and scribbles meanwhile
        scratch = torch.full((1 << 20,), 0x7F, dtype=torch.uint8, device="cuda")
        del scratch
        side.synchronize()
        assert np.array_equal(ids.cpu().numpy()[ok], r["ids"][ok])
        assert np.allclose(lse.cpu().numpy(), r["lse"], rtol=1e-4, atol=0)
