"""GPU test: token calls captured in a HIP graph and replayed.

Callers under graph capture are the reason for sb_project_tokens_static, and
a caller-provided workspace keeps sb_project_tokens allocation-free as well.
Every launch of these calls is a kernel (the slice counters are cleared by a
kernel, never by a memset node), so a captured call must give, on every
replay, the IDs that the same call gives eagerly on the inputs of that
moment.  Each head below is captured once; between replays the hidden rows
are overwritten in place with new values and the eager call runs on the same
inputs, with synchronizations in between.  Heads: one split into K slices
(clear, head and combine launches), one of 48 rows (hidden-row pack, head,
combine) and one of 200 rows (the large-batch kernel).
"""
import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from tests.gpu_common import upload

pytestmark = pytest.mark.gpu

HEADS = [
    # B, H, V, k
    (16, 2048, 4096, 2),
    (48, 1024, 30000, 3),
    (200, 256, 9000, 3),
]
REPLAYS = 5


def _capture(call):
    """Warm the call up on a side stream, then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("static", [True, False], ids=["static", "workspace"])
@pytest.mark.parametrize("B,H,V,k", HEADS)
def test_captured_token_call_replays(require_gpu, B, H, V, k, static):
    print(f"graph replay B={B} H={H} V={V} k={k} static={static}", flush=True)
    off = inputs.equal_lanes(V, k)
    d = inputs.make_random(B, H, V, off, seed=700 + B)
    head = upload(d, lanes_separate=True)
    ids = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    ws = None if static else sb.workspace(head, sb.SB_SURF_TOKENS)

    def call(stream):
        if static:
            sb.sb_project_tokens_static(head, ids, stream=stream)
        else:
            sb.sb_project_tokens(head, ids, ws=ws, stream=stream)

    g = _capture(call)
    eager_ids = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    for rep in range(REPLAYS):
        x_bits = inputs.draw_hidden(B, H, seed=800 + 10 * B + rep)
        head.x.copy_(sb.to_device_bf16(x_bits))
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = ids.cpu().numpy()
        sb.sb_project_tokens(head, eager_ids)
        torch.cuda.synchronize()
        assert np.array_equal(got, eager_ids.cpu().numpy()), f"replay {rep}"
        if rep in (0, REPLAYS - 1):
            r = oracle.project(oracle.logits(x_bits, d["w"]), off)
            ok = ~r["near_tie"]
            assert np.array_equal(got[ok], r["ids"][ok]), f"replay {rep} vs oracle"


@pytest.mark.parametrize("B,H,V,k", HEADS)
def test_captured_logprob_call_replays(require_gpu, B, H, V, k):
    """The log-prob call with complete log-probs (head, combine and normalize
    launches): every replay equals the eager call bit for bit."""
    print(f"graph replay (log-probs) B={B} H={H} V={V} k={k}", flush=True)
    off = inputs.equal_lanes(V, k)
    d = inputs.make_random(B, H, V, off, seed=900 + B)
    head = upload(d, lanes_separate=True)
    ldv = (V + 3) // 4 * 4
    out = [dict(ids=torch.full((B,), -1, dtype=torch.int32, device="cuda"),
                lse=torch.empty(B, dtype=torch.float32, device="cuda"),
                sel=torch.empty(B, dtype=torch.float32, device="cuda"),
                lp=torch.empty((B, ldv), dtype=torch.float32, device="cuda")[:, :V])
           for _ in range(2)]
    ws = sb.workspace(head, sb.SB_SURF_LOGPROBS_FULL)

    def call(o, stream=None):
        sb.sb_project_logprobs(head, o["ids"], o["lse"], o["sel"], o["lp"], ws=ws, stream=stream)

    g = _capture(lambda s: call(out[0], s))
    for rep in range(REPLAYS):
        head.x.copy_(sb.to_device_bf16(inputs.draw_hidden(B, H, seed=950 + 10 * B + rep)))
        for t in out[0].values():
            t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(out[1])
        torch.cuda.synchronize()
        for key in ("ids", "lse", "sel", "lp"):
            assert torch.equal(out[0][key], out[1][key]), (rep, key)
