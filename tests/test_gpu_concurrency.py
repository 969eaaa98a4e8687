"""GPU test of the library's thread safety: several host threads call it at
once, each on its own stream with its own workspace and outputs, on heads of
different dispatch paths.  The library keeps no state between calls beyond a
per-device note of the kernels whose LDS limit it has raised, so every result
must equal the same call made alone, bit for bit."""
import threading

import numpy as np
import pytest
import torch

from logit_source_projection_amd import inputs, sb
from tests.gpu_common import upload

pytestmark = pytest.mark.gpu

HEADS = [
    # B, H, V, k
    (16, 1024, 30000, 4),
    (48, 1024, 20000, 2),
    (16, 2048, 4096, 2),     # K slices
    (200, 256, 9000, 3),     # large-batch kernel (LDS limit raised on first use)
]
CALLS = 25


def _run(head, B, ws, stream):
    ids = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lse = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    tok = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    sb.sb_project_logprobs(head, ids, lse, ws=ws, stream=stream)
    sb.sb_project_tokens(head, tok, ws=ws, stream=stream)
    stream.synchronize()
    return ids.cpu().numpy(), lse.cpu().numpy(), tok.cpu().numpy()


def test_threads_on_their_own_streams(require_gpu):
    heads = []
    for i, (B, H, V, k) in enumerate(HEADS):
        d = inputs.make_random(B, H, V, inputs.equal_lanes(V, k), seed=60 + i)
        heads.append((B, upload(d, lanes_separate=True)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in heads]
    spaces = [sb.workspace(h, sb.SB_SURF_LOGPROBS) for _, h in heads]
    ref = [_run(h, B, ws, s) for (B, h), ws, s in zip(heads, spaces, streams)]
    errors = []

    def worker(i):
        B, h = heads[i]
        try:
            for _ in range(CALLS):
                got = _run(h, B, spaces[i], streams[i])
                for a, b in zip(got, ref[i]):
                    if not np.array_equal(a, b):
                        errors.append((i, a, b))
                        return
        except Exception as e:  # reported below, in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(heads))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors[:2]
