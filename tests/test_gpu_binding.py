"""GPU test of the Python binding's argument checks with device tensors:
wrong dtypes, short outputs and strided layouts are refused with a clear
error before anything is enqueued, and the outputs stay untouched."""
import pytest
import torch

from logit_source_projection_amd import inputs, sb
from tests.gpu_common import upload

pytestmark = pytest.mark.gpu


def test_binding_checks_device_arguments(require_gpu):
    d = inputs.make_random(8, 256, 3000, [0, 1000, 3000], seed=77)
    head = upload(d, lanes_separate=True)
    B, V = 8, 3000
    dev = "cuda"
    ids = torch.full((B,), -1, dtype=torch.int32, device=dev)
    with pytest.raises(TypeError, match="ids must be torch.int32"):
        sb.sb_project_tokens(head, torch.zeros(B, dtype=torch.int64, device=dev))
    with pytest.raises(ValueError, match="ids must be contiguous with at least 8"):
        sb.sb_project_tokens(head, torch.zeros(B - 1, dtype=torch.int32, device=dev))
    with pytest.raises(ValueError, match="ids must be contiguous"):
        sb.sb_project_tokens(head, torch.zeros(2 * B, dtype=torch.int32, device=dev)[::2])
    with pytest.raises(TypeError, match="ws must be torch.uint8"):
        sb.sb_project_tokens(head, ids, ws=torch.zeros(1 << 20, dtype=torch.int32, device=dev))
    with pytest.raises(TypeError, match="lane_max must be torch.float32"):
        sb.sb_project_lane_results(head, ids, None,
                                   torch.zeros(B, 2, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError, match="lane_ids must be contiguous with at least 16"):
        sb.sb_project_lane_results(head, ids, torch.zeros(B, dtype=torch.int32, device=dev))
    lse = torch.zeros(B, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="logprobs must be a"):
        sb.sb_project_logprobs(head, ids, lse, None,
                               torch.zeros(B, 2 * V, device=dev)[:, ::2])
    with pytest.raises(ValueError, match="logits must be a"):
        sb.sb_full_logits(head, torch.zeros(B, V - 1, device=dev))
    torch.cuda.synchronize()
    assert bool((ids == -1).all())  # nothing ran
    # and the same call with valid arguments runs
    sb.sb_project_tokens(head, ids)
    torch.cuda.synchronize()
    assert bool((ids >= 0).all())
