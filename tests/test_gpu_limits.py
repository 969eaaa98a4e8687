"""GPU parity at the largest strides validation accepts.

The kernels address a K step of a shard and a block of hidden rows with
32-bit byte offsets from the step's or block's base, and validation refuses
strides at which those offsets would reach 4 GiB (tests/test_abi_cpu.py
checks both sides of each limit).  Here every surface runs at the largest
accepted stride of each kind, with a full block of rows, so that the last
row of a block (or the last row of a step) sits just below 4 GiB from its
base:

  * decode kernel: 64 rows of x at ldx = 2^25 - 8 (63 * ldx * 2 = 4.23e9 B);
    40 shard rows at ldw = 53,687,088 (39 * ldw * 2 = 4.19e9 B);
  * large-batch kernel, 128-row blocks: 128 rows at ldx = 2^24 - 8;
  * large-batch kernel, 256-row blocks: 256 rows at ldx = 2^23 - 8, and 72
    shard rows at ldw = 29,826,160 (71 * ldw * 2 = 4.24e9 B);
  * partial completion: a 1024-row weight chunk (plus 8 rows of slack) at
    ldw = 2,080,888 and 64 activation rows at ldx = 2^25 - 8.

The strides are padding around a small head (H = 64): the padding holds NaN
bits that must never be read.  Each case moves a few GB to the device.
"""
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs
from oracle import partial as opart
from tests.gpu_common import check_against_oracle, check_internal, run_surfaces, upload
from tests.test_gpu_partial import check, run
from tests.test_gpu_partial import upload as upload_partial

pytestmark = pytest.mark.gpu

H = 64

CASES = [
    # name, B, V, lane offsets, ldx, ldw (None: the natural stride)
    ("decode-ldx", 64, 1000, [0, 504, 1000], (1 << 25) - 8, None),
    ("decode-ldw", 16, 1000, [0, 1000], None, 53687088),
    ("large128-ldx", 128, 1000, [0, 504, 1000], (1 << 24) - 8, None),
    ("large256-ldx", 256, 1000, [0, 504, 1000], (1 << 23) - 8, None),
    ("large256-ldw", 300, 1000, [0, 1000], None, 29826160),
]


@pytest.mark.parametrize("name,B,V,off,ldx,ldw", CASES, ids=[c[0] for c in CASES])
def test_largest_accepted_strides(require_gpu, name, B, V, off, ldx, ldw):
    print(f"stride limit {name}: B={B} H={H} V={V} ldx={ldx} ldw={ldw}", flush=True)
    d = inputs.make_random(B, H, V, off, seed=5000 + B)
    widest = max(off[i + 1] - off[i] for i in range(len(off) - 1))
    head = upload(d, lanes_separate=True,
                  pad_x=0 if ldx is None else ldx - H,
                  pad_w=0 if ldw is None else ldw - (widest + 7) // 8 * 8)
    if ldx is not None:
        assert head.desc.ldx == ldx
    if ldw is not None:
        assert head.desc.ldw == ldw
    g = run_surfaces(head)
    check_internal(g)
    check_against_oracle(g, oracle.logits(d["x"], d["w"]), off)
    del head
    torch.cuda.empty_cache()


# Partial completion: a chunk of 1024 weight rows (plus 8 of slack) and a
# group of 64 activation rows are addressed from their bases the same way.
PARTIAL_CASES = [
    # name, B, K per lane, N, ldx, ldw
    ("partial-ldw", 16, (1100,), 100, None, 2080888),   # 1023 * ldw * 2 = 4.26e9 B
    ("partial-ldx", 64, (300, 200), 100, (1 << 25) - 8, None),
]


@pytest.mark.parametrize("name,B,Ks,N,ldx,ldw", PARTIAL_CASES, ids=[c[0] for c in PARTIAL_CASES])
def test_largest_accepted_partial_strides(require_gpu, name, B, Ks, N, ldx, ldw):
    print(f"stride limit {name}: B={B} Ks={Ks} N={N} ldx={ldx} ldw={ldw}", flush=True)
    xs, ws = inputs.draw_partial(B, N, Ks, seed=5100 + B, sigma_w=0.05)
    part = upload_partial(xs, ws,
                          pad_x=0 if ldx is None else ldx - (max(Ks) + 7) // 8 * 8,
                          pad_w=0 if ldw is None else ldw - (N + 7) // 8 * 8)
    if ldx is not None:
        assert part.desc.ldx == ldx
    if ldw is not None:
        assert part.desc.ldw == ldw
    P = opart.partials(xs, ws)
    for op in opart.OPS:
        check(run(part, op), P, op)
    del part
    torch.cuda.empty_cache()
