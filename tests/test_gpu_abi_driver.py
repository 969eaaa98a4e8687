"""GPU test of libsb as a standalone C ABI: tests/abi_driver (a C99 program
built from tests/abi_driver.c by build(), linking only libsb.so and the HIP
runtime) allocates its own device buffers, calls every head entry point on
one stream and writes the results to files.  Its results must meet the same
acceptance rules against the oracle as the Python binding's, agree across
surfaces bit for bit, and equal the binding's results on the same inputs bit
for bit (both place every shard at the start of an allocation)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from logit_source_projection_amd import inputs, sb
from logit_source_projection_amd.build import DRIVER, build_abi_driver
from tests.gpu_common import check_against_oracle, check_internal, run_surfaces, upload

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, V, lane offsets
    ("tiny", None, None, None, None),
    ("ragged", 37, 777, 5003, [0, 1000, 1001, 2999, 4000, 5003]),
    ("large-batch", 150, 300, 3000, [0, 1200, 2100, 3000]),
]


def _run_driver(tmp_path, d):
    B, H, V = d["B"], d["H"], d["V"]
    off = d["lane_off"]
    (tmp_path / "head.txt").write_text(" ".join(str(v) for v in [B, H, V, len(off) - 1] + off))
    d["x"].astype(np.uint16).tofile(tmp_path / "x.bin")
    d["w"].astype(np.uint16).tofile(tmp_path / "w.bin")
    r = subprocess.run([DRIVER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    k = len(off) - 1

    def load(name, dtype, shape):
        return np.fromfile(tmp_path / name, dtype=dtype).reshape(shape)

    return dict(ids_tok=load("ids_tok.bin", np.int32, (B,)),
                ids_static=load("ids_static.bin", np.int32, (B,)),
                ids_lp=load("ids_lp.bin", np.int32, (B,)),
                ids_r0=load("ids_r0.bin", np.int32, (B,)),
                lane_ids=load("lane_ids.bin", np.int32, (B, k)),
                lane_max=load("lane_max.bin", np.float32, (B, k)),
                lse=load("lse.bin", np.float32, (B,)),
                sel_lp=load("sel.bin", np.float32, (B,)),
                logprobs=load("lp.bin", np.float32, (B, V)),
                logits=load("logits.bin", np.float32, (B, V)))


@pytest.mark.parametrize("name,B,H,V,off", CASES, ids=[c[0] for c in CASES])
def test_c_driver(require_gpu, tmp_path, name, B, H, V, off):
    if not os.path.exists(DRIVER):
        build_abi_driver()  # built by build(); compiled here only if it is missing
    print(f"C driver case {name}", flush=True)
    d = (inputs.make_workload("tiny") if name == "tiny"
         else inputs.make_random(B, H, V, off, seed=B + H))
    g = _run_driver(tmp_path, d)
    check_internal(g)
    assert np.array_equal(g["ids_static"], g["ids_tok"])
    off = d["lane_off"]
    for i in range(len(off) - 1):
        seg = g["logits"][:, off[i]:off[i + 1]]
        assert np.array_equal(g["lane_ids"][:, i], off[i] + np.argmax(seg, axis=1)), i
        assert np.array_equal(g["lane_max"][:, i], seg.max(axis=1)), i
    z = oracle.logits(d["x"], d["w"])
    check_against_oracle(g, z, off)
    if name == "tiny":
        row, a, _ = d["planted"][0]
        assert g["ids_tok"][row] == a

    # the Python binding on the same inputs, every lane in its own allocation
    # and x at the driver's row stride (H rounded up to a multiple of 8)
    b = run_surfaces(upload(d, lanes_separate=True, pad_x=(8 - d["H"] % 8) % 8))
    for key in ("ids_tok", "ids_lp", "ids_r0", "lse", "sel_lp", "logits", "logprobs"):
        assert np.array_equal(g[key], b[key]), key
    torch.cuda.synchronize()
