"""The C ABI library on the host: it loads, exports every call that
include/sb.h declares, and its validation rejects bad arguments with the
documented status before any GPU work (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from logit_source_projection_amd import sb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "sb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sb_\w+)\s*\(", text)))


def test_header_declares_the_calls():
    assert header_functions() == sorted(sb.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = sb.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sb.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    # the header's calls and nothing else: the C++ launchers stay local
    assert exported == set(header_functions()), exported ^ set(header_functions())


def test_status_strings():
    for st in range(-7, 1):
        s = sb.status_string(st)
        assert s and s != "unknown status"
    assert sb.status_string(-99) == "unknown status"


# Fake, aligned host "device" pointers: validation never dereferences them and
# every call below fails validation before anything is launched.
FAKE = 1 << 20


def fake_head(B=16, H=512, V=4096, off=(0, 2048, 4096), ldx=None, ldw=None,
              x_ptr=FAKE, w_ptrs=None):
    x = torch.empty(0)
    off = list(off)
    k = len(off) - 1
    if w_ptrs is None:
        w_ptrs = [FAKE + 2 * off[i] for i in range(k)]
    return sb.Head(x, torch.empty(0), off, B=B, H=H, V=V,
                   ldx=H if ldx is None else ldx, ldw=V if ldw is None else ldw,
                   x_ptr=x_ptr, w_ptrs=w_ptrs)


def ws_status(head, surface=sb.SB_SURF_TOKENS):
    st = ctypes.c_int(123)
    sb.lib().sb_workspace_bytes(head.ref(), surface, ctypes.byref(st))
    return st.value


def tokens_status(head, ids=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return sb.lib().sb_project_tokens(head.ref(), ids, ws, ws_bytes, None)


def up256(n):
    return (n + 255) // 256 * 256


# Every workspace starts with one fixed region, whatever the call: 2048
# per-tile slice counters (u32) of a head split into K slices.
ZERO = 2048 * 4


def cap(off):
    """Tile capacity: per lane ceil((V_i + 56) / 128), room for a lane grid
    shifted by up to 56 columns onto a cache-line boundary."""
    return sum((off[i + 1] - off[i] + 56 + 127) // 128 for i in range(len(off) - 1))


def pairs(B, off):
    """The (row, tile) results the combine launch folds: 8 B per (row, tile)."""
    return up256(B * cap(off) * 8)


def test_workspace_bytes_for_the_workloads():
    assert ZERO == 8192
    off = (0, 37984, 75968, 113952, 151936)
    h = fake_head(B=16, H=5120, V=151936, off=off)
    assert cap(off) == 4 * 298
    # the dense head has enough tiles (1187) for one workgroup each: no
    # slices; the (max, lowest index) pair of every (row, tile)
    assert sb.sb_workspace_bytes(h, sb.SB_SURF_TOKENS) == ZERO + pairs(16, off)
    # + the (tile max, sum-exp) pairs
    lp = sb.sb_workspace_bytes(h, sb.SB_SURF_LOGPROBS)
    assert lp == ZERO + 2 * pairs(16, off)
    assert sb.sb_workspace_bytes(h, sb.SB_SURF_LOGPROBS_FULL) == lp
    # large batches: the same regions
    hl = fake_head(B=300, H=5120, V=151936, off=off)
    assert sb.sb_workspace_bytes(hl, sb.SB_SURF_TOKENS) == ZERO + pairs(300, off)
    full = sb.sb_workspace_bytes(h, sb.SB_SURF_FULL_LOGITS)
    assert full >= ZERO + 16 * 151936 * 4
    assert sb.sb_workspace_bytes(fake_head(B=0), sb.SB_SURF_TOKENS) == 0


def test_workspace_bytes_of_a_split_head():
    # A head of 64 tiles (V = 8192) splits its 160 hidden steps into 4 slices
    # of 40, and each slice writes a 16 x 128 fp32 partial tile per tile of
    # the capacity (65 tiles, with room for a lane grid shifted by 56 columns).
    off = (0, 8192)
    h = fake_head(B=16, H=5120, V=8192, off=off)
    assert sb.sb_workspace_bytes(h, sb.SB_SURF_TOKENS) == \
        ZERO + 65 * 4 * 16 * 128 * 4 + pairs(16, off)
    # the split depends on (B, H, V), not on the lane split
    off4 = (0, 2048, 4096, 6144, 8192)
    h4 = fake_head(B=16, H=5120, V=8192, off=off4)
    assert sb.sb_workspace_bytes(h4, sb.SB_SURF_TOKENS) == \
        ZERO + 4 * 17 * 4 * 16 * 128 * 4 + pairs(16, off4)
    # 127 tiles: 3 slices (of 56, 56 and 48 steps); 64 rows: 64-row partial tiles,
    # then the hidden rows packed per 32-deep step (4 row blocks x 64 lanes x 16 B)
    off = (0, 16256)
    h = fake_head(B=64, H=5120, V=16256, off=off)
    assert sb.sb_workspace_bytes(h, sb.SB_SURF_TOKENS) == \
        ZERO + 128 * 3 * 64 * 128 * 4 + 160 * 4096 + pairs(64, off)
    # one GPU's lane of the dense head (297 tiles, just past one tile per CU,
    # 16 rows): 2 slices of 80 steps, partial tiles for the 298 tiles of capacity
    off = (0, 37984)
    assert sb.sb_workspace_bytes(fake_head(B=16, H=5120, V=37984, off=off),
                                 sb.SB_SURF_TOKENS) == ZERO + 298 * 2 * 16 * 128 * 4 + pairs(16, off)
    # ... but not at 17 rows, at H = 2048 (64 steps), at 256 or at 353 tiles
    for kw in (dict(B=17, H=5120, V=37984), dict(B=16, H=2048, V=37984),
               dict(B=16, H=5120, V=256 * 128), dict(B=16, H=5120, V=353 * 128)):
        off = (0, kw["V"])
        assert sb.sb_workspace_bytes(fake_head(off=off, **kw),
                                     sb.SB_SURF_TOKENS) == ZERO + pairs(kw["B"], off), kw
    # one GPU's lane of the MoE head (594 tiles): the packed hidden rows only
    off = (0, 75968)
    assert sb.sb_workspace_bytes(fake_head(B=64, H=4096, V=75968, off=off),
                                 sb.SB_SURF_TOKENS) == ZERO + 128 * 4096 + pairs(64, off)
    # fewer than 32 hidden steps (H <= 992): never split
    off = (0, 1024)
    assert sb.sb_workspace_bytes(fake_head(B=16, H=992, V=1024, off=off),
                                 sb.SB_SURF_TOKENS) == ZERO + pairs(16, off)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), sb.SB_ERR_SHAPE),
    (dict(H=-5), sb.SB_ERR_SHAPE),
    (dict(V=0, off=(0, 0)), sb.SB_ERR_SHAPE),
    (dict(off=(0, 4096), V=4000), sb.SB_ERR_LANES),
    (dict(off=(0, 2048, 2048, 4096)), sb.SB_ERR_LANES),
    (dict(off=(0, 3000, 2048, 4096)), sb.SB_ERR_LANES),
    (dict(off=(8, 2048, 4096)), sb.SB_ERR_LANES),
    (dict(ldx=256), sb.SB_ERR_SHAPE),
    (dict(ldw=2000), sb.SB_ERR_SHAPE),
    (dict(ldx=516), sb.SB_ERR_ALIGN),
    (dict(ldw=4100), sb.SB_ERR_ALIGN),
    (dict(x_ptr=FAKE + 2), sb.SB_ERR_ALIGN),
    (dict(w_ptrs=[FAKE, FAKE + 2 * 2047]), sb.SB_ERR_ALIGN),
    (dict(x_ptr=0), sb.SB_ERR_NULL),
    (dict(w_ptrs=[FAKE, 0]), sb.SB_ERR_NULL),
    (dict(B=1 << 24), sb.SB_ERR_UNSUPPORTED),  # the combine's grid: 2^32 work items
    (dict(ldx=1 << 25), sb.SB_ERR_UNSUPPORTED),  # 64 rows of x span 4 GiB
    (dict(V=(1 << 31) - 8, off=(0, (1 << 31) - 8), ldw=(1 << 31) - 8), sb.SB_ERR_UNSUPPORTED),
])
def test_descriptor_validation(kw, status):
    h = fake_head(**kw)
    assert ws_status(h) == status
    assert tokens_status(h) == status


def test_large_batch_offset_limits():
    """The kernels' 32-bit buffer offsets: up to 64 rows the decode kernels
    reach 64 rows of x and 40 rows of a shard; from 65 to 128 rows the
    large-batch kernel's 128-row blocks reach 128 rows of x and 32-row K
    stages (plus 8 rows of slack: 40 shard rows); from 129 rows its 256-row
    blocks reach 256 rows of x and 64-row K stages (72 shard rows).
    Validation rejects strides where those reach 4 GiB and accepts them just
    below."""
    lim = 1 << 32
    ldx256 = 1 << 23                # 256 rows x 2 B = 4 GiB
    ldx128 = 1 << 24                # 128 rows x 2 B = 4 GiB
    ldw = 29826168                  # 72 rows x 2 B >= 4 GiB > 40 rows x 2 B
    assert 256 * ldx256 * 2 >= lim and 128 * ldx128 * 2 >= lim and 64 * (ldx128 - 8) * 2 < lim
    assert 72 * ldw * 2 >= lim and 40 * ldw * 2 < lim
    # x: 256-row blocks from 129 rows, 128-row blocks from 65 to 128 rows
    assert ws_status(fake_head(B=129, ldx=ldx256)) == sb.SB_ERR_UNSUPPORTED
    assert ws_status(fake_head(B=129, ldx=ldx256 - 8)) == sb.SB_OK
    assert ws_status(fake_head(B=128, ldx=ldx256)) == sb.SB_OK
    assert ws_status(fake_head(B=128, ldx=ldx128)) == sb.SB_ERR_UNSUPPORTED
    assert ws_status(fake_head(B=65, ldx=ldx128)) == sb.SB_ERR_UNSUPPORTED
    assert ws_status(fake_head(B=65, ldx=ldx128 - 8)) == sb.SB_OK
    assert ws_status(fake_head(B=64, ldx=ldx128 - 8)) == sb.SB_OK
    # shard rows: 72 from 129 rows, 40 below
    assert ws_status(fake_head(B=129, ldw=ldw)) == sb.SB_ERR_UNSUPPORTED
    assert ws_status(fake_head(B=128, ldw=ldw)) == sb.SB_OK
    assert ws_status(fake_head(B=65, ldw=ldw)) == sb.SB_OK
    assert ws_status(fake_head(B=2048, ldw=ldw - 8)) == sb.SB_OK
    assert tokens_status(fake_head(B=129, ldx=ldx256)) == sb.SB_ERR_UNSUPPORTED
    assert tokens_status(fake_head(B=100, ldx=ldx128)) == sb.SB_ERR_UNSUPPORTED
    assert tokens_status(fake_head(B=300, ldw=ldw)) == sb.SB_ERR_UNSUPPORTED


def test_launch_size_limits():
    """Every launch of a call fits one grid: fewer than 2^32 work items in its
    x dimension.  The launches with one row per y index run over batches of
    more than 65535 rows in slices, so B is not bounded by the y dimension."""
    lim = 1 << 32
    # (accepted descriptors are only sized, never run: their pointers are fake)
    for B in (65535, 65536, 70000, 1 << 20):
        assert ws_status(fake_head(B=B)) == sb.SB_OK, B
    # the combine: one 256-item workgroup per row
    assert (1 << 24) * 256 >= lim and ((1 << 24) - 1) * 256 < lim
    assert ws_status(fake_head(B=(1 << 24) - 1)) == sb.SB_OK
    assert ws_status(fake_head(B=1 << 24)) == sb.SB_ERR_UNSUPPORTED
    # the large-batch kernel: 512-item workgroups over 256-row m-blocks and
    # 256-column n-blocks, here 4096 m-blocks in super tiles of 8 x 4 blocks
    # (32 workgroups), a multiple of 8 super tiles; an n-block count includes
    # up to 56 columns of tile shift
    def items(nblocks):
        supers = 4096 // 8 * -(-nblocks // 4)
        return -(-supers // 8) * 8 * 32 * 512

    B = 1 << 20
    big = fake_head(B=B, V=1 << 20, off=(0, 1 << 20))
    small = fake_head(B=B, V=1 << 18, off=(0, 1 << 18))
    assert items(4097) >= lim > items(1025)
    assert ws_status(big) == sb.SB_ERR_UNSUPPORTED
    assert tokens_status(big) == sb.SB_ERR_UNSUPPORTED
    assert ws_status(small) == sb.SB_OK


def test_vocabulary_limit():
    """V <= 2^30 (32-bit column arithmetic with room for rounding), here over
    64 lanes so that no shard's 72-row step reaches 4 GiB; the decode
    kernel's one 256-item workgroup per 128-column tile then stays below
    2^32 work items."""
    for V, status in ((1 << 30, sb.SB_OK), ((1 << 30) + 8, sb.SB_ERR_UNSUPPORTED)):
        off = [V * i // 64 // 8 * 8 for i in range(64)] + [V]
        wide = max(off[i + 1] - off[i] for i in range(64))
        assert 72 * wide * 2 < 1 << 32 and (V // 128 + 64 + 8) * 256 < 1 << 32
        for B in (1, 64, 65, 200):
            h = fake_head(B=B, V=V, off=off, ldw=(wide + 7) // 8 * 8, w_ptrs=[FAKE] * 64)
            assert ws_status(h) == status, (V, B)


def test_partial_launch_size_limits():
    """The chunked partial GEMM runs ceil(B / 64) row groups (from 33 rows)
    for every chunk and 128-column tile in one grid of 256-item workgroups:
    18 chunks x 40 tiles here."""
    lim = 1 << 32
    ok_rows = (lim - 1) // (18 * 40 * 256) * 64
    assert 18 * 40 * (ok_rows // 64) * 256 < lim <= 18 * 40 * (ok_rows // 64 + 1) * 256
    for B, status in ((70000, sb.SB_OK), (ok_rows, sb.SB_OK),
                      (ok_rows + 1, sb.SB_ERR_UNSUPPORTED)):
        p = fake_partial(B=B)
        st = ctypes.c_int(123)
        sb.lib().sb_partial_workspace_bytes(p.ref(), ctypes.byref(st))
        assert st.value == status, B
    # (only the refused descriptor is passed to the call: the pointers are fake)
    assert partial_status(fake_partial(B=ok_rows + 1), ws_bytes=1 << 62) == sb.SB_ERR_UNSUPPORTED


def test_lane_results_checks():
    h = fake_head()
    L = sb.lib()
    need = sb.sb_workspace_bytes(h, sb.SB_SURF_TOKENS)
    # ids are required, the per-lane outputs are optional; the token
    # surface's workspace size applies
    assert L.sb_project_lane_results(h.ref(), None, FAKE, FAKE, FAKE, need, None) == sb.SB_ERR_NULL
    assert L.sb_project_lane_results(h.ref(), FAKE, None, None, FAKE, need - 1,
                                     None) == sb.SB_ERR_WORKSPACE
    assert L.sb_project_lane_results(fake_head(B=-1).ref(), FAKE, FAKE, FAKE, FAKE, need,
                                     None) == sb.SB_ERR_SHAPE
    assert L.sb_project_lane_results(fake_head(B=0, x_ptr=0).ref(), None, None, None, None, 0,
                                     None) == sb.SB_OK


def test_static_scratch_call_checks():
    """The no-allocation token call validates like sb_project_tokens and
    refuses, before touching the device, a call whose workspace would not fit
    its static array."""
    L = sb.lib()
    assert L.sb_project_tokens_static(fake_head(B=-1).ref(), FAKE, None) == sb.SB_ERR_SHAPE
    assert L.sb_project_tokens_static(fake_head().ref(), None, None) == sb.SB_ERR_NULL
    assert L.sb_project_tokens_static(fake_head(B=0, x_ptr=0).ref(), None, None) == sb.SB_OK
    big = fake_head(B=4096, H=64, V=151936, off=(0, 37984, 75968, 113952, 151936))
    assert sb.sb_workspace_bytes(big, sb.SB_SURF_TOKENS) > sb.SB_STATIC_SCRATCH_BYTES
    assert L.sb_project_tokens_static(big.ref(), FAKE, None) == sb.SB_ERR_WORKSPACE
    text = open(os.path.join(ROOT, "include", "sb.h")).read()
    assert "#define SB_STATIC_SCRATCH_BYTES ((size_t)32 << 20)" in text
    assert sb.SB_STATIC_SCRATCH_BYTES == 32 << 20


def test_too_many_lanes():
    V = 8 * 65
    off = list(range(0, V + 1, 8))
    assert len(off) - 1 == 65
    assert ws_status(fake_head(V=V, off=off, ldw=V)) == sb.SB_ERR_LANES


def test_output_and_workspace_checks():
    h = fake_head()
    need = sb.sb_workspace_bytes(h, sb.SB_SURF_TOKENS)
    assert tokens_status(h, ids=None) == sb.SB_ERR_NULL
    assert tokens_status(h, ws=None) == sb.SB_ERR_NULL
    assert tokens_status(h, ws_bytes=need - 1) == sb.SB_ERR_WORKSPACE
    assert tokens_status(h, ws=FAKE + 4) == sb.SB_ERR_ALIGN
    L = sb.lib()
    # log-prob surface: lse required, logprobs stride / alignment
    assert L.sb_project_logprobs(h.ref(), FAKE, None, None, None, 0, FAKE, 1 << 30, None) == sb.SB_ERR_NULL
    assert L.sb_project_logprobs(h.ref(), FAKE, FAKE, None, FAKE, 4000, FAKE, 1 << 30, None) == sb.SB_ERR_SHAPE
    assert L.sb_project_logprobs(h.ref(), FAKE, FAKE, None, FAKE, 4098, FAKE, 1 << 30, None) == sb.SB_ERR_ALIGN
    assert L.sb_project_logprobs(h.ref(), FAKE, FAKE, None, FAKE + 8, 4096, FAKE, 1 << 30, None) == sb.SB_ERR_ALIGN
    # full-logit plan
    assert L.sb_full_logits(h.ref(), None, 4096, None, FAKE, 1 << 30, None) == sb.SB_ERR_NULL
    assert L.sb_full_logits(h.ref(), FAKE, 4095, None, FAKE, 1 << 30, None) == sb.SB_ERR_SHAPE
    assert L.sb_full_logits(h.ref(), FAKE, 4098, None, FAKE, 1 << 30, None) == sb.SB_ERR_ALIGN
    need_full = sb.sb_workspace_bytes(h, sb.SB_SURF_FULL_LOGITS)
    assert L.sb_full_logits(h.ref(), FAKE, 4096, None, FAKE, need_full - 1, None) == sb.SB_ERR_WORKSPACE


def test_empty_batch_is_a_noop():
    h = fake_head(B=0, x_ptr=0)
    # nothing to do: no pointer is needed and nothing is launched
    assert tokens_status(h, ids=None, ws=None, ws_bytes=0) == sb.SB_OK
    L = sb.lib()
    assert L.sb_project_logprobs(h.ref(), None, None, None, None, 0, None, 0, None) == sb.SB_OK
    assert L.sb_full_logits(h.ref(), None, 0, None, None, 0, None) == sb.SB_OK


def test_binding_raises_on_error():
    h = fake_head(B=-1)
    with pytest.raises(sb.SbError) as e:
        sb.sb_workspace_bytes(h, sb.SB_SURF_TOKENS)
    assert e.value.status == sb.SB_ERR_SHAPE


# ---------------------------------------------------------------------------
# partial completion
# ---------------------------------------------------------------------------
def fake_partial(B=16, N=5120, lane_k=(0, 8704, 17408), ldx=None, ldw=None,
                 x_ptrs=None, w_ptrs=None):
    k = len(lane_k) - 1
    Ks = [lane_k[i + 1] - lane_k[i] for i in range(k)]
    return sb.Partial([torch.empty(0, 1)] * k, [torch.empty(0, 1)] * k, B=B, N=N,
                      lane_k=list(lane_k), ldx=max(Ks) if ldx is None else ldx,
                      ldw=N if ldw is None else ldw,
                      x_ptrs=[FAKE] * k if x_ptrs is None else x_ptrs,
                      w_ptrs=[FAKE] * k if w_ptrs is None else w_ptrs)


def partial_status(p, op=sb.SB_RED_SUM, out=FAKE, ldo=None, ws=FAKE, ws_bytes=1 << 30):
    return sb.lib().sb_partial_complete(p.ref(), op, out, p.N if ldo is None else ldo, ws,
                                        ws_bytes, None)


def test_partial_workspace_bytes():
    # two lanes of 8704 rows -> 9 + 9 chunks of 1024 rows, fp32 [B][N] each
    # (after the head calls' counter region, so that one workspace serves both)
    p = fake_partial()
    assert sb.sb_partial_workspace_bytes(p) == ZERO + 18 * 16 * 5120 * 4
    # ragged: 1000 + 1025 rows -> 1 + 2 chunks; N = 130 -> row stride 132
    p = fake_partial(B=3, N=130, lane_k=(0, 1000, 2025), ldx=1032, ldw=136)
    assert sb.sb_partial_workspace_bytes(p) == ZERO + up256(3 * 3 * 132 * 4)
    assert sb.sb_partial_workspace_bytes(fake_partial(B=0)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), sb.SB_ERR_SHAPE),
    (dict(N=0, ldw=8), sb.SB_ERR_SHAPE),
    (dict(lane_k=(0, 100, 100)), sb.SB_ERR_LANES),
    (dict(lane_k=(8, 100)), sb.SB_ERR_LANES),
    (dict(lane_k=tuple(range(0, 8 * 66, 8))), sb.SB_ERR_LANES),
    (dict(ldx=8000), sb.SB_ERR_SHAPE),
    (dict(ldw=5000), sb.SB_ERR_SHAPE),
    (dict(ldx=8708), sb.SB_ERR_ALIGN),
    (dict(ldw=5124), sb.SB_ERR_ALIGN),
    (dict(x_ptrs=[FAKE, FAKE + 8]), sb.SB_ERR_ALIGN),
    (dict(w_ptrs=[FAKE + 2, FAKE]), sb.SB_ERR_ALIGN),
    (dict(x_ptrs=[FAKE, 0]), sb.SB_ERR_NULL),
    (dict(w_ptrs=[0, FAKE]), sb.SB_ERR_NULL),
    (dict(B=1 << 24), sb.SB_ERR_UNSUPPORTED),  # the chunked GEMM's grid
    (dict(ldw=1 << 21), sb.SB_ERR_UNSUPPORTED),  # a 1024-row chunk spans 4 GiB
])
def test_partial_descriptor_validation(kw, status):
    p = fake_partial(**kw)
    st = ctypes.c_int(123)
    sb.lib().sb_partial_workspace_bytes(p.ref(), ctypes.byref(st))
    assert st.value == status
    assert partial_status(p) == status


def test_partial_output_and_workspace_checks():
    p = fake_partial()
    need = sb.sb_partial_workspace_bytes(p)
    assert partial_status(p, op=4) == sb.SB_ERR_SHAPE
    assert partial_status(p, op=-1) == sb.SB_ERR_SHAPE
    assert partial_status(p, out=None) == sb.SB_ERR_NULL
    assert partial_status(p, ldo=5119) == sb.SB_ERR_SHAPE
    assert partial_status(p, ldo=5122) == sb.SB_ERR_ALIGN
    assert partial_status(p, out=FAKE + 8) == sb.SB_ERR_ALIGN
    assert partial_status(p, ws=None) == sb.SB_ERR_NULL
    assert partial_status(p, ws_bytes=need - 1) == sb.SB_ERR_WORKSPACE
    assert partial_status(p, ws=FAKE + 4) == sb.SB_ERR_ALIGN
    # an empty batch is a valid no-op that touches nothing
    assert partial_status(fake_partial(B=0), out=None, ws=None, ws_bytes=0) == sb.SB_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libsb.so every call raises; nothing falls back to another path."""
    monkeypatch.setattr(sb, "_lib", None)
    monkeypatch.setattr(sb, "LIB_PATH", str(tmp_path / "libsb.so"))
    with pytest.raises(RuntimeError, match="libsb.so not found"):
        sb.lib()
    with pytest.raises(RuntimeError, match="libsb.so not found"):
        sb.sb_workspace_bytes(fake_head(), sb.SB_SURF_TOKENS)


def test_header_compiles_as_c99():
    """include/sb.h is a C header: it compiles as strict C99 with every
    warning an error, with no C++ and no HIP header."""
    import shutil
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    with tempfile.TemporaryDirectory() as t:
        src = os.path.join(t, "use_sb.c")
        with open(src, "w") as f:
            f.write('#include "sb.h"\n'
                    "int use(const sb_head_desc *d, int32_t *ids) {\n"
                    "    return (int)sb_project_tokens(d, ids, (void *)0, 0, (void *)0);\n"
                    "}\n")
        r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                            "-fsyntax-only", "-I", inc, src], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_binding_refuses_arguments_the_abi_cannot_take():
    """The Python binding raises, before anything reaches the library, on host
    tensors and wrong dtypes (which would otherwise reach a kernel as raw
    pointers).  Without a GPU only each call's first checked argument can be
    exercised; the GPU tests run every call with valid device arguments."""
    h = fake_head()                                  # raw device pointers: B=16, V=4096
    with pytest.raises(ValueError, match="ids must be a device tensor"):
        sb.sb_project_tokens(h, torch.empty(16, dtype=torch.int32))
    with pytest.raises(ValueError, match="ids must be a device tensor"):
        sb.sb_project_tokens_static(h, torch.empty(16, dtype=torch.int64))
    with pytest.raises(ValueError, match="ids must be a device tensor"):
        sb.sb_project_lane_results(h, torch.empty(16, dtype=torch.int32))
    with pytest.raises(ValueError, match="ids must be a device tensor"):
        sb.sb_project_logprobs(h, torch.empty(16, dtype=torch.int32), torch.empty(16))
    with pytest.raises(ValueError, match="logits must be a device tensor"):
        sb.sb_full_logits(h, torch.empty(16, 4096))
    # a descriptor built from host tensors is refused as a whole
    host = sb.Head(torch.empty(16, 512, dtype=torch.bfloat16),
                   torch.empty(512, 4096, dtype=torch.bfloat16), [0, 2048, 4096])
    with pytest.raises(ValueError, match="x must be a device tensor"):
        sb.sb_project_tokens(host, None)
    part = sb.Partial([torch.empty(4, 64, dtype=torch.bfloat16)],
                      [torch.empty(64, 128, dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="x must be a device tensor"):
        sb.sb_partial_complete(part, "sum", None)
