"""Seeded synthetic inputs for the output-head workloads.

This module only *draws* inputs: hidden rows X [B, H] and head weights W [H, V]
as bfloat16 bit patterns (numpy uint16), plus the lane offsets.  It holds none
of the projection's arithmetic, so both the GPU path's tests and the CPU oracle
can consume what it produces.

Recipe (the pages measure on real checkpoints and prompts that are not
available; these draws stand in for them with the same head shapes):

* X is drawn with ``numpy.random.default_rng([seed, 0])`` as float32
  ``standard_normal``, optionally RMS-normalised per row in float32
  (``x / sqrt(mean(x^2) + 1e-6)``, unit gain), then rounded to bf16
  (round-to-nearest-even).
* W is drawn in row chunks of ``_CHUNK_ROWS`` rows; chunk c uses
  ``numpy.random.default_rng([seed, 1, c])`` and draws float32
  ``standard_normal``, times sigma, then rounds to bf16.  Chunks are
  independent streams, so they are drawn on a thread pool.
* Lanes are contiguous column ranges; the named workloads use k equal lanes.
* Planted ties: the tiny head plants an exact tie in one row; the large-vocab
  head plants near-ties (gap about 1e-4) in ceil(10%) of its rows.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_CHUNK_ROWS = 256


def f32_to_bf16_bits(a):
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits.
    Inputs are finite by construction."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns (uint16) to float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def equal_lanes(V, k):
    """k contiguous lanes; equal when k divides V, else the first V % k lanes
    are one column wider."""
    if k < 1 or k > V:
        raise ValueError("need 1 <= k <= V")
    base, extra = divmod(V, k)
    off = [0]
    for i in range(k):
        off.append(off[-1] + base + (1 if i < extra else 0))
    return off


def draw_hidden(B, H, seed=0, rms_norm=False, sigma=1.0):
    """X [B, H] as bf16 bits."""
    rng = np.random.default_rng([seed, 0])
    x = rng.standard_normal((B, H), dtype=np.float32) * np.float32(sigma)
    if rms_norm:
        ms = (x * x).mean(axis=1, keepdims=True, dtype=np.float32)
        x = x / np.sqrt(ms + np.float32(1e-6))
    return f32_to_bf16_bits(x)


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_weight(H, V, sigma, seed=0):
    """W [H, V] as bf16 bits, drawn in independent row chunks."""
    w = np.empty((H, V), dtype=np.uint16)
    s = np.float32(sigma)

    def chunk(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(H, r0 + _CHUNK_ROWS)
        rng = np.random.default_rng([seed, 1, c])
        a = rng.standard_normal((r1 - r0, V), dtype=np.float32)
        a *= s
        w[r0:r1] = f32_to_bf16_bits(a)

    nchunks = (H + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(chunk, range(nchunks)))
    return w


def plant_equal_columns(x_bits, w_bits, row, cols, target):
    """Make the columns ``cols`` of W identical and equal to
    bf16(target * x_r / |x_r|^2) for hidden row r, so that row r's logits at
    those columns are exactly equal and close to ``target``."""
    xr = bf16_bits_to_f32(x_bits[row]).astype(np.float64)
    col = f32_to_bf16_bits((target * xr / np.dot(xr, xr)).astype(np.float32))
    for c in cols:
        w_bits[:, c] = col
    return w_bits


def plant_near_tie(x_bits, w_bits, row, a, b, target=8.0, delta=1e-4):
    """Plant a near-tie in row r between columns a < b: both columns get
    bf16(target * x_r / |x_r|^2), then column b's element at the h whose
    |x_r[h]| is closest to 2 is raised by about delta / x_r[h], so column b
    wins by about delta (the realised gap is whatever bf16 rounding leaves)."""
    plant_equal_columns(x_bits, w_bits, row, (a, b), target)
    xr = bf16_bits_to_f32(x_bits[row]).astype(np.float64)
    h = int(np.argmin(np.abs(np.abs(xr) - 2.0)))
    wa = float(bf16_bits_to_f32(w_bits[h, a]))
    w_bits[h, b] = f32_to_bf16_bits(np.float32(wa + delta / xr[h]))
    return h


# --------------------------------------------------------------------------
# Named workloads (head shapes of the pages' Dense TP4, MoE TP2 and MiniMax
# deployments; SemBridge section 6.1).
# --------------------------------------------------------------------------

WORKLOADS = {
    # name: (B, H, V, k, sigma_w, rms_norm_x)
    "tiny": (4, 256, 4096, 2, 0.02, False),
    "dense_decode": (16, 5120, 151936, 4, 0.02, False),
    "moe_decode": (64, 4096, 151936, 2, 0.02, True),
    "large_vocab": (16, 6144, 200064, 4, 0.015, False),
    "prefill": (2048, 5120, 151936, 4, 0.02, False),
    # one GPU's lane of the dense head when it is sharded over 4 GPUs
    "dense_share": (16, 5120, 37984, 1, 0.02, False),
}

# Weight row stride (elements) where it is not V: the dense share's rows are
# padded to 76,032 bytes (an odd multiple of 256), as a deployment would lay
# out one GPU's shard; its own width puts every other row 64 bytes into a
# cache line.
WORKLOAD_LDW = {"dense_share": 38016}

TINY_TIE_ROW = 1
TINY_TIE_COLS = (1000, 3000)


def near_tie_rows(B):
    """Rows that carry a planted near-tie: n = ceil(0.1 B) rows at
    floor(j B / n)."""
    n = max(1, math.ceil(0.1 * B))
    return [(j * B) // n for j in range(n)]


def near_tie_cols(lane_off):
    """Column pairs (a < b) for the planted near-ties: the first straddles the
    boundary between lanes 0 and 1, the second lies inside the last lane."""
    off = lane_off
    k = len(off) - 1
    pairs = []
    if k >= 2:
        pairs.append((off[1] - 1, off[1]))
    last0 = off[k - 1]
    pairs.append((last0 + (off[k] - last0) // 3, last0 + 2 * (off[k] - last0) // 3))
    return pairs


def workload_weight(name, seed=0):
    """The unplanted head weight of a named workload (workloads with the same
    H, V, sigma and seed share it)."""
    _, H, V, _, sw, _ = WORKLOADS[name]
    return draw_weight(H, V, sw, seed)


def make_workload(name, seed=0, B=None, w=None):
    """Inputs of a named workload.

    Returns a dict: x (uint16 [B,H]), w (uint16 [H,V]), lane_off (list of
    k+1 ints), name, B, H, V, k, planted (list of (row, a, b) near-tie or tie
    plants).  ``B`` overrides the row count (the large-vocab sweep runs
    B in {1, 8, 16}).  ``w`` may pass the unplanted weight from
    ``workload_weight`` to skip drawing it again; it is never modified
    (workloads that plant ties work on a copy).
    """
    if name not in WORKLOADS:
        raise KeyError(name)
    B0, H, V, k, sw, rms = WORKLOADS[name]
    B = B0 if B is None else int(B)
    x = draw_hidden(B, H, seed, rms_norm=rms)
    if w is None:
        w = draw_weight(H, V, sw, seed)
    else:
        if w.shape != (H, V) or w.dtype != np.uint16:
            raise ValueError("weight does not match the workload")
        w = w.copy() if (name in ("tiny", "large_vocab")) else w
    lane_off = equal_lanes(V, k)
    planted = []
    if name == "tiny":
        plant_equal_columns(x, w, TINY_TIE_ROW, TINY_TIE_COLS, 4.0)
        planted.append((TINY_TIE_ROW,) + TINY_TIE_COLS)
    elif name == "large_vocab":
        pairs = near_tie_cols(lane_off)
        for j, r in enumerate(near_tie_rows(B)):
            a, b = pairs[j % len(pairs)]
            plant_near_tie(x, w, r, a, b)
            planted.append((r, a, b))
    return dict(name=name, x=x, w=w, lane_off=lane_off, B=B, H=H, V=V, k=k,
                planted=planted, ldw=WORKLOAD_LDW.get(name, V))


def make_random(B, H, V, lane_off, seed=0, sigma_x=1.0, sigma_w=0.02):
    """Plain random head of any shape (parity tests with ragged sizes)."""
    x = draw_hidden(B, H, seed, sigma=sigma_x)
    w = draw_weight(H, V, sigma_w, seed)
    return dict(name="random", x=x, w=w, lane_off=list(lane_off), B=B, H=H,
                V=V, k=len(lane_off) - 1, planted=[])


# --------------------------------------------------------------------------
# Partial-completion workloads (the row-parallel MLP down projection of the
# pages' Qwen3-14B layer: 17408 intermediate columns in two lanes of 8704,
# hidden size 5120; SemBridge section 6.4).  Lane i's activation shard is
# drawn from rng [seed, 2, i] and its weight rows from rng [seed, 3, i, c].
# --------------------------------------------------------------------------

PARTIAL_WORKLOADS = {
    # name: (B, N, K per lane, sigma_w)
    "mlp_down": (16, 5120, (8704, 8704), 0.02),
}


def draw_partial(B, N, Ks, seed=0, sigma_x=1.0, sigma_w=0.02):
    """Activation shards xs[i] (uint16 [B, K_i]) and weight blocks ws[i]
    (uint16 [K_i, N]) of a partial-completion boundary."""
    xs, ws = [], []
    for i, K in enumerate(Ks):
        rx = np.random.default_rng([seed, 2, i])
        xs.append(f32_to_bf16_bits(rx.standard_normal((B, K), dtype=np.float32) * sigma_x))
        rows = []
        for c in range(0, K, 256):
            rw = np.random.default_rng([seed, 3, i, c // 256])
            rows.append(f32_to_bf16_bits(
                rw.standard_normal((min(256, K - c), N), dtype=np.float32) * sigma_w))
        ws.append(np.concatenate(rows, axis=0))
    return xs, ws


def make_partial(name, seed=0, B=None):
    """Inputs of a named partial-completion workload: dict(xs, ws, B, N, Ks)."""
    B0, N, Ks, sw = PARTIAL_WORKLOADS[name]
    B = B0 if B is None else int(B)
    xs, ws = draw_partial(B, N, Ks, seed, sigma_w=sw)
    return dict(name=name, xs=xs, ws=ws, B=B, N=N, Ks=list(Ks))
