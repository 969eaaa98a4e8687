"""Plain CPU oracle for source projection of a vocab-sharded output head.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``logit_source_projection_amd``) and imports nothing from
it; the product path never calls it.

Sources (SemBridge: Compiling Consumer Observations into Cross-Stack
Communication Plans):

* section 5.2 (Data, Result, and Control Paths): the output head produces
  the logits; the full-logit plan cuts them into per-lane shards, moves the
  shards and rebuilds the whole tensor at the destination, whereas the
  token-only plan runs the deterministic sampler on the same logits at the
  source and moves int32 token IDs only;
* section 5.3 / section 6 (Plan Realization, Evaluation): under source
  projection each lane runs the argmax before the transfer, so a lane
  contributes one int32 result per row;
* section 3.1 (Boundary Contract): a projection operator must declare how it
  breaks ties, deterministically; section 3.2 (Consumer Observation): a
  log-probability consumer needs the complete logits as well as the IDs;
* Figure 1 caption: both plans hand the consumer the same token ID.

Readings taken where the pages are silent:

* the deterministic sampler is greedy argmax over the raw logits, and ties go
  to the lowest global vocabulary index;
* log-probabilities are log-softmax of the raw logits (no temperature, bias or
  soft-cap); the selected-token log-probability belongs to the argmax token;
* the argmax is decided on the fp64 logits themselves (the plain definition);
* non-finite logits follow numpy's argmax: a NaN ranks above every number
  (the first NaN wins), +inf above every finite value, so every row has an
  ID among its columns; the log-prob values of a row holding a NaN or +inf
  are not defined by the pages (NaN falls out of the formulas here);
* a row is a "near tie" when its fp64 top-2 gap (largest logit minus the
  next largest, over distinct indices) is below 2e-3 * max_v |z|.

Parity pins: every function here is pinned in ``tests/test_oracle_*.py`` by
exact-rational brute force, closed forms, invariants and planted mistakes --
top2_gap and the near-tie flag included (exact gaps on every row of the
tiny heads, rows planted just above, at and just below the threshold).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

NEAR_TIE_REL = 2e-3


def _load():
    """Load liboracle.so, building it first only when it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_logits.restype = ctypes.c_int
    lib.oracle_logits.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def max_threads():
    """Threads the C oracle's parallel loop uses when nthreads is not given."""
    return _load().oracle_max_threads()


def bf16_bits_to_f64(bits):
    """Exact decode of bfloat16 bit patterns (uint16) to float64.

    A bf16 pattern is the top half of the float32 with the same value, so the
    decode is a shift into a uint32 followed by a float32 -> float64 widening,
    both exact.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def logits(x_bits, w_bits, rows=None, nthreads=0):
    """fp64 head logits z = X . W (SemBridge section 5.2: the tail output head
    materialises the full logits before either result plan).

    x_bits : uint16 [B, H] bf16 bit patterns of the hidden rows
    w_bits : uint16 [H, V] bf16 bit patterns of the head weight (all k lanes
             side by side: lane i is columns [off_i, off_{i+1}))
    rows   : optional list of row indices of X to evaluate (sampled checks)
    Returns float64 [len(rows) or B, V]; each entry is summed in ascending h.
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[0]:
        raise ValueError("oracle.logits: need x [B,H] and w [H,V]")
    B, H = x.shape
    V = w.shape[1]
    if rows is None:
        sel = None
        n = B
    else:
        sel = np.ascontiguousarray(rows, dtype=np.int32)
        if sel.ndim != 1 or (sel.size and (sel.min() < 0 or sel.max() >= B)):
            raise ValueError("oracle.logits: row index out of range")
        n = sel.size
    z = np.empty((n, V), dtype=np.float64)
    rc = _load().oracle_logits(
        x.ctypes.data, H, None if sel is None else sel.ctypes.data, n,
        w.ctypes.data, V, H, V, z.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_logits failed")
    return z


def check_lanes(lane_off, V):
    """Lanes are contiguous, non-empty vocab ranges covering [0, V)
    (SemBridge section 5.2: the logits are sliced by TP lane)."""
    off = [int(o) for o in lane_off]
    if len(off) < 2 or off[0] != 0 or off[-1] != V:
        raise ValueError("lane offsets must start at 0 and end at V")
    if any(b <= a for a, b in zip(off[:-1], off[1:])):
        raise ValueError("lane offsets must be strictly increasing")
    return off


def lane_pairs(z, lane_off):
    """Per-lane projection on every row (SemBridge section 6 / Figure 1:
    argmax runs once per lane, "argmax x k", and each lane yields one result).

    For lane i = [off_i, off_{i+1}) and each row b, all in fp64:
      M_i[b]  = max over the lane
      A_i[b]  = smallest global index in the lane attaining M_i[b]
      S_i[b]  = sum over the lane of exp(z - M_i)
    Returns arrays of shape [B, k]: M, A, S.
    """
    B, V = z.shape
    off = check_lanes(lane_off, V)
    k = len(off) - 1
    M = np.empty((B, k), dtype=np.float64)
    A = np.empty((B, k), dtype=np.int64)
    S = np.empty((B, k), dtype=np.float64)
    for i in range(k):
        seg = z[:, off[i]:off[i + 1]]
        # np.argmax returns the first occurrence of the maximum: lowest index.
        a = np.argmax(seg, axis=1)
        A[:, i] = off[i] + a
        M[:, i] = seg[np.arange(B), a]
        S[:, i] = np.exp(seg - M[:, i:i + 1]).sum(axis=1)
    return M, A, S


def combine(M, A, S):
    """Fold the per-lane results in ascending lane order (one int32 result per
    lane is what source projection ships, SemBridge section 6).

      id  = A_j for the first lane j whose M_j is the largest, m = M_j
      lse = m + log(sum_i S_i * exp(M_i - m))
    "Largest" is np.argmax's order, the same as the per-lane argmax: a NaN
    ranks above every number (the first NaN wins), so the fold picks the lane
    of the row's first NaN when there is one; with finite values it is the
    first lane attaining max_i M_i.
    Returns (ids int64 [B], lse float64 [B]).
    """
    B, k = M.shape
    rows = np.arange(B)
    j = np.argmax(M, axis=1)  # first lane holding the largest result
    m = M[rows, j]
    ids = A[rows, j]
    lse = m + np.log((S * np.exp(M - m[:, None])).sum(axis=1))
    return ids, lse


def full_logit_argmax(z, lane_off):
    """The full-logit plan inside the oracle (SemBridge section 5.2): the lane
    shards are reconstructed into the complete [B, V] tensor (the
    destination-local AllGather) and a plain first-occurrence argmax runs on
    it."""
    off = check_lanes(lane_off, z.shape[1])
    shards = [z[:, off[i]:off[i + 1]] for i in range(len(off) - 1)]
    full = np.concatenate(shards, axis=1)
    return np.argmax(full, axis=1).astype(np.int64)


def top2_gap(z):
    """Per row, the largest logit minus the second largest, where the two are
    taken at distinct indices: z_(1) - z_(2) >= 0, and 0 for an exact tie.
    np.partition with kth = V - 2 leaves the two largest entries of the row in
    its last two slots, the larger last.  +inf for a one-column row."""
    if z.shape[1] < 2:
        return np.full(z.shape[0], np.inf)
    top = np.partition(z, -2, axis=1)[:, -2:]
    return top[:, 1] - top[:, 0]


def near_tie(z, gap):
    """Rows whose top-2 gap lies strictly below NEAR_TIE_REL * max_v |z|: their
    IDs may differ between fp32 and fp64 logits, so they are reported rather
    than compared."""
    return gap < NEAR_TIE_REL * np.abs(z).max(axis=1)


def project(z, lane_off):
    """Token and log-probability surfaces from fp64 logits z [B, V].

    Returns a dict with
      ids       int64 [B]  argmax token IDs over the fp64 logits, lowest index
                           on ties
      lse       float64 [B] logsumexp of each row
      sel_lp    float64 [B] log-probability of the argmax token
      lane_max, lane_arg, lane_sumexp   per-lane results, [B, k]
      gap       float64 [B] fp64 top-2 gap
      near_tie  bool [B]   gap < 2e-3 * max_v |z|
    and checks the pages' invariant that the full-logit plan yields the same
    IDs as per-lane projection (Figure 1 caption; section 6.3).
    """
    M, A, S = lane_pairs(z, lane_off)
    ids, lse = combine(M, A, S)
    r0 = full_logit_argmax(z, lane_off)
    if not np.array_equal(ids, r0):
        raise AssertionError("oracle: per-lane projection differs from the full-logit argmax")
    sel = z[np.arange(z.shape[0]), ids]
    gap = top2_gap(z)
    return dict(ids=ids, lse=lse, sel_lp=sel - lse,
                lane_max=M, lane_arg=A, lane_sumexp=S,
                gap=gap, near_tie=near_tie(z, gap))


def logprobs(z, lse):
    """Complete log-probabilities lp[b, v] = z[b, v] - lse[b] (the
    log-probability surface keeps the complete logits, SemBridge section 3.2
    and 3.4)."""
    return z - np.asarray(lse, dtype=np.float64)[:, None]
