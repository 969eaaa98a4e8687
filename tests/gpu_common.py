"""Shared helpers of the GPU parity tests: run every surface of libsb on one
input and compare with the oracle under the acceptance rules.

Acceptance (written here, used by every parity test):
  * logits: per row, max_v |g - z| <= LOGIT_REL * max_v |z|  (row-max relative)
  * lse:    |g - lse| <= LSE_REL * max(|lse|, 1)
  * ids:    equal to the oracle's fp64 argmax on every row whose top-2 gap
            is >= 2e-3 * max|z|; rows below that are near ties and are
            reported, not compared.  The exempt set itself is recomputed
            here from a full sort of each row and must equal the oracle's.
  * token-only, log-prob and full-logit IDs: bit-identical on every row.
"""
import numpy as np
import torch

import oracle
from logit_source_projection_amd import sb

LOGIT_REL = 2e-3
LSE_REL = 1e-4


def upload(d, device="cuda", lanes_separate=False, pad_w=0, pad_x=0, pad_bits=0x7FC0,
           lane_base_bytes=None):
    """Device tensors for a workload dict; optionally each lane in its own
    allocation and/or row padding filled with ``pad_bits`` (NaN by default)
    that the kernels must never use.  One weight allocation whose width is
    not a multiple of 8 is padded to the next multiple (the ABI's stride
    rule).  ``lane_base_bytes`` (with separate
    lanes) starts lane i's shard that many bytes (a multiple of 16) into its
    allocation, which the caching allocator aligns to at least 512 bytes."""
    x_bits, w_bits, off = d["x"], d["w"], d["lane_off"]
    B, H = x_bits.shape
    if pad_x:
        xp = np.full((B, H + pad_x), pad_bits, dtype=np.uint16)
        xp[:, :H] = x_bits
        x = sb.to_device_bf16(xp, device)[:, :H]
    else:
        x = sb.to_device_bf16(x_bits, device)
    if lanes_separate:
        widths = [off[i + 1] - off[i] for i in range(len(off) - 1)]
        ldw = ((max(widths) + 7) // 8) * 8 + pad_w
        shards = []
        for i, wi in enumerate(widths):
            s = np.full((H, ldw), pad_bits, dtype=np.uint16)
            s[:, :wi] = w_bits[:, off[i]:off[i + 1]]
            if lane_base_bytes is None:
                shards.append(sb.to_device_bf16(s, device)[:, :wi])
                continue
            e = lane_base_bytes[i] // 2
            assert lane_base_bytes[i] % 16 == 0
            flat = np.full(H * ldw + e + 64, pad_bits, dtype=np.uint16)
            flat[e:e + H * ldw] = s.ravel()
            t = sb.to_device_bf16(flat, device)[e:e + H * ldw].view(H, ldw)
            assert t.data_ptr() % 128 == lane_base_bytes[i] % 128
            shards.append(t[:, :wi])
        w = shards
    elif pad_w or w_bits.shape[1] % 8:
        # one allocation at a row stride of a multiple of 8 plus pad_w
        V = w_bits.shape[1]
        ldw = (V + 7) // 8 * 8 + pad_w
        wp = np.full((H, ldw), pad_bits, dtype=np.uint16)
        wp[:, :V] = w_bits
        w = sb.to_device_bf16(wp, device)[:, :V]
    else:
        w = sb.to_device_bf16(w_bits, device)
    return sb.Head(x, w, off)


def run_surfaces(head, device="cuda", full_logprobs=True):
    """Call all three surfaces; returns numpy results."""
    B, V = head.B, head.V
    ids_tok = torch.full((B,), -1, dtype=torch.int32, device=device)
    ids_lp = torch.full((B,), -1, dtype=torch.int32, device=device)
    ids_r0 = torch.full((B,), -1, dtype=torch.int32, device=device)
    lse = torch.full((B,), float("nan"), dtype=torch.float32, device=device)
    sel = torch.full((B,), float("nan"), dtype=torch.float32, device=device)
    ldv = (V + 3) // 4 * 4  # fp32 outputs need a row stride that is a multiple of 4
    lp = (torch.full((B, ldv), float("nan"), dtype=torch.float32, device=device)[:, :V]
          if full_logprobs else None)
    logits = torch.full((B, ldv), float("nan"), dtype=torch.float32, device=device)[:, :V]
    sb.sb_project_tokens(head, ids_tok)
    sb.sb_project_logprobs(head, ids_lp, lse, sel, lp)
    sb.sb_full_logits(head, logits, ids_r0)
    torch.cuda.synchronize()
    out = dict(ids_tok=ids_tok.cpu().numpy(), ids_lp=ids_lp.cpu().numpy(),
               ids_r0=ids_r0.cpu().numpy(), lse=lse.cpu().numpy(),
               sel_lp=sel.cpu().numpy(), logits=logits.cpu().numpy())
    out["logprobs"] = lp.cpu().numpy() if lp is not None else None
    return out


def check_internal(g):
    """GPU surfaces against each other (bitwise)."""
    assert np.array_equal(g["ids_tok"], g["ids_r0"]), "token-only vs full-logit IDs"
    assert np.array_equal(g["ids_lp"], g["ids_r0"]), "log-prob vs full-logit IDs"
    # the full-logit argmax is the lowest index of the row maximum
    lg = g["logits"]
    assert np.array_equal(g["ids_r0"], np.argmax(lg, axis=1)), "full-logit argmax"
    if g["logprobs"] is not None:
        # complete log-probs are the same logits minus the same lse, in fp32
        exp = (lg - g["lse"][:, None]).astype(np.float32)
        assert np.array_equal(g["logprobs"], exp), "complete log-probs vs logits - lse"
    rows = np.arange(lg.shape[0])
    assert np.array_equal(g["sel_lp"], (lg[rows, g["ids_r0"]] - g["lse"]).astype(np.float32))


def sorted_near_ties(z):
    """Near-tie rows recomputed without the oracle: each row sorted in full,
    gap = largest - second largest, flagged when below 2e-3 * max |z|."""
    srt = np.sort(z, axis=1)
    gap = srt[:, -1] - srt[:, -2] if z.shape[1] > 1 else np.full(z.shape[0], np.inf)
    scale = np.maximum(np.abs(srt[:, 0]), np.abs(srt[:, -1]))
    return gap < 2e-3 * scale, gap


def check_against_oracle(g, z, lane_off, rows=None, report=None):
    """Compare GPU results on `rows` (all rows if None) with oracle logits z
    (one row of z per entry of rows)."""
    rows = np.arange(z.shape[0]) if rows is None else np.asarray(rows)
    r = oracle.project(z, lane_off)
    near_sorted, gap_sorted = sorted_near_ties(z)
    assert np.array_equal(r["near_tie"], near_sorted), (
        f"exempt rows: oracle {rows[r['near_tie']]} vs sorted {rows[near_sorted]}")
    assert np.array_equal(r["gap"], gap_sorted), "top-2 gap differs from a full sort"
    lg = g["logits"][rows].astype(np.float64)
    scale = np.abs(z).max(axis=1)
    err = np.abs(lg - z).max(axis=1)
    bad = err > LOGIT_REL * scale
    assert not bad.any(), f"logit error rows {rows[bad]}: {err[bad]} vs scale {scale[bad]}"
    lse = g["lse"][rows].astype(np.float64)
    lerr = np.abs(lse - r["lse"])
    assert np.all(lerr <= LSE_REL * np.maximum(np.abs(r["lse"]), 1.0)), f"lse error {lerr.max()}"
    ids = g["ids_r0"][rows]
    near = r["near_tie"]
    mism = (ids != r["ids"]) & ~near
    assert not mism.any(), f"id mismatch on rows {rows[mism]}: {ids[mism]} vs {r['ids'][mism]}"
    sel = g["sel_lp"][rows].astype(np.float64)
    sel_ref = z[np.arange(len(rows)), ids] - r["lse"]
    serr = np.abs(sel - sel_ref)
    assert np.all(serr <= LOGIT_REL * scale + LSE_REL * np.maximum(np.abs(r["lse"]), 1.0))
    if g["logprobs"] is not None:
        lp = g["logprobs"][rows].astype(np.float64)
        lpo = oracle.logprobs(z, r["lse"])
        lperr = np.abs(lp - lpo).max(axis=1)
        assert np.all(lperr <= LOGIT_REL * scale + LSE_REL * np.maximum(np.abs(r["lse"]), 1.0))
    near_rows = [(int(rows[i]), float(r["gap"][i]), int(ids[i]), int(r["ids"][i]))
                 for i in np.nonzero(near)[0]]
    if report is not None:
        report.extend(near_rows)
    if near_rows:
        print("near-tie rows (row, fp64 gap, gpu id, oracle id):", near_rows, flush=True)
    return r
