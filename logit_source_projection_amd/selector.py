"""Fabric-aware plan selection between legal result plans.

Follows the selection criterion of the SemBridge paper ("SemBridge: Compiling
Consumer Observations into Cross-Stack Communication Plans", section 8.2,
Equation 7).  A plan i moves B_i cross-domain payload bytes in F_i frames and
spends L_i seconds of non-overlapped projection and local-collective work.
Over a link with effective payload rate beta (bytes/s) and effective
per-frame startup alpha (s), a specialised plan s improves on a reference
plan r exactly when

    (B_r - B_s) / beta + alpha * (F_r - F_s)  >  L_s - L_r.

Payload and frame counts follow the Figure 1 caption: the full-logit plan R0
moves the V logits of every row in k frames (one per lane), source projection
P0 moves k int32 IDs per row in k frames, and owner-token delivery S1 moves
one int32 ID per row in one frame (its local broadcast counts as local work).
Logits travel as fp32 (the pages do not state the dtype; fp32 is the logit
precision of this library).

Pure host arithmetic: no device code, no measurement of its own.  The local
costs come from timed calls of the two plans on the same input.
"""
import math

LOGIT_BYTES = 4  # fp32 logit element
ID_BYTES = 4     # int32 token ID


def plan_payload(plan, B, V, k):
    """(payload bytes, frames) a plan sends across the boundary per step."""
    if plan == "R0":
        return LOGIT_BYTES * B * V, k
    if plan == "P0":
        return ID_BYTES * k * B, k
    if plan == "S1":
        return ID_BYTES * B, 1
    raise ValueError(f"unknown plan {plan!r}")


def improves(L_s, L_r, B_s, B_r, F_s, F_r, alpha, beta):
    """Equation 7: does plan s beat plan r on a link (alpha s/frame, beta B/s)?"""
    if beta <= 0:
        raise ValueError("beta must be positive")
    return (B_r - B_s) / beta + alpha * (F_r - F_s) > L_s - L_r


def region(L_s, L_r, B_s, B_r, F_s, F_r):
    """The links on which plan s beats plan r, as a dict.

    dL = L_s - L_r is the extra local cost of s, dB = B_r - B_s and
    dF = F_r - F_s the payload and frames it saves.  With dB > 0, s wins on
    every link whose rate is below ``beta_max(alpha)`` = dB / (dL - alpha*dF)
    (infinite once alpha*dF >= dL: then s wins at any rate).  ``always`` is
    True when s wins for every alpha >= 0 and beta > 0.
    """
    dL, dB, dF = L_s - L_r, B_r - B_s, F_r - F_s
    out = dict(dL_s=dL, dB=dB, dF=dF)
    if dB < 0 or dF < 0:
        raise ValueError("region() expects plan s to save bytes and frames")
    # at alpha = 0 the condition is dB / beta > dL
    out["always"] = dL < 0 or (dL == 0 and dB > 0)
    out["beta_max_at_alpha0"] = math.inf if out["always"] else (dB / dL if dB > 0 else 0.0)
    # per-frame startup above which s wins at any rate
    if dL <= 0:
        out["alpha_any_beta"] = 0.0
    else:
        out["alpha_any_beta"] = dL / dF if dF > 0 else math.inf
    return out


def beta_max(L_s, L_r, B_s, B_r, F_s, F_r, alpha):
    """Largest link rate (B/s) at which plan s still beats plan r, given the
    per-frame startup alpha; math.inf when s wins at every rate."""
    dL, dB, dF = L_s - L_r, B_r - B_s, F_r - F_s
    margin = dL - alpha * dF
    if margin < 0 or (margin == 0 and dB > 0):
        return math.inf
    return dB / margin if margin > 0 else 0.0


def report(ms_p0, ms_r0, B, V, k):
    """Selector summary for a measured P0 / R0 pair on one input (ms per call)."""
    B_p, F_p = plan_payload("P0", B, V, k)
    B_r, F_r = plan_payload("R0", B, V, k)
    reg = region(ms_p0 * 1e-3, ms_r0 * 1e-3, B_p, B_r, F_p, F_r)
    bm = reg["beta_max_at_alpha0"]
    return dict(
        criterion="(B_r - B_s)/beta + alpha (F_r - F_s) > L_s - L_r",
        L_p0_s=ms_p0 * 1e-3, L_r0_s=ms_r0 * 1e-3,
        bytes_p0=B_p, frames_p0=F_p, bytes_r0=B_r, frames_r0=F_r,
        p0_wins_on_every_link=reg["always"],
        beta_max_GBps_at_alpha0=None if math.isinf(bm) else bm / 1e9,
        alpha_any_beta_s=reg["alpha_any_beta"])
