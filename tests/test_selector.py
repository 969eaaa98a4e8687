"""Pins of the plan selector (SemBridge paper, section 8.2, Equation 7; payload
accounting of the Figure 1 caption and Figure 2)."""
import json
import math
import os
import random

import pytest

from logit_source_projection_amd import selector

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "pages_result_traffic.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_payload_accounting_follows_figure_1():
    # R0: V logits per row in k frames; P0: k IDs per row in k frames;
    # S1: one ID per row in one frame
    assert selector.plan_payload("R0", 16, 151936, 4) == (4 * 16 * 151936, 4)
    assert selector.plan_payload("P0", 16, 151936, 4) == (4 * 4 * 16, 4)
    assert selector.plan_payload("S1", 16, 151936, 4) == (4 * 16, 1)
    with pytest.raises(ValueError):
        selector.plan_payload("X9", 1, 1, 1)


# Per-frame header bytes implied by Figure 2: the totals printed there exceed
# the payloads of four rows by exactly 130 B per logit-shard frame and 48 B
# per token frame.
LOGIT_HDR, TOKEN_HDR = 130, 48


def test_payload_is_within_the_frame_totals_printed_in_figure_2():
    # Figure 2 (MiniMax-M2.7, V = 200064, four lanes): four logit-shard
    # frames for R0 and four token frames for P0 per step.  The rows per step
    # are not printed; reading them as four, the payloads are 3,201,024 B and
    # 64 B and the rest is the per-frame header.
    f = golden()["figure_2"]
    V, k = f["vocab"], f["lanes"]
    r0, fr = selector.plan_payload("R0", 4, V, k)
    p0, fp = selector.plan_payload("P0", 4, V, k)
    assert (fr, fp) == (f["R0"]["frames"], f["P0"]["frames"])
    assert r0 == 3201024 and f["R0"]["bytes"] - r0 == fr * LOGIT_HDR
    assert p0 == 64 and f["P0"]["bytes"] - p0 == fp * TOKEN_HDR


def test_payload_matches_the_live_switching_run_of_section_6_3():
    # The live surface-switching run prints frames and bytes per plan but not
    # the rows.  With the Figure 2 header sizes, all three totals leave
    # payloads of exactly 17 rows on the same head: R0 17 x V x 4 B, P0
    # 17 x k int32 IDs, S1 17 int32 IDs (one owner).
    f = golden()["live_switch"]
    V, k, rows = f["vocab"], f["lanes"], 17
    for plan, hdr in (("R0", LOGIT_HDR), ("P0", TOKEN_HDR), ("S1", TOKEN_HDR)):
        payload, _ = selector.plan_payload(plan, rows, V, k)
        assert f[plan]["bytes"] == payload + f[plan]["frames"] * hdr, plan


def test_equation_7_by_hand():
    # saves 1e6 B and 2 frames, costs 1 ms more locally
    args = dict(L_s=2e-3, L_r=1e-3, B_s=0, B_r=1_000_000, F_s=1, F_r=3)
    # 1 GB/s, no startup: 1 ms saved == 1 ms spent -> not strictly better
    assert not selector.improves(alpha=0.0, beta=1e9, **args)
    assert selector.improves(alpha=0.0, beta=0.9e9, **args)
    assert not selector.improves(alpha=0.0, beta=1.1e9, **args)
    # 0.25 ms startup per frame saves 0.5 ms: wins up to 2 GB/s
    assert selector.improves(alpha=0.25e-3, beta=1.9e9, **args)
    assert not selector.improves(alpha=0.25e-3, beta=2.1e9, **args)
    # 0.5 ms per frame covers the whole local cost: wins at any rate
    assert selector.improves(alpha=0.5001e-3, beta=1e15, **args)
    with pytest.raises(ValueError):
        selector.improves(alpha=0.0, beta=0.0, **args)


def test_beta_max_is_the_break_even_rate():
    rng = random.Random(7)
    for _ in range(200):
        L_r = rng.uniform(0, 1e-3)
        L_s = L_r + rng.uniform(1e-6, 1e-3)
        B_s, B_r = rng.randint(0, 1000), rng.randint(10**4, 10**8)
        F_s, F_r = rng.randint(1, 4), rng.randint(4, 40)
        alpha = rng.uniform(0, (L_s - L_r) / (F_r - F_s) * 0.99) if F_r > F_s else 0.0
        bm = selector.beta_max(L_s, L_r, B_s, B_r, F_s, F_r, alpha)
        assert math.isfinite(bm) and bm > 0
        a = dict(L_s=L_s, L_r=L_r, B_s=B_s, B_r=B_r, F_s=F_s, F_r=F_r, alpha=alpha)
        assert selector.improves(beta=bm * (1 - 1e-9), **a)
        assert not selector.improves(beta=bm * (1 + 1e-9), **a)


def test_region_when_the_specialised_plan_is_also_cheaper_locally():
    reg = selector.region(L_s=1e-3, L_r=1.2e-3, B_s=64, B_r=10**7, F_s=4, F_r=4)
    assert reg["always"] and math.isinf(reg["beta_max_at_alpha0"])
    assert reg["alpha_any_beta"] == 0.0
    for beta in (1e6, 1e9, 1e12, 1e18):
        assert selector.improves(1e-3, 1.2e-3, 64, 10**7, 4, 4, 0.0, beta)
    rep = selector.report(0.2429, 0.261, 16, 151936, 4)
    assert rep["p0_wins_on_every_link"] and rep["beta_max_GBps_at_alpha0"] is None


def test_region_when_projection_costs_more_locally():
    # P0 slower by 10 us, saves 4*16*151936 - 4*4*16 = 9,723,648 B at B=16,
    # V=151936, k=4, and no frames
    rep = selector.report(0.251, 0.241, 16, 151936, 4)
    assert not rep["p0_wins_on_every_link"]
    assert rep["beta_max_GBps_at_alpha0"] == pytest.approx(9723648 / 10e-6 / 1e9)
    assert math.isinf(rep["alpha_any_beta_s"])  # equal frame counts
