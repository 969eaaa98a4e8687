"""Property test of the head descriptor's validation (CPU, host only).

Random descriptors -- shapes, lane offsets, strides and pointers, valid and
not -- go to sb_workspace_bytes, which validates and enqueues nothing (the
pointers are fake, so no compute call is ever made with them).  The rules of
include/sb.h, written out here from the header's text, decide the outcome:

  * a descriptor that breaks none of them is accepted (SB_OK);
  * one that breaks some is refused with the status of one of the broken
    rules (the header does not order the checks, so any of them will do).

The ranges keep every launch far below the grid limits, whose own boundary
tests are in tests/test_abi_cpu.py.
"""
import ctypes

from hypothesis import given, settings, strategies as st

from logit_source_projection_amd import sb

FAKE = 1 << 20
LIM = 1 << 32


def expected_failures(B, H, V, k, off, x_ptr, ldx, w_ptrs, ldw):
    """The statuses of the rules the descriptor breaks (empty: valid)."""
    bad = set()
    if B < 0 or H < 0 or V < 1:
        bad.add(sb.SB_ERR_SHAPE)
    if k < 1 or k > 64:
        bad.add(sb.SB_ERR_LANES)
        return bad  # the offsets of an invalid lane count are not read
    if off[0] != 0 or off[k] != V or any(off[i + 1] <= off[i] for i in range(k)):
        bad.add(sb.SB_ERR_LANES)
    maxw = max(off[i + 1] - off[i] for i in range(k))
    if ldx < H or ldw < maxw:
        bad.add(sb.SB_ERR_SHAPE)
    if B > 0 and H > 0:
        if x_ptr == 0 or any(p == 0 for p in w_ptrs):
            bad.add(sb.SB_ERR_NULL)
        if x_ptr % 16 or ldx % 8 or ldw % 8 or any(p % 16 for p in w_ptrs):
            bad.add(sb.SB_ERR_ALIGN)
    if V > (1 << 30):
        bad.add(sb.SB_ERR_UNSUPPORTED)
    # the 32-bit per-step offsets: 40 shard rows and 64 rows of x; from 65
    # to 128 rows 128 rows of x; from 129 rows 72 shard rows and 256 rows of x
    if 40 * ldw * 2 >= LIM or 64 * ldx * 2 >= LIM:
        bad.add(sb.SB_ERR_UNSUPPORTED)
    if 65 <= B <= 128 and 128 * ldx * 2 >= LIM:
        bad.add(sb.SB_ERR_UNSUPPORTED)
    if B >= 129 and (72 * ldw * 2 >= LIM or 256 * ldx * 2 >= LIM):
        bad.add(sb.SB_ERR_UNSUPPORTED)
    return bad


def up8(n):
    return (n + 7) // 8 * 8


# Strides just below and at the 4 GiB boundaries of the per-step offsets
# (all multiples of 8): 256, 128 and 64 rows of x; 72 and 40 shard rows.
X_STRIDES = [(1 << 23) - 8, 1 << 23, (1 << 24) - 8, 1 << 24, (1 << 25) - 8, 1 << 25]
W_STRIDES = [29826160, 29826168, 53687088, 53687096]
BREAKS = ["B<0", "H<0", "V", "k=0", "k=65", "off0", "dup", "ldx<H", "ldw<w", "x=0", "w=0",
          "x%16", "w%16", "ldx%8", "ldw%8"]


@st.composite
def descriptors(draw):
    """A valid descriptor (strides often at a 4 GiB boundary), then half of
    the time one broken rule."""
    B = draw(st.one_of(st.sampled_from([0, 1, 16, 64, 65, 100, 128, 129, 2048, 65535, 70000]),
                       st.integers(0, 70000)))
    H = draw(st.one_of(st.integers(0, 6000), st.sampled_from([0, 1, 8, 5120])))
    k = draw(st.one_of(st.integers(1, 8), st.sampled_from([63, 64])))
    widths = draw(st.lists(st.one_of(st.integers(1, 5000), st.sampled_from([1, 8, 37])),
                           min_size=k, max_size=k))
    off = [0]
    for wdt in widths:
        off.append(off[-1] + wdt)
    V = off[-1]
    maxw = max(widths)
    ldx = draw(st.one_of(st.builds(lambda d: up8(H) + 8 * d, st.integers(0, 2)),
                         st.sampled_from(X_STRIDES)))
    ldw = draw(st.one_of(st.builds(lambda d: up8(maxw) + 8 * d, st.integers(0, 2)),
                         st.sampled_from(W_STRIDES)))
    x_ptr = FAKE
    w_ptrs = [FAKE + 16 * i for i in range(k)]
    brk = draw(st.one_of(st.just("none"), st.sampled_from(BREAKS)))
    if brk == "B<0":
        B = draw(st.integers(-3, -1))
    elif brk == "H<0":
        H = -1
    elif brk == "V":
        V += draw(st.sampled_from([1, -1]))
    elif brk == "k=0":
        k = 0
    elif brk == "k=65":
        k = 65
    elif brk == "off0":
        off[0] = draw(st.sampled_from([1, -8]))
    elif brk == "dup" and k > 1:
        i = draw(st.integers(1, k - 1))
        off[i] = off[i - 1]
    elif brk == "ldx<H" and H > 0:
        ldx = H - 1
    elif brk == "ldw<w":
        ldw = maxw - 1
    elif brk == "x=0":
        x_ptr = 0
    elif brk == "w=0":
        w_ptrs[draw(st.integers(0, len(w_ptrs) - 1))] = 0
    elif brk == "x%16":
        x_ptr = FAKE + draw(st.sampled_from([2, 8]))
    elif brk == "w%16":
        w_ptrs[draw(st.integers(0, len(w_ptrs) - 1))] += 8
    elif brk == "ldx%8":
        ldx += 4
    elif brk == "ldw%8":
        ldw += 2
    off = off + [0] * max(0, k + 1 - len(off))  # room for k + 1 offsets when k grew
    w_ptrs = w_ptrs + [FAKE] * max(0, k - len(w_ptrs))
    return B, H, V, k, off, x_ptr, ldx, w_ptrs, ldw


@settings(max_examples=600, deadline=None)
@given(descriptors())
def test_validation_matches_the_header(d):
    B, H, V, k, off, x_ptr, ldx, w_ptrs, ldw = d
    n_off = max(len(off), 1)
    c_off = (ctypes.c_int32 * n_off)(*off)
    c_w = (ctypes.c_void_p * max(len(w_ptrs), 1))(*w_ptrs)
    desc = sb.sb_head_desc(B=B, H=H, V=V, k=k, lane_off=c_off, x=x_ptr, ldx=ldx,
                           w=c_w, ldw=ldw)
    status = ctypes.c_int(123)
    size = sb.lib().sb_workspace_bytes(ctypes.byref(desc), sb.SB_SURF_TOKENS,
                                       ctypes.byref(status))
    bad = expected_failures(B, H, V, k, off, x_ptr, ldx, w_ptrs, ldw)
    if not bad:
        assert status.value == sb.SB_OK, (status.value, d)
        assert (size == 0) == (B == 0)
    else:
        assert status.value in bad, (status.value, bad, d)
        assert size == 0
