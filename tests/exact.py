"""Exact-rational brute force for tiny heads (test helper, pins the oracle).

bf16 values are dyadic rationals, so the logits of a tiny head can be computed
exactly with ``fractions.Fraction`` and exact ties are visible as equality.
This decodes bf16 from the sign / exponent / mantissa fields, independently of
the oracle's bit-shift decode.
"""
from fractions import Fraction


def bf16_to_fraction(bits):
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("inf/nan in exact brute force")
    if e == 0:
        mag = Fraction(m, 128) * Fraction(2) ** (-126)
    else:
        mag = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return sign * mag


def exact_logits(x_bits, w_bits):
    """z[b][v] as Fractions, from the definition sum_h x[b][h] * w[h][v]."""
    B, H = x_bits.shape
    V = w_bits.shape[1]
    xf = [[bf16_to_fraction(x_bits[b, h]) for h in range(H)] for b in range(B)]
    wf = [[bf16_to_fraction(w_bits[h, v]) for v in range(V)] for h in range(H)]
    z = []
    for b in range(B):
        row = []
        for v in range(V):
            s = Fraction(0)
            for h in range(H):
                if xf[b][h] and wf[h][v]:
                    s += xf[b][h] * wf[h][v]
            row.append(s)
        z.append(row)
    return z


def exact_argmax(row):
    """Lowest index attaining the exact maximum."""
    best = max(row)
    return row.index(best)
