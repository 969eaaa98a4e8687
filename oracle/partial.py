"""Oracle of the partial-completion workload.  TEST INFRASTRUCTURE ONLY: only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the GPU library.

What it computes (SemBridge paper, "SemBridge: Compiling Consumer Observations
into Cross-Stack Communication Plans"):

* section 6.4 (Exact Shards and Partial Completion): in the MLP down
  projection each lane multiplies its own slice of the intermediate
  activations by its own rows of the weight, so every lane ends up with a
  full-width but incomplete result P_i = X_i . W_i that is not an observable
  value on its own;
* section 3.6 (Contract Construction and Static Validation): the contract
  carries an elementwise operator (sum, product, minimum or maximum in the
  paper's reference) that the plan must apply to all the partials before
  any consumer sees the output.

Reading taken where the pages are silent: the k partials are folded in
ascending lane order, out = op(...op(op(P_0, P_1), P_2)..., P_{k-1}).  Every
operator is exact up to rounding order, so in fp64 the order only moves the
last bits.

Parity pins: ``tests/test_oracle_partial.py`` checks every operator against
exact-rational brute force, closed forms and invariants; nothing here is
"parity unpinned".
"""
import numpy as np

from . import logits as _products

OPS = ("sum", "prod", "min", "max")


def partials(x_list, w_list):
    """fp64 partials P_i = X_i . W_i, one per lane (section 6.4).

    x_list[i] : uint16 [B, K_i] bf16 bits of lane i's activation shard
    w_list[i] : uint16 [K_i, N] bf16 bits of lane i's weight rows
    Returns float64 [k, B, N]; each entry summed in ascending reduction index.
    """
    if len(x_list) != len(w_list) or not x_list:
        raise ValueError("need one activation shard and one weight block per lane")
    N = w_list[0].shape[1]
    out = []
    for x, w in zip(x_list, w_list):
        if w.shape[1] != N:
            raise ValueError("all lanes produce partials of the same width")
        # a partial is the same bf16 x bf16 product sum as a logit row
        out.append(_products(x, w))
    return np.stack(out)


def complete(P, op):
    """Complete the registered reduction over the lanes of P [k, B, N]
    (section 3.6), folding in ascending lane order."""
    if op not in OPS:
        raise ValueError(f"unknown reduction {op!r}")
    acc = P[0].copy()
    for i in range(1, P.shape[0]):
        if op == "sum":
            acc = acc + P[i]
        elif op == "prod":
            acc = acc * P[i]
        elif op == "min":
            acc = np.minimum(acc, P[i])
        else:
            acc = np.maximum(acc, P[i])
    return acc


def partial_complete(x_list, w_list, op):
    """The complete observation: the registered reduction of the partials."""
    return complete(partials(x_list, w_list), op)
