"""Grouped (mixture-of-experts) SALR linear oracle.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module; the product path never
imports, calls or links it.

Sources, cited by page title and section:
  [summary]  gist.science technical summary of "Sparsity-Aware Low-Rank
             Representation for Efficient Fine-Tuning of Large Language
             Models", Experimental Results (SALR is evaluated on the
             mixture-of-experts models Mixtral-8x7B and DeepSeek-V2-Lite)
             and Methodology 1-4 (what one SALR layer computes).

What is computed: E experts, each its own SALR layer (own bitmap, values,
A_cat, B_cat) of one shape N x K.  The tokens routed to expert e are the
contiguous rows [off[e], off[e+1]) of X (the caller groups the rows by
expert), and their outputs are the same rows of Y:
    Y[off[e]:off[e+1]] = X[off[e]:off[e+1]] W_s,e^T
                         + (X[off[e]:off[e+1]] A_cat,e) B_cat,e
in float64 with no intermediate rounding.

Readings (listed in the design doc): the pages name the MoE models but say
nothing of how their expert layers are launched; applying SALR to every
expert's linear layer, each with its own encoding, is the plain reading of
SALR applied to those models.  Routing (which expert takes a token, and the
weighted combination of expert outputs) is not part of the SALR layer: the
grouped layer takes the rows already grouped and returns the rows in the
same order.
"""

from __future__ import annotations

import numpy as np

from . import salr


def check_offsets(offsets, E: int, T: int) -> np.ndarray:
    """Expert row boundaries: int [E + 1], off[0] = 0, nondecreasing,
    off[E] = T."""
    off = np.asarray(offsets, dtype=np.int64)
    if off.shape != (E + 1,) or off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("expert offsets must run from 0 to T without decreasing")
    return off


def grouped_forward(X_bits, offsets, experts, K: int) -> np.ndarray:
    """Y [T x N] float64 for bf16 X [T x K] whose rows [off[e], off[e+1])
    go to expert e; experts[e] = (masks, values, A_cat_bits [K x r],
    B_cat_bits [r x N])."""
    X_bits = np.asarray(X_bits, dtype=np.uint16)
    T = X_bits.shape[0]
    off = check_offsets(offsets, len(experts), T)
    N = np.asarray(experts[0][0]).shape[0]
    Y = np.zeros((T, N), dtype=np.float64)
    for e, (masks, values, A, B) in enumerate(experts):
        s, t = int(off[e]), int(off[e + 1])
        if t > s:
            Y[s:t] = salr.forward(X_bits[s:t], masks, values, K, A, B)
    return Y


def grouped_forward_rows(X_bits, offsets, experts, K: int, rows) -> np.ndarray:
    """The same for the output columns `rows` only: Y[:, rows]."""
    X_bits = np.asarray(X_bits, dtype=np.uint16)
    T = X_bits.shape[0]
    off = check_offsets(offsets, len(experts), T)
    rows = np.asarray(rows)
    Y = np.zeros((T, rows.size), dtype=np.float64)
    for e, (masks, values, A, B) in enumerate(experts):
        s, t = int(off[e]), int(off[e + 1])
        if t > s:
            Y[s:t] = salr.forward_rows(X_bits[s:t], masks, values, K, A, B, rows)
    return Y
