"""Backward-pass oracle for fine-tuning the SALR adapters with the base
weight frozen.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module; the product path never
imports, calls or links it.

Sources, cited by page title and section:
  [summary]  gist.science technical summary of "Sparsity-Aware Low-Rank
             Representation for Efficient Fine-Tuning of Large Language
             Models", Methodology 2 ("Trainable Residual": the SVD-derived
             residual adapter is fine-tuned together with the LoRA adapters)
             and Methodology 1 (the static mask applies to the frozen base
             weight only); Experimental Results, Ablation Studies (freezing
             the SVD residual costs accuracy).

What is computed, for the layer Y = X W_s^T + (X A_cat) B_cat and an
upstream gradient dY = dL/dY (all float64, no intermediate rounding):
  dX     = dY W_s + (dY B_cat^T) A_cat^T        [M x K]
  dA_cat = X^T (dY B_cat^T)                     [K x r_cat]
  dB_cat = (X A_cat)^T dY                       [r_cat x N]
W_s (the bitmap and its values) is frozen: it has no gradient.

Readings (listed in the design doc): the gradient of the concatenated adapters is
taken as one block (its residual and LoRA column blocks are the per-adapter
gradients, by the concatenation identity); the frozen W_s is read through a
column-major copy of its encoding (the transposed layer below), built once.
"""

from __future__ import annotations

import numpy as np

from . import salr
from .bf16 import bits_to_f64

WORD = 64
OFFSET_GROUP = 1024


def transpose_encoding(masks, values, K: int):
    """The encoding of W_s^T [K x N] from that of W_s [N x K]: bitmap words
    along N, each row k holding column k's kept values in ascending row
    order, rows padded with +0.0 patterns to the largest column count.
    Returns (masks_T, values_T, offsets_T, n_keep_T)."""
    keep = salr.decode_keep(masks, K)          # [N x K] bool
    N = keep.shape[0]
    W = salr.decode_dense_bits(masks, values, K)  # [N x K] uint16 (0 where pruned)
    keep_T = keep.T
    counts = keep_T.sum(axis=1)
    n_keep_T = int(counts.max()) if counts.size else 0
    values_T = np.zeros((K, n_keep_T), dtype=np.uint16)
    WT = W.T
    for k in range(K):
        values_T[k, : counts[k]] = WT[k, keep_T[k]]
    masks_T = salr.pack_masks(keep_T)
    offsets_T = salr.block_offsets(keep_T)
    return masks_T, values_T, offsets_T, n_keep_T


def backward(X_bits, dY_bits, masks, values, K: int, A_cat_bits, B_cat_bits):
    """(dX, dA_cat, dB_cat) in float64 for bf16 inputs X [M x K],
    dY [M x N], A_cat [K x r_cat], B_cat [r_cat x N]."""
    X = bits_to_f64(X_bits)
    dY = bits_to_f64(dY_bits)
    Ws = salr.decode_dense(masks, values, K)
    A = bits_to_f64(A_cat_bits)
    B = bits_to_f64(B_cat_bits)
    G = dY @ B.T                       # dL/dT, T = X A_cat
    dX = dY @ Ws + G @ A.T
    dA = X.T @ G
    dB = (X @ A).T @ dY
    return dX, dA, dB
