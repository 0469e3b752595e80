"""SALR oracle: plain, slow, CPU-only definition of what the layer computes.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
imports nothing from the product package.

Sources, cited by page title and section:
  [abstract]  "Sparsity-Aware Low-Rank Representation for Efficient
              Fine-Tuning of Large Language Models", authors' abstract (as
              listed on the scholarfeed.org author page "Danning Ke" and on
              the arxiv.science author listing).
  [summary]   gist.science technical summary of paper 2601.16991 (an
              AI-written explainer of the same paper), sections
              "Methodology" 1-4.

Every floating-point step is float64 unless stated.  bf16 tensors enter and
leave as uint16 bit patterns.

Readings of points the pages leave open (each is listed in the design doc):
  * W is [N x K] = [out x in]; pruning is per output row, along K.
  * n_keep per row is an integer argument (K - floor(s*K) for sparsity s).
  * Magnitude = the 15 low bits of the bf16 pattern (|w|, +0 == -0).  Among
    equal magnitudes at the threshold the lower column index is kept, so the
    kept set is unique.
  * Bitmap: one uint64 per 64 columns, least significant bit = lowest
    column, padding bits beyond K are 0.  The bit marks a KEPT entry (a kept
    zero still sets its bit).
  * The "lookup table" read beside the bitmap is a per-row table of running
    kept counts at every 1024th column (offsets[n][g] = kept columns < 1024g).
  * The residual is the pruned part of the frozen weight, R = W - W_s.
  * Truncated SVD factors are split evenly: A' = V_r sqrt(S_r) [K x r],
    B' = sqrt(S_r) U_r^T [r x N], each rounded to bf16; sign fixed so that the
    largest-magnitude entry of each right singular vector is positive.
  * Concatenation: residual adapter first, then the LoRA adapters in the
    order given; no extra scaling.
  * Forward: Y = X W_s^T + (X A_cat) B_cat with no intermediate rounding.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .bf16 import bits_to_f64, f64_to_bits, is_nonfinite_bits

WORD = 64          # columns per bitmap word
OFFSET_GROUP = 1024  # columns per running-count table entry


class NonFiniteWeight(ValueError):
    """W holds an Inf or NaN (exponent field all ones)."""


# ---------------------------------------------------------------------------
# Encode.  [summary] Methodology 1 (static magnitude mask on the frozen base
# weight only), 2 (residual E = W - W_hat, rank-r truncated SVD), 3 (adapters
# stacked along the rank dimension), 4 (bitmap + compact value array).
# ---------------------------------------------------------------------------

def select_keep(W_bits: np.ndarray, n_keep: int) -> np.ndarray:
    """Static magnitude mask of the frozen weight ([summary] Methodology 1;
    [abstract]: prune the frozen base weights by magnitude).

    Returns bool [N x K]: per row, the n_keep entries of largest |w|, ties at
    equal magnitude broken toward the lower column.  A stable sort of the
    negated magnitudes orders each row by (|w| descending, column ascending);
    the first n_keep positions are kept.
    """
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    if not 0 <= n_keep <= K:
        raise ValueError("n_keep must lie in [0, K]")
    if is_nonfinite_bits(W_bits).any():
        raise NonFiniteWeight("W contains Inf or NaN")
    mag = (W_bits & np.uint16(0x7FFF)).astype(np.int32)
    order = np.argsort(-mag, axis=1, kind="stable")
    keep = np.zeros((N, K), dtype=bool)
    np.put_along_axis(keep, order[:, :n_keep], True, axis=1)
    return keep


def pack_masks(keep: np.ndarray) -> np.ndarray:
    """Bitmap ([summary] Methodology 4): uint64 [N x ceil(K/64)], bit b of
    word w set iff column 64w+b is kept."""
    N, K = keep.shape
    nw = -(-K // WORD)
    padded = np.zeros((N, nw * WORD), dtype=np.uint64)
    padded[:, :K] = keep
    weights = np.left_shift(np.uint64(1), np.arange(WORD, dtype=np.uint64))
    return (padded.reshape(N, nw, WORD) * weights).sum(axis=2, dtype=np.uint64)


def pack_values(W_bits: np.ndarray, keep: np.ndarray, n_keep: int) -> np.ndarray:
    """Compact array of kept values ([summary] Methodology 4): uint16
    [N x n_keep], each row's kept bf16 patterns in ascending column order,
    copied bit for bit."""
    N = W_bits.shape[0]
    return np.asarray(W_bits, dtype=np.uint16)[keep].reshape(N, n_keep)


def block_offsets(keep: np.ndarray) -> np.ndarray:
    """Per-row lookup table read beside the bitmap ([summary] Methodology 4,
    stage 1): uint32 [N x ceil(K/1024)], entry g = kept columns < 1024*g."""
    N, K = keep.shape
    ng = -(-K // OFFSET_GROUP)
    out = np.zeros((N, ng), dtype=np.uint32)
    for g in range(ng):
        out[:, g] = keep[:, : g * OFFSET_GROUP].sum(axis=1)
    return out


def residual(W_bits: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Pruning residual R = W - W_s = W with the kept entries zeroed
    ([summary] Methodology 2, residual decomposition).  float64, exact."""
    return np.where(keep, 0.0, bits_to_f64(W_bits))


def truncated_svd(R: np.ndarray, r: int):
    """Rank-r truncated SVD of the residual ([summary] Methodology 2).

    LAPACK (numpy.linalg.svd, thin) in float64.  Returns U_r [N x r],
    S_r [r], V_r [K x r] with each (u_i, v_i) pair's sign chosen so that the
    largest-magnitude entry of v_i is positive (first such entry on ties).
    """
    N, K = R.shape
    if not 0 <= r <= min(N, K):
        raise ValueError("rank must lie in [0, min(N, K)]")
    if r == 0:
        return np.zeros((N, 0)), np.zeros(0), np.zeros((K, 0))
    U, S, Vt = np.linalg.svd(R, full_matrices=False)
    U, S, V = U[:, :r], S[:r], Vt[:r].T
    pivot = np.argmax(np.abs(V), axis=0)
    sign = np.sign(V[pivot, np.arange(r)])
    sign[sign == 0] = 1.0
    return U * sign, S, V * sign


def singular_values(R: np.ndarray) -> np.ndarray:
    """Every singular value of the residual, descending ([summary]
    Methodology 2: the residual's spectrum, whose discarded tail is the
    error of the rank-r factorization).  LAPACK in float64, values only."""
    return np.linalg.svd(R, compute_uv=False)


def residual_factors(U_r, S_r, V_r):
    """Balanced split of the truncated SVD into an adapter pair, float64:
    A' = V_r diag(sqrt(S_r)) [K x r], B' = diag(sqrt(S_r)) U_r^T [r x N],
    so that A'B' = (U_r S_r V_r^T)^T."""
    root = np.sqrt(S_r)
    return V_r * root, (U_r * root).T


def concat_adapters(blocks_A, blocks_B):
    """Stack adapters along the rank dimension ([summary] Methodology 3):
    A_cat = [A_0 | A_1 | ...] [K x r_cat], B_cat = [B_0; B_1; ...]
    [r_cat x N]."""
    return np.concatenate(blocks_A, axis=1), np.concatenate(blocks_B, axis=0)


@dataclass
class Encoded:
    masks: np.ndarray      # uint64 [N x ceil(K/64)]
    values: np.ndarray     # uint16 [N x n_keep]
    offsets: np.ndarray    # uint32 [N x ceil(K/1024)]
    A_cat: np.ndarray      # uint16 [K x r_cat]  (bf16 patterns)
    B_cat: np.ndarray      # uint16 [r_cat x N]  (bf16 patterns)
    keep: np.ndarray       # bool   [N x K]
    S: np.ndarray          # float64 [r_svd], singular values of R
    R_energy: float        # ||R||_F^2
    tail_energy: float     # sum of sigma_i^2 for i > r_svd  (optimal error)


def encode(W_bits, n_keep: int, r_svd: int, lora_A=(), lora_B=()) -> Encoded:
    """SALR encode, steps in the pages' order: magnitude mask, bitmap +
    values (+ lookup table), residual, truncated SVD, adapter concatenation.

    lora_A[i] is the adapter's down projection in nn.Linear layout
    [r_i x K] (= A_i^T) and lora_B[i] its up projection [N x r_i] (= B_i^T),
    both bf16 patterns; their bits are copied unchanged into A_cat / B_cat.
    """
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    keep = select_keep(W_bits, n_keep)
    masks = pack_masks(keep)
    values = pack_values(W_bits, keep, n_keep)
    offsets = block_offsets(keep)
    R = residual(W_bits, keep)
    U, S, V = truncated_svd(R, r_svd)
    A1, B1 = residual_factors(U, S, V)
    blocks_A = [f64_to_bits(A1)] + [np.asarray(a, dtype=np.uint16).T for a in lora_A]
    blocks_B = [f64_to_bits(B1)] + [np.asarray(b, dtype=np.uint16).T for b in lora_B]
    A_cat, B_cat = concat_adapters(blocks_A, blocks_B)
    R_energy = float(np.sum(R * R))
    tail = max(0.0, R_energy - float(np.sum(S * S)))
    return Encoded(masks, values, offsets, np.ascontiguousarray(A_cat),
                   np.ascontiguousarray(B_cat), keep, S, R_energy, tail)


# ---------------------------------------------------------------------------
# Decode and forward.  [summary] Methodology 4: stage 1 rebuilds dense blocks
# of the pruned weight from bitmap + values; stage 2 multiplies them.
# [summary] Methodology 3: one concatenated low-rank product.
# ---------------------------------------------------------------------------

def decode_keep(masks: np.ndarray, K: int) -> np.ndarray:
    """The kept set, bool [N x K], from the bitmap words."""
    masks = np.asarray(masks, dtype=np.uint64)
    N, nw = masks.shape
    bits = (masks[:, :, None] >> np.arange(WORD, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(N, nw * WORD)[:, :K].astype(bool)


def decode_dense_bits(masks: np.ndarray, values: np.ndarray, K: int) -> np.ndarray:
    """Stage-1 decode keeping bit patterns: uint16 [N x K], row n's values at
    the set bits of its bitmap in ascending column order, 0 elsewhere."""
    keep = decode_keep(masks, K)
    N = keep.shape[0]
    out = np.zeros((N, K), dtype=np.uint16)
    values = np.asarray(values, dtype=np.uint16)
    for n in range(N):
        c = int(keep[n].sum())
        out[n, keep[n]] = values[n, :c]
    return out


def decode_dense(masks: np.ndarray, values: np.ndarray, K: int) -> np.ndarray:
    """Stage-1 decode to a dense float64 W_s [N x K]: row n's values are
    placed, in ascending column order, at the set bits of its bitmap."""
    masks = np.asarray(masks, dtype=np.uint64)
    N, nw = masks.shape
    bits = (masks[:, :, None] >> np.arange(WORD, dtype=np.uint64)) & np.uint64(1)
    keep = bits.reshape(N, nw * WORD)[:, :K].astype(bool)
    counts = keep.sum(axis=1)
    vals = bits_to_f64(values)
    if np.any(counts > vals.shape[1]):
        raise ValueError("bitmap holds more set bits than values per row")
    Ws = np.zeros((N, K), dtype=np.float64)
    for n in range(N):
        Ws[n, keep[n]] = vals[n, : counts[n]]
    return Ws


def forward(X_bits, masks, values, K: int, A_cat_bits, B_cat_bits) -> np.ndarray:
    """Y = X W_s^T + (X A_cat) B_cat in float64, no intermediate rounding.
    X [M x K], A_cat [K x r_cat], B_cat [r_cat x N], all bf16 patterns."""
    X = bits_to_f64(X_bits)
    Ws = decode_dense(masks, values, K)
    A = bits_to_f64(A_cat_bits)
    B = bits_to_f64(B_cat_bits)
    return X @ Ws.T + (X @ A) @ B


def forward_rows(X_bits, masks, values, K: int, A_cat_bits, B_cat_bits, rows) -> np.ndarray:
    """The same forward for a subset of output columns `rows` (indices into
    N) only: Y[:, rows].  Used to check full-size results on samples."""
    rows = np.asarray(rows)
    X = bits_to_f64(X_bits)
    Ws = decode_dense(np.asarray(masks)[rows], np.asarray(values)[rows], K)
    A = bits_to_f64(A_cat_bits)
    B = bits_to_f64(np.asarray(B_cat_bits)[:, rows])
    return X @ Ws.T + (X @ A) @ B


# ---------------------------------------------------------------------------
# Multi-projection fusion.  [summary] Methodology 3 runs every adapter as one
# low-rank product on the shared input; projections that share an input
# (q/k/v, gate/up) are fused the same way: W_s rows stacked, adapter ranks
# stacked, each projection's up-projection kept on its own ranks only.
# ---------------------------------------------------------------------------

def fuse(parts):
    """One encoding from `parts` (each with masks, values, offsets, A_cat
    [K x r_p], B_cat [r_p x N_p]; all with the same K and n_keep): masks,
    values and offsets stacked along N, A_cat = [A_0 | A_1 | ...] and B_cat
    block diagonal (B_p at rows R_p.., columns N_0 + ... + N_{p-1}..).
    Returns a dict with those five arrays."""
    parts = list(parts)
    Ns = [p.masks.shape[0] for p in parts]
    ranks = [p.A_cat.shape[1] for p in parts]
    B = np.zeros((sum(ranks), sum(Ns)), dtype=np.uint16)
    r0 = n0 = 0
    for p, n, r in zip(parts, Ns, ranks):
        B[r0:r0 + r, n0:n0 + n] = p.B_cat
        r0 += r
        n0 += n
    return {
        "masks": np.concatenate([p.masks for p in parts], axis=0),
        "values": np.concatenate([p.values for p in parts], axis=0),
        "offsets": np.concatenate([p.offsets for p in parts], axis=0),
        "A_cat": np.concatenate([p.A_cat for p in parts], axis=1),
        "B_cat": B,
    }


def max_rel_err(Y_hat, Y) -> float:
    """Error metric for Y: max_ij |Y_hat - Y| / max(|Y_ij|, rms(Y)).
    A pure elementwise relative error is dominated by outputs that happen to
    be near zero; flooring the denominator at rms(Y) keeps the metric a
    statement about the layer's precision."""
    Y = np.asarray(Y, dtype=np.float64)
    Y_hat = np.asarray(Y_hat, dtype=np.float64)
    if Y.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(Y * Y)))
    den = np.maximum(np.abs(Y), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(Y_hat - Y) / den))
