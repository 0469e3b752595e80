"""Pins of the grouped (mixture-of-experts) oracle (oracle/moe.py).

The grouped forward is checked against a per-token brute force that never
goes through the encoding: each token finds its expert by scanning the row
boundaries, the expert's pruned weight is the original W with the entries
outside a brute-force top-n_keep set zeroed, and every output is an explicit
sum over k of the token's activations times that weight, plus the LoRA
product summed rank by rank.
Planted mistakes (a boundary off by one, two experts swapped) must fail it;
empty groups, a one-token group and E = 1 are covered."""

import numpy as np
import pytest

from oracle import bf16 as ob
from oracle import moe
from oracle import salr as osl


def _brute_keep(W_bits, n_keep):
    """Per row: rank every entry by (magnitude descending, column
    ascending) with a pairwise count, keep the n_keep best."""
    N, K = W_bits.shape
    mag = (W_bits & 0x7FFF).astype(np.int64)
    keep = np.zeros((N, K), dtype=bool)
    for n in range(N):
        for k in range(K):
            better = sum(1 for j in range(K) if mag[n, j] > mag[n, k] or (mag[n, j] == mag[n, k] and j < k))
            keep[n, k] = better < n_keep
    return keep


def _experts(E, N, K, n_keep, ranks, seed):
    rng = np.random.default_rng(seed)
    raw, enc = [], []
    for e in range(E):
        W = ob.f64_to_bits(rng.standard_normal((N, K)))
        r = ranks[e]
        A = ob.f64_to_bits(rng.standard_normal((r, K)) * 0.3)      # LoRA down, [r][K]
        B = ob.f64_to_bits(rng.standard_normal((N, r)) * 0.3)      # LoRA up, [N][r]
        en = osl.encode(W, n_keep, 0, [A], [B])
        raw.append((W, A, B))
        enc.append((en.masks, en.values, en.A_cat, en.B_cat))
    return raw, enc


def _brute(X_bits, offsets, raw, n_keep):
    X = ob.bits_to_f64(X_bits)
    T, K = X.shape
    N = raw[0][0].shape[0]
    Y = np.zeros((T, N))
    for t in range(T):
        e = 0
        while not (offsets[e] <= t < offsets[e + 1]):
            e += 1
        W, A, B = raw[e]
        Wd = ob.bits_to_f64(W) * _brute_keep(W, n_keep)
        Af, Bf = ob.bits_to_f64(A), ob.bits_to_f64(B)
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += X[t, k] * Wd[n, k]
            for j in range(Af.shape[0]):
                s += sum(X[t, k] * Af[j, k] for k in range(K)) * Bf[n, j]
            Y[t, n] = s
    return Y


CASES = [
    # E, N, K, n_keep, ranks, offsets
    (3, 5, 12, 6, (2, 1, 3), (0, 2, 2, 5)),          # an empty middle expert
    (4, 4, 8, 3, (1, 1, 1, 1), (0, 1, 4, 4, 6)),     # a one-token group, an empty last
    (1, 6, 16, 9, (2,), (0, 3)),                     # one expert: the plain layer
]


@pytest.mark.parametrize("E,N,K,n_keep,ranks,offsets", CASES)
def test_grouped_forward_matches_brute_force(E, N, K, n_keep, ranks, offsets):
    raw, enc = _experts(E, N, K, n_keep, ranks, seed=E * 10 + N)
    T = offsets[-1]
    X = ob.f64_to_bits(np.random.default_rng(7).standard_normal((T, K)))
    Y = moe.grouped_forward(X, offsets, enc, K)
    Yb = _brute(X, offsets, raw, n_keep)
    assert np.max(np.abs(Y - Yb)) <= 1e-12 * max(1.0, np.max(np.abs(Yb)))
    rows = np.array([N - 1, 0])
    assert np.array_equal(moe.grouped_forward_rows(X, offsets, enc, K, rows), Y[:, rows])


def test_planted_mistakes_are_caught():
    E, N, K, n_keep = 3, 5, 12, 6
    raw, enc = _experts(E, N, K, n_keep, (2, 2, 2), seed=3)
    offsets = (0, 2, 3, 6)
    X = ob.f64_to_bits(np.random.default_rng(8).standard_normal((6, K)))
    Yb = _brute(X, offsets, raw, n_keep)
    tol = 1e-12 * np.max(np.abs(Yb))
    # a boundary off by one (token 2 computed by expert 0)
    shifted = moe.grouped_forward(X, (0, 3, 3, 6), enc, K)
    assert np.max(np.abs(shifted - Yb)) > tol
    # two experts' encodings swapped
    swapped = moe.grouped_forward(X, offsets, [enc[1], enc[0], enc[2]], K)
    assert np.max(np.abs(swapped - Yb)) > tol


def test_offsets_validation():
    _, enc = _experts(2, 4, 8, 4, (1, 1), seed=1)
    X = np.zeros((3, 8), dtype=np.uint16)
    for bad in ((0, 2), (1, 2, 3), (0, 2, 1), (0, 4, 3), (0, 1, 4)):
        with pytest.raises(ValueError):
            moe.grouped_forward(X, bad, enc, 8)
    assert not moe.grouped_forward(X, (0, 1, 3), enc, 8).any()
