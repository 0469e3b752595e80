"""Pins of the backward oracle (oracle/backward.py): the gradients against
central finite differences of the forward (the loss sum(Y * dY) is linear in
X, in A_cat and in B_cat separately, so a step of 1 is exact up to
rounding), the transposed encoding against the dense transpose bit for bit,
and a planted missing term that the finite-difference pin catches."""

import numpy as np
import pytest

from oracle import backward as ob_
from oracle import bf16 as ob
from oracle import salr as osl


def _case(N, K, M, n_keep, r, seed):
    rng = np.random.default_rng(seed)
    W = ob.f64_to_bits(rng.standard_normal((N, K)) * 0.5)
    enc = osl.encode(W, n_keep, 0, [ob.f64_to_bits(rng.standard_normal((r, K)))],
                     [ob.f64_to_bits(rng.standard_normal((N, r)))])
    X = ob.f64_to_bits(rng.standard_normal((M, K)))
    dY = ob.f64_to_bits(rng.standard_normal((M, N)))
    return enc, X, dY


def _loss(X, enc, K, A, B, dY):
    Y = osl.forward(X, enc.masks, enc.values, K, A, B)
    return float(np.sum(Y * ob.bits_to_f64(dY)))


def _fd(enc, X, dY, K):
    """Central differences with step 1 on float64 copies (the forward takes
    bf16 patterns, so the perturbed inputs are passed as float64 through a
    thin wrapper that skips the bf16 decode)."""
    Xf, A, B = ob.bits_to_f64(X), ob.bits_to_f64(enc.A_cat), ob.bits_to_f64(enc.B_cat)
    Ws = osl.decode_dense(enc.masks, enc.values, K)
    dYf = ob.bits_to_f64(dY)

    def L(Xv, Av, Bv):
        return float(np.sum((Xv @ Ws.T + (Xv @ Av) @ Bv) * dYf))

    def grad(arr, f):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += 1.0
            m[idx] -= 1.0
            g[idx] = (f(p) - f(m)) / 2.0
        return g

    return (grad(Xf, lambda v: L(v, A, B)), grad(A, lambda v: L(Xf, v, B)), grad(B, lambda v: L(Xf, A, v)))


@pytest.mark.parametrize("N,K,M,n_keep,r", [(12, 16, 3, 7, 2), (9, 24, 2, 24, 3), (16, 8, 4, 0, 1)])
def test_backward_matches_finite_differences(N, K, M, n_keep, r):
    enc, X, dY = _case(N, K, M, n_keep, r, seed=N + K + M)
    dX, dA, dB = ob_.backward(X, dY, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
    gX, gA, gB = _fd(enc, X, dY, K)
    scale = lambda a: max(1.0, float(np.max(np.abs(a))))
    assert np.max(np.abs(dX - gX)) <= 1e-9 * scale(gX)
    assert np.max(np.abs(dA - gA)) <= 1e-9 * scale(gA)
    assert np.max(np.abs(dB - gB)) <= 1e-9 * scale(gB)


def test_planted_missing_adapter_term_is_caught():
    """dX without the low-rank term (dY W_s only) must fail the pin."""
    enc, X, dY = _case(12, 16, 3, 7, 2, seed=4)
    gX, _, _ = _fd(enc, X, dY, 16)
    wrong = ob.bits_to_f64(dY) @ osl.decode_dense(enc.masks, enc.values, 16)
    assert np.max(np.abs(wrong - gX)) > 1e-3 * max(1.0, float(np.max(np.abs(gX))))


@pytest.mark.parametrize("N,K,n_keep", [(70, 130, 40), (64, 64, 64), (30, 200, 0), (129, 72, 35)])
def test_transpose_encoding_is_the_dense_transpose(N, K, n_keep):
    rng = np.random.default_rng(N * K)
    W = ob.f64_to_bits(rng.standard_normal((N, K)))
    enc = osl.encode(W, n_keep, 0)
    mT, vT, oT, nT = ob_.transpose_encoding(enc.masks, enc.values, K)
    dense = osl.decode_dense_bits(enc.masks, enc.values, K)
    assert np.array_equal(osl.decode_dense_bits(mT, vT, N), dense.T)
    keepT = osl.decode_keep(mT, N)
    assert nT == (keepT.sum(axis=1).max() if K else 0)
    assert np.array_equal(oT, osl.block_offsets(keepT))
    # every kept entry of W appears once in the transposed values
    assert int(keepT.sum()) == N * n_keep
