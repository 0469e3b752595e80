"""Encode parity: salr_encode on the GPU against the oracle.

Bitmap, packed values, lookup table and the LoRA blocks of A_cat / B_cat are
compared bit for bit.  The truncated-SVD block is compared by what is unique
about it (several factorizations are correct): the error it leaves,
||R - (A' B')^T||^2, must recover at least 99% of the optimal reduction
(Eckart-Young: the oracle's discarded singular values) and satisfy the
per-entry MSE bound (1 - r/min(N,K)) from the pages; the reported singular
values must match LAPACK's to 1e-2 relative."""

import numpy as np
import pytest

from oracle import bf16 as ob
from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits

pytestmark = pytest.mark.gpu


def _weights(N, K, kind, seed):
    if kind == "ties":
        # few distinct magnitudes: nearly every row has ties at the cut
        rng = np.random.default_rng(seed)
        return ob.f64_to_bits(rng.integers(-4, 5, size=(N, K)).astype(np.float64) * 0.01)
    if kind == "t3":
        return synth.make_w(N, K, seed, dist="t3")
    return synth.make_w(N, K, seed)


def _loras(N, K, ranks, seed):
    rng = np.random.default_rng(seed + 1)
    As = [ob.f64_to_bits(rng.standard_normal((q, K)).astype(np.float32) * 0.01) for q in ranks]
    Bs = [ob.f64_to_bits(rng.standard_normal((N, q)).astype(np.float32) * 0.01) for q in ranks]
    return As, Bs


# N, K, n_keep, r_svd, LoRA ranks, weight kind
CASES = [
    (512, 512, 256, 16, (8,), "normal"),
    (100, 520, 260, 4, (3, 5), "normal"),
    (64, 4096, 1229, 8, (), "ties"),
    (96, 2048, 614, 12, (4,), "t3"),
    (33, 1024, 1024, 0, (16,), "normal"),
    (40, 1032, 0, 0, (8,), "normal"),
    (5, 20480, 10240, 2, (), "ties"),   # > 256 bitmap words per row: segmented scan
]


def _gpu_encode(W, n_keep, r_svd, As, Bs, **kw):
    import torch
    import sparse_rank_linear_amd as srl

    layer, sigma = srl.encode(to_dev(W), n_keep, r_svd, [to_dev(a) for a in As], [to_dev(b) for b in Bs], **kw)
    torch.cuda.synchronize()
    return layer, np.array(sigma)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}_K{c[1]}_keep{c[2]}_r{c[3]}_{c[5]}")
def test_encode_matches_oracle(case):
    N, K, n_keep, r_svd, ranks, kind = case
    say(f"encode N={N} K={K} n_keep={n_keep} r_svd={r_svd} loras={ranks} {kind}")
    W = _weights(N, K, kind, seed=N * 7 + K)
    As, Bs = _loras(N, K, ranks, seed=N + K)
    enc = osl.encode(W, n_keep, r_svd, As, Bs)
    layer, sigma = _gpu_encode(W, n_keep, r_svd, As, Bs)
    got = layer.to_numpy()
    assert np.array_equal(got["masks"], enc.masks)
    assert np.array_equal(got["values"], enc.values)
    assert np.array_equal(got["offsets"], enc.offsets)
    # LoRA blocks: bit copies in call order
    assert np.array_equal(got["a_cat"][r_svd:], enc.A_cat[:, r_svd:].T)
    assert np.array_equal(got["b_cat"][:, r_svd:], enc.B_cat[r_svd:].T)
    if r_svd == 0:
        return
    R = osl.residual(W, enc.keep)
    A1 = ob.bits_to_f64(got["a_cat"][:r_svd])        # [r][K] = A'^T
    B1 = ob.bits_to_f64(got["b_cat"][:, :r_svd])     # [N][r] = B'^T
    before = float(np.sum(R * R))
    after = float(np.sum((R - B1 @ A1) ** 2))
    optimal = enc.tail_energy
    say(f"  residual energy before={before:.6e} gpu={after:.6e} optimal={optimal:.6e}")
    assert before - after >= 0.99 * (before - optimal)
    assert after / (N * K) <= (1 - r_svd / min(N, K)) * before / (N * K)
    rel = np.abs(sigma - enc.S) / enc.S
    say(f"  max sigma rel err={rel.max():.2e}")
    assert rel.max() <= 1e-2


def _signed_zero_subnormal_weight(N, K, seed):
    """Rows of +0.0, -0.0, subnormal and small normal bf16 patterns (about
    40% / 40% / 20%): at a high n_keep the kept set holds every normal and
    subnormal entry plus the lowest-column zeros of both signs."""
    rng = np.random.default_rng(seed)
    u = rng.random((N, K))
    sign = rng.integers(0, 2, size=(N, K)).astype(np.uint16) << 15
    sub = rng.integers(1, 0x80, size=(N, K)).astype(np.uint16)        # exponent 0, fraction != 0
    normal = rng.integers(0x0080, 0x3C00, size=(N, K)).astype(np.uint16)
    W = np.where(u < 0.4, np.uint16(0), np.where(u < 0.8, sub, normal)) | sign
    return W.astype(np.uint16)


@pytest.mark.parametrize("n_keep", [900, 1000])
def test_encode_keeps_signed_zeros_and_subnormals(n_keep):
    """A kept -0.0 still sets its bit and is stored as 0x8000, kept
    subnormals keep their patterns, and +0/-0 tie (lower column kept)."""
    N, K = 48, 1024
    say(f"encode signed zeros / subnormals N={N} K={K} n_keep={n_keep}")
    W = _signed_zero_subnormal_weight(N, K, seed=n_keep)
    enc = osl.encode(W, n_keep, 0)
    kept = enc.values
    assert np.any(kept == 0x8000) and np.any(kept == 0x0000), "case must keep zeros of both signs"
    assert np.any(((kept & 0x7F80) == 0) & ((kept & 0x7F) != 0)), "case must keep subnormals"
    layer, _ = _gpu_encode(W, n_keep, 0, [], [])
    got = layer.to_numpy()
    assert np.array_equal(got["masks"], enc.masks)
    assert np.array_equal(got["values"], enc.values)
    assert np.array_equal(got["offsets"], enc.offsets)


def test_encode_zero_residual_with_residual_rank():
    """Nothing pruned (n_keep = K) with a residual rank requested: the
    residual is zero, so its singular values and the adapter block are zero
    (oracle: S = 0)."""
    N, K, r_svd = 64, 512, 4
    W = synth.make_w(N, K, seed=3)
    As, Bs = _loras(N, K, (8,), seed=3)
    enc = osl.encode(W, K, r_svd, As, Bs)
    assert enc.R_energy == 0.0 and np.all(enc.S == 0)
    layer, sigma = _gpu_encode(W, K, r_svd, As, Bs)
    got = layer.to_numpy()
    assert np.array_equal(got["masks"], enc.masks) and np.array_equal(got["values"], enc.values)
    assert np.all(sigma == 0.0)
    A1 = ob.bits_to_f64(got["a_cat"][:r_svd])
    B1 = ob.bits_to_f64(got["b_cat"][:, :r_svd])
    assert np.all(B1 @ A1 == 0.0)
    assert np.array_equal(got["a_cat"][r_svd:], enc.A_cat[:, r_svd:].T)


def test_encode_rejects_nonfinite():
    import sparse_rank_linear_amd as srl

    W = synth.make_w(32, 64, seed=1)
    W[5, 7] = 0x7FC0  # NaN
    with pytest.raises(srl.SalrError, match="NONFINITE"):
        _gpu_encode(W, 32, 2, [], [])
    W[5, 7] = 0xFF80  # -Inf
    with pytest.raises(srl.SalrError, match="NONFINITE"):
        _gpu_encode(W, 32, 0, [], [])


def test_encode_then_forward_end_to_end():
    """GPU encode -> GPU forward against oracle encode -> oracle forward."""
    import torch
    import sparse_rank_linear_amd as srl

    wl = synth.WORKLOADS["tiny_512"]
    inp = synth.make_inputs(wl)
    enc = osl.encode(inp.W, wl.n_keep, wl.r_svd, inp.lora_A, inp.lora_B)
    layer, _ = _gpu_encode(inp.W, wl.n_keep, wl.r_svd, inp.lora_A, inp.lora_B)
    for M in (wl.M, 100):
        X = synth.make_x(wl.K, M, seed=M) if M != wl.M else inp.X
        Y = srl.linear_forward(layer, to_dev(X))
        torch.cuda.synchronize()
        Yref = osl.forward(X, enc.masks, enc.values, wl.K, enc.A_cat, enc.B_cat)
        mr, nw = errors(to_host_bits(Y), Yref)
        say(f"end-to-end M={M}: max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE
