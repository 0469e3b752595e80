"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against an independent statement: a library
conversion routine, hand-worked values, brute force on tiny inputs written
with different code, closed forms the pages state, or matrices whose SVD is
known by construction.  A few tests plant a plausible mistake in a copy of an
oracle function and check that the corresponding pin catches it.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import bf16 as ob
from oracle import salr as osl
from sparse_rank_linear_amd import synth


def _rand_bits(rng, shape, scale=0.02):
    x = (rng.standard_normal(shape) * scale).astype(np.float32).astype(np.float64)
    return ob.f64_to_bits(x)


# ---------------------------------------------------------------- bf16 -----

def test_bf16_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200_000).astype(np.float32)
    x *= np.exp(rng.uniform(-60, 60, x.size)).astype(np.float32)
    x = x[np.isfinite(x)]
    ours = ob.f64_to_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_hand_cases():
    f = lambda v: int(ob.f64_to_bits(np.array([v]))[0])
    assert f(1.0) == 0x3F80
    assert f(-2.0) == 0xC000
    assert f(1 + 2 ** -8) == 0x3F80            # tie -> even (fraction 0)
    assert f(1 + 3 * 2 ** -8) == 0x3F82        # tie -> even (fraction 2)
    assert f(1 + 2 ** -8 + 2 ** -40) == 0x3F81  # direct rounding: just above the tie
    assert f(-0.0) == 0x8000
    assert f(np.inf) == 0x7F80 and f(-np.inf) == 0xFF80
    assert f(np.nan) == 0x7FC0
    assert f(3.4e38) == 0x7F80                 # beyond (2 - 2^-8) 2^127 -> Inf
    assert f(2.0 ** -133) == 0x0001            # smallest subnormal
    assert f(2.0 ** -134) == 0x0000            # tie to even at zero
    back = ob.bits_to_f64(np.array([0x3F81, 0x8000, 0x0001], dtype=np.uint16))
    assert back[0] == 1 + 2 ** -7 and np.signbit(back[1]) and back[2] == 2.0 ** -133


# ----------------------------------------------------------- selection -----

def _brute_keep(W_bits, n_keep):
    """Independent selection: column c is kept iff fewer than n_keep columns
    beat it, where j beats c when |w_j| > |w_c| or (equal and j < c)."""
    N, K = W_bits.shape
    keep = np.zeros((N, K), dtype=bool)
    for n in range(N):
        mags = [int(b) & 0x7FFF for b in W_bits[n]]
        for c in range(K):
            beaten = sum(1 for j in range(K) if mags[j] > mags[c] or (mags[j] == mags[c] and j < c))
            keep[n, c] = beaten < n_keep
    return keep


@pytest.mark.parametrize("K,n_keep", [(7, 3), (64, 32), (100, 50), (130, 1), (33, 33), (40, 0)])
def test_select_matches_brute_force(K, n_keep):
    rng = np.random.default_rng(K * 31 + n_keep)
    # a narrow value range forces many equal magnitudes (ties at the cut)
    W = ob.f64_to_bits(rng.integers(-6, 7, size=(5, K)).astype(np.float64) * 0.25)
    assert np.array_equal(osl.select_keep(W, n_keep), _brute_keep(W, n_keep))


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 4), st.integers(1, 150), st.data())
def test_select_properties(N, K, data):
    n_keep = data.draw(st.integers(0, K))
    vals = data.draw(st.lists(st.integers(-5, 5), min_size=N * K, max_size=N * K))
    W = ob.f64_to_bits(np.array(vals, dtype=np.float64).reshape(N, K) * 0.5)
    keep = osl.select_keep(W, n_keep)
    mag = (W & 0x7FFF).astype(int)
    assert np.all(keep.sum(axis=1) == n_keep)
    for n in range(N):
        kept, pruned = mag[n][keep[n]], mag[n][~keep[n]]
        if kept.size and pruned.size:
            assert kept.min() >= pruned.max()
            t = kept.min()
            if t == pruned.max():
                ties = np.nonzero(mag[n] == t)[0]
                # among the tied columns the kept ones are a prefix
                flags = keep[n][ties]
                assert np.all(flags[: flags.sum()]) and not np.any(flags[flags.sum():])


def test_select_signed_zero_ties_and_nonfinite():
    W = np.array([[0x8000, 0x0000, 0x3F80, 0xBF80]], dtype=np.uint16)  # -0, +0, 1, -1
    keep = osl.select_keep(W, 3)
    assert keep.tolist() == [[True, False, True, True]]   # -0 and +0 tie: lower column kept
    with pytest.raises(osl.NonFiniteWeight):
        osl.select_keep(np.array([[0x3F80, 0x7F80]], dtype=np.uint16), 1)
    with pytest.raises(osl.NonFiniteWeight):
        osl.select_keep(np.array([[0x7FC1, 0x0000]], dtype=np.uint16), 1)


def test_planted_tie_flip_is_caught():
    """A selection that breaks ties toward the higher column must fail the
    brute-force pin."""
    def wrong(W_bits, n_keep):
        mag = (W_bits & 0x7FFF).astype(np.int64)
        K = W_bits.shape[1]
        key = -mag * (K + 1) - np.arange(K)      # ties: higher column first
        order = np.argsort(key, axis=1, kind="stable")
        keep = np.zeros(W_bits.shape, dtype=bool)
        np.put_along_axis(keep, order[:, :n_keep], True, axis=1)
        return keep

    W = ob.f64_to_bits(np.array([[1, 1, 2, 1, 0, 1, 2, 1.0]]))
    assert np.array_equal(osl.select_keep(W, 4), _brute_keep(W, 4))
    assert not np.array_equal(wrong(W, 4), _brute_keep(W, 4))


# ------------------------------------------------------------- packing -----

def test_pack_hand_example():
    # row 0 keeps columns 0, 2, 63, 64, 69; row 1 keeps columns 1, 3, 10, 65, 66
    K = 70
    keep = np.zeros((2, K), dtype=bool)
    keep[0, [0, 2, 63, 64, 69]] = True
    keep[1, [1, 3, 10, 65, 66]] = True
    masks = osl.pack_masks(keep)
    assert masks.dtype == np.uint64 and masks.shape == (2, 2)
    assert int(masks[0, 0]) == (1 << 0) | (1 << 2) | (1 << 63)
    assert int(masks[0, 1]) == (1 << 0) | (1 << 5)
    assert int(masks[1, 0]) == (1 << 1) | (1 << 3) | (1 << 10)
    assert int(masks[1, 1]) == (1 << 1) | (1 << 2)
    W = (np.arange(2 * K, dtype=np.uint16).reshape(2, K) + 0x3F00).astype(np.uint16)
    vals = osl.pack_values(W, keep, 5)
    assert vals.tolist() == [[0x3F00, 0x3F02, 0x3F00 + 63, 0x3F00 + 64, 0x3F00 + 69],
                             [0x3F00 + 71, 0x3F00 + 73, 0x3F00 + 80, 0x3F00 + 135, 0x3F00 + 136]]


def test_offsets_hand_example():
    K = 2500
    keep = np.zeros((1, K), dtype=bool)
    keep[0, [5, 1023, 1024, 2047, 2048, 2499]] = True
    assert osl.block_offsets(keep).tolist() == [[0, 2, 4]]


@pytest.mark.parametrize("N,K,n_keep", [(3, 64, 32), (4, 100, 50), (2, 1030, 515), (3, 65, 65), (2, 10, 0)])
def test_roundtrip_bitwise(N, K, n_keep):
    rng = np.random.default_rng(N * K + n_keep)
    W = _rand_bits(rng, (N, K))
    W[0, : min(4, K)] = 0x8000  # kept signed zeros must survive
    enc = osl.encode(W, n_keep, 0)
    # per-bit loop over the bitmap, independent of pack_masks
    for n in range(N):
        for c in range(K):
            bit = (int(enc.masks[n, c // 64]) >> (c % 64)) & 1
            assert bit == int(enc.keep[n, c])
        for c in range(K, enc.masks.shape[1] * 64):
            assert (int(enc.masks[n, c // 64]) >> (c % 64)) & 1 == 0
    popc = np.array([[bin(int(w)).count("1") for w in row] for row in enc.masks])
    assert np.all(popc.sum(axis=1) == n_keep)
    for n in range(N):
        for g in range(enc.offsets.shape[1]):
            assert enc.offsets[n, g] == sum(enc.keep[n, : 1024 * g])
    dense = osl.decode_dense(enc.masks, enc.values, K)
    got = ob.f64_to_bits(dense)
    want = np.where(enc.keep, W, np.uint16(0))
    assert np.array_equal(got, want)


def test_planted_reversed_value_order_is_caught():
    rng = np.random.default_rng(3)
    W = _rand_bits(rng, (2, 64))
    enc = osl.encode(W, 32, 0)
    bad = enc.values[:, ::-1].copy()
    got = ob.f64_to_bits(osl.decode_dense(enc.masks, bad, 64))
    assert not np.array_equal(got, np.where(enc.keep, W, np.uint16(0)))


# ----------------------------------------------------------------- SVD -----

def _known_svd_matrix(rng, N, K, s):
    U, _ = np.linalg.qr(rng.standard_normal((N, len(s))))
    V, _ = np.linalg.qr(rng.standard_normal((K, len(s))))
    return U, V, (U * s) @ V.T


def test_svd_on_known_spectrum():
    rng = np.random.default_rng(11)
    s = np.array([9.0, 7.0, 5.0, 3.0, 2.0, 1.0, 0.5])
    U, V, R = _known_svd_matrix(rng, 40, 30, s)
    Ur, Sr, Vr = osl.truncated_svd(R, 3)
    assert np.allclose(Sr, s[:3], rtol=1e-12)
    assert np.allclose((Ur * Sr) @ Vr.T, (U[:, :3] * s[:3]) @ V[:, :3].T, atol=1e-11)
    # sign convention: largest-|.| entry of each right vector is positive
    for i in range(3):
        assert Vr[np.argmax(np.abs(Vr[:, i])), i] > 0
    A1, B1 = osl.residual_factors(Ur, Sr, Vr)
    assert A1.shape == (30, 3) and B1.shape == (3, 40)
    # balanced split: ||A'_i|| = ||B'_i|| = sqrt(sigma_i)
    assert np.allclose(np.linalg.norm(A1, axis=0), np.sqrt(s[:3]))
    assert np.allclose(np.linalg.norm(B1, axis=1), np.sqrt(s[:3]))
    assert np.allclose(A1 @ B1, ((U[:, :3] * s[:3]) @ V[:, :3].T).T, atol=1e-11)


def test_singular_values_on_known_spectrum():
    """The values-only spectrum used for the full-size fixtures: a matrix of
    known singular values (rank 7 in 40 x 30: the rest are zero), and the
    tail energy identity sum(sigma^2) = ||R||_F^2."""
    rng = np.random.default_rng(13)
    s = np.array([9.0, 7.0, 5.0, 3.0, 2.0, 1.0, 0.5])
    _, _, R = _known_svd_matrix(rng, 40, 30, s)
    S = osl.singular_values(R)
    assert S.shape == (30,)
    assert np.allclose(S[:7], s, rtol=1e-12)
    assert np.all(np.abs(S[7:]) < 1e-12)
    assert np.isclose(np.sum(S ** 2), np.sum(R * R), rtol=1e-12)


def test_svd_full_rank_reconstructs():
    rng = np.random.default_rng(12)
    R = rng.standard_normal((20, 13))
    U, S, V = osl.truncated_svd(R, 13)
    A1, B1 = osl.residual_factors(U, S, V)
    assert np.max(np.abs(A1 @ B1 - R.T)) < 1e-13


@pytest.mark.parametrize("N,K,n_keep,r,dist", [(512, 512, 256, 16, "normal"), (256, 384, 115, 24, "t3"),
                                             (300, 200, 200, 10, "normal")])
def test_mse_bound_from_the_pages(N, K, n_keep, r, dist):
    """[summary] Methodology 2 / [abstract]: the rank-r correction lowers the
    per-entry MSE of the pruning residual by at least (1 - r/min(d,k)).
    Checked with the bf16-rounded factors the encoding stores."""
    W = synth.make_w(N, K, seed=N + K, dist=dist)
    enc = osl.encode(W, n_keep, r)
    R = osl.residual(W, enc.keep)
    A1 = ob.bits_to_f64(enc.A_cat[:, :r])
    B1 = ob.bits_to_f64(enc.B_cat[:r])
    before = np.mean(R * R)
    after = np.mean((R - (A1 @ B1).T) ** 2)
    if n_keep == K:
        assert before == 0 and after == 0
    else:
        assert after <= (1 - r / min(N, K)) * before
        # and the optimum (sum of the discarded sigma^2) is reached up to bf16
        assert after <= enc.tail_energy / (N * K) * (1 + 1e-3)


def _known_residual_weight(seed):
    """A bf16 weight whose pruned residual has a spectrum known in closed
    form.  Every row holds n_keep entries of magnitude 1.0 (the kept set,
    strictly larger than everything else), and the other columns hold a
    row- and column-permuted block diagonal of 2x2 blocks [[a, b], [b, a]]
    (singular values |a + b| and |a - b|) and 1x1 blocks [d] (singular value
    |d|), all exact in bf16.  Returns W bits, n_keep and the residual's
    singular values (descending, zeros included)."""
    rng = np.random.default_rng(seed)
    pairs = [(0.375, 0.125), (-0.25, 0.1875), (0.09375, -0.03125)]
    singles = [0.4375, -0.15625, 0.0078125]
    N = 2 * len(pairs) + len(singles)                 # 9 rows
    K_res, n_keep = N + 3, 7                          # 3 residual columns stay zero
    block = np.zeros((N, K_res))
    spec = []
    i = 0
    for a, b in pairs:
        block[i:i + 2, i:i + 2] = [[a, b], [b, a]]
        spec += [abs(a + b), abs(a - b)]
        i += 2
    for d in singles:
        block[i, i] = d
        spec.append(abs(d))
        i += 1
    block = block[rng.permutation(N)][:, rng.permutation(K_res)]
    K = K_res + n_keep
    W = np.zeros((N, K))
    big_cols = np.sort(rng.choice(K, n_keep, replace=False))
    W[:, big_cols] = rng.choice([-1.0, 1.0], size=(N, n_keep))
    W[:, np.setdiff1d(np.arange(K), big_cols)] = block
    spec = np.sort(np.array(spec))[::-1]
    return ob.f64_to_bits(W), n_keep, spec


def _tail_pin_holds(enc, spec, r):
    """R_energy is the sum of all sigma^2 and tail_energy the sum of the
    sigma^2 beyond rank r (Eckart-Young: the optimal rank-r error)."""
    return (np.isclose(enc.R_energy, float(np.sum(spec ** 2)), rtol=1e-12, atol=0)
            and np.isclose(enc.tail_energy, float(np.sum(spec[r:] ** 2)), rtol=1e-10, atol=1e-300))


@pytest.mark.parametrize("r", [0, 1, 3, 8, 9])
def test_tail_energy_closed_form(r):
    """[summary] Methodology 2: the rank-r truncation of the residual leaves
    exactly the discarded part of its spectrum.  Pinned two-sided on a
    residual whose singular values are known by construction."""
    W, n_keep, spec = _known_residual_weight(seed=r + 3)
    enc = osl.encode(W, n_keep, r)
    assert np.all(enc.keep == (np.abs(ob.bits_to_f64(W)) == 1.0))
    assert _tail_pin_holds(enc, spec, r)
    if r == spec.size:
        assert enc.tail_energy == 0.0


def test_tail_energy_nothing_pruned_and_tiny_layer():
    # n_keep = K: empty residual, no energy on either side of the cut
    rng = np.random.default_rng(21)
    W = _rand_bits(rng, (12, 40))
    enc = osl.encode(W, 40, 5)
    assert enc.R_energy == 0.0 and enc.tail_energy == 0.0
    # the small workload: tail and total against the values-only spectrum of
    # the residual (LAPACK without vectors) at several ranks
    wl = synth.WORKLOADS["tiny_512"]
    W = synth.make_inputs(wl, with_x=False).W
    S_all = osl.singular_values(osl.residual(W, osl.select_keep(W, wl.n_keep)))
    for r in (0, 1, wl.r_svd, 100):
        enc = osl.encode(W, wl.n_keep, r)
        assert np.isclose(enc.R_energy, float(np.sum(S_all ** 2)), rtol=1e-12)
        assert np.isclose(enc.tail_energy, float(np.sum(S_all[r:] ** 2)), rtol=1e-9)


def test_planted_undiscounted_tail_is_caught():
    """A tail that forgets to subtract the captured spectrum (tail = total
    residual energy) must fail the closed-form pin."""
    W, n_keep, spec = _known_residual_weight(seed=5)
    enc = osl.encode(W, n_keep, 3)
    assert _tail_pin_holds(enc, spec, 3)
    planted = osl.Encoded(**{**enc.__dict__, "tail_energy": enc.R_energy})
    assert not _tail_pin_holds(planted, spec, 3)


def test_zero_sparsity_special_case():
    rng = np.random.default_rng(5)
    W = _rand_bits(rng, (6, 70))
    enc = osl.encode(W, 70, 4)
    assert np.all(enc.keep)
    assert enc.R_energy == 0.0 and np.all(enc.S == 0)
    X = _rand_bits(rng, (3, 70), 1.0)
    Y = osl.forward(X, enc.masks, enc.values, 70, enc.A_cat, enc.B_cat)
    assert np.allclose(Y, ob.bits_to_f64(X) @ ob.bits_to_f64(W).T, rtol=0, atol=1e-14)


# -------------------------------------------------------------- forward -----

def _brute_forward(X_bits, enc, K, lora_A, lora_B, r_svd):
    """Triple loop over set bits for the sparse part; each adapter applied
    separately (no concatenation)."""
    X = ob.bits_to_f64(X_bits)
    M = X.shape[0]
    N = enc.masks.shape[0]
    Y = np.zeros((M, N))
    for n in range(N):
        j = 0
        for c in range(K):
            if (int(enc.masks[n, c // 64]) >> (c % 64)) & 1:
                w = float(ob.bits_to_f64(enc.values[n, j:j + 1])[0])
                j += 1
                for m in range(M):
                    Y[m, n] += X[m, c] * w
    A1 = ob.bits_to_f64(enc.A_cat[:, :r_svd])
    B1 = ob.bits_to_f64(enc.B_cat[:r_svd])
    Y += (X @ A1) @ B1
    for a, b in zip(lora_A, lora_B):
        Y += (X @ ob.bits_to_f64(a).T) @ ob.bits_to_f64(b).T
    return Y


@pytest.mark.parametrize("N,K,M,n_keep,r,lr", [(24, 70, 3, 35, 4, (2, 3)), (16, 64, 5, 20, 3, (4,)),
                                              (10, 129, 2, 100, 0, (1, 1, 1))])
def test_forward_matches_brute_force(N, K, M, n_keep, r, lr):
    rng = np.random.default_rng(N + K + M)
    W = _rand_bits(rng, (N, K))
    As = [_rand_bits(rng, (q, K), 0.01) for q in lr]
    Bs = [_rand_bits(rng, (N, q), 0.01) for q in lr]
    X = _rand_bits(rng, (M, K), 1.0)
    enc = osl.encode(W, n_keep, r, As, Bs)
    assert enc.A_cat.shape == (K, r + sum(lr)) and enc.B_cat.shape == (r + sum(lr), N)
    Y = osl.forward(X, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
    Yb = _brute_forward(X, enc, K, As, Bs, r)
    assert np.max(np.abs(Y - Yb)) <= 1e-12 * max(1.0, np.max(np.abs(Yb)))
    # LoRA blocks are copied bit for bit, in call order
    col = r
    for a, b in zip(As, Bs):
        q = a.shape[0]
        assert np.array_equal(enc.A_cat[:, col:col + q], a.T)
        assert np.array_equal(enc.B_cat[col:col + q], b.T)
        col += q
    rows = np.array([0, N - 1, N // 2])
    assert np.allclose(osl.forward_rows(X, enc.masks, enc.values, K, enc.A_cat, enc.B_cat, rows), Y[:, rows],
                       rtol=0, atol=1e-14)


def test_forward_identity_input():
    """X = I_K gives Y = W_eff^T with W_eff = W_s + (A_cat B_cat)^T."""
    rng = np.random.default_rng(9)
    K, N = 48, 20
    W = _rand_bits(rng, (N, K))
    enc = osl.encode(W, 24, 5, [_rand_bits(rng, (3, K), 0.01)], [_rand_bits(rng, (N, 3), 0.01)])
    eye = ob.f64_to_bits(np.eye(K))
    Y = osl.forward(eye, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
    Weff = np.where(enc.keep, ob.bits_to_f64(W), 0.0) + (ob.bits_to_f64(enc.A_cat) @ ob.bits_to_f64(enc.B_cat)).T
    assert np.allclose(Y, Weff.T, rtol=0, atol=1e-15)


def test_error_metric():
    Y = np.array([[1.0, -2.0, 0.0, 1e-9]])
    assert osl.max_rel_err(Y, Y) == 0.0
    rms = np.sqrt(np.mean(Y * Y))
    Yh = Y.copy()
    Yh[0, 3] += 0.01
    assert abs(osl.max_rel_err(Yh, Y) - 0.01 / rms) < 1e-12
    Yh = Y.copy()
    Yh[0, 1] *= 1.01
    assert abs(osl.max_rel_err(Yh, Y) - 0.01) < 1e-12


# ------------------------------------------------------- fusion ----------

def test_fused_forward_equals_the_parts():
    """A fused encoding computes every part: its forward is the column-wise
    concatenation of the parts' separate forwards (different code: one
    product over stacked arrays against one product per part)."""
    rng = np.random.default_rng(11)
    K, n_keep, M = 192, 97, 5
    parts = []
    for N, r_svd, loras in ((40, 3, (2,)), (16, 0, (5, 1)), (24, 2, ())):
        W = _rand_bits(rng, (N, K))
        As = [_rand_bits(rng, (q, K), 0.01) for q in loras]
        Bs = [_rand_bits(rng, (N, q), 0.01) for q in loras]
        parts.append(osl.encode(W, n_keep, r_svd, As, Bs))
    f = osl.fuse(parts)
    X = _rand_bits(rng, (M, K), 1.0)
    Y = osl.forward(X, f["masks"], f["values"], K, f["A_cat"], f["B_cat"])
    ref = np.concatenate([osl.forward(X, p.masks, p.values, K, p.A_cat, p.B_cat) for p in parts], axis=1)
    assert Y.shape == (M, 80)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)
    # the lookup table of the stack is the stack of the tables
    assert np.array_equal(f["offsets"][40:56], parts[1].offsets)
    # off-diagonal blocks of B_cat hold nothing (ranks 5, 6 and 2 per part)
    B = f["B_cat"]
    assert B.shape == (13, 80)
    assert not B[0:5, 40:].any() and not B[5:11, :40].any() and not B[5:11, 56:].any() and not B[11:, :56].any()


def test_planted_misplaced_block_is_caught():
    """A fusion that puts every part's B block at rank 0 (a plausible
    off-by-offset mistake) fails the forward pin above."""
    rng = np.random.default_rng(12)
    K, n_keep = 128, 64
    parts = [osl.encode(_rand_bits(rng, (N, K)), n_keep, r) for N, r in ((16, 2), (16, 3))]
    f = osl.fuse(parts)
    bad = f["B_cat"].copy()
    bad[:] = 0
    bad[0:2, 0:16] = parts[0].B_cat
    bad[0:3, 16:32] = parts[1].B_cat
    X = _rand_bits(rng, (3, K), 1.0)
    ref = np.concatenate([osl.forward(X, p.masks, p.values, K, p.A_cat, p.B_cat) for p in parts], axis=1)
    Y_bad = osl.forward(X, f["masks"], f["values"], K, f["A_cat"], bad)
    assert not np.allclose(Y_bad, ref, rtol=1e-6, atol=1e-9)
