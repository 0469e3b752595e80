"""Pins of the NF4 value-codec oracle (oracle/nf4.py) to things other than
itself: the defining equal-probability placement of the levels checked with
the normal CDF (a different routine from the quantile function that builds
them), brute force on tiny inputs, exact round trips of level points, the
quantization error bound, and planted mistakes that these pins catch."""

import numpy as np
import pytest
from scipy.stats import norm

from oracle import bf16 as ob
from oracle import nf4
from oracle import salr as osl
from sparse_rank_linear_amd import synth


def _cdf_spacing_holds(levels) -> bool:
    """NF4 definition: the positive levels sit at CDF values evenly spaced
    from 1 - delta (the largest, +1) down to 1/2 in 8 steps, the negative ones
    mirror 7 steps, and 0 is a level."""
    levels = np.asarray(levels, dtype=np.float64)
    if levels.shape != (16,) or not np.all(np.diff(levels) > 0):
        return False
    z = norm.ppf(1.0 - nf4.nf4_delta())
    pos = levels[levels > 0]
    neg = levels[levels < 0]
    if pos.size != 8 or neg.size != 7 or not np.any(levels == 0.0):
        return False
    top = 1.0 - nf4.nf4_delta()
    p_pos = norm.cdf(pos * z)[::-1]            # descending from top
    p_neg = norm.cdf(-neg * z)                 # mirrored, descending from top
    want_pos = top - np.arange(8) * (top - 0.5) / 8
    want_neg = top - np.arange(7) * (top - 0.5) / 7
    return bool(np.allclose(p_pos, want_pos, atol=2e-7) and np.allclose(p_neg, want_neg, atol=2e-7))


def test_levels_structure_and_cdf_spacing():
    L = nf4.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert L[0] == -1.0 and L[nf4.ZERO_CODE] == 0.0 and L[15] == 1.0
    assert _cdf_spacing_holds(L)
    # the delta of the definition: half of 1/30 + 1/32
    assert abs(nf4.nf4_delta() - 0.0322916666) < 1e-9


def test_planted_symmetric_levels_are_caught():
    """Levels of a symmetric 16-quantile construction (no exact zero, equal
    counts per side) must fail the CDF pin."""
    top = 1.0 - nf4.nf4_delta()
    v = norm.ppf(np.linspace(1.0 - top, top, 16))
    wrong = (v / v.max()).astype(np.float32)
    assert not _cdf_spacing_holds(wrong)
    # and levels built with the wrong delta
    v = np.sort(np.concatenate([norm.ppf(np.linspace(0.99, 0.5, 9)[:-1]), [0.0],
                                -norm.ppf(np.linspace(0.99, 0.5, 8)[:-1])]))
    assert not _cdf_spacing_holds((v / v.max()).astype(np.float32))


def _brute_quantize(values):
    """Value by value with Python loops: scale = max |v| of the block,
    x = float32(v) / float32(s), nearest level by a strict-less scan."""
    L = [np.float32(x) for x in nf4.nf4_levels()]
    N, n = values.shape
    codes = np.zeros((N, n), dtype=np.uint8)
    scales = np.zeros((N, -(-n // 64)), dtype=np.uint16)
    for r in range(N):
        for b0 in range(0, n, 64):
            blk = [float(ob.bits_to_f64(np.array([values[r, j]], dtype=np.uint16))[0]) for j in range(b0, min(n, b0 + 64))]
            s = max(abs(v) for v in blk)
            scales[r, b0 // 64] = ob.f64_to_bits(np.array([s]))[0]
            for k, v in enumerate(blk):
                if s == 0.0:
                    codes[r, b0 + k] = nf4.ZERO_CODE
                    continue
                x = np.float32(v) / np.float32(s)
                best, bd = 0, None
                for j, lv in enumerate(L):
                    d = abs(np.float32(x - lv))
                    if bd is None or d < bd:
                        best, bd = j, d
                codes[r, b0 + k] = best
    return codes, scales


@pytest.mark.parametrize("N,n,seed", [(3, 64, 1), (2, 150, 2), (4, 7, 3)])
def test_quantize_matches_brute_force(N, n, seed):
    rng = np.random.default_rng(seed)
    v = ob.f64_to_bits(rng.standard_normal((N, n)) * 0.02)
    v[0, :5] = [0x8000, 0x0000, 0x0001, 0x8003, 0x3C00]   # signed zeros, subnormals, 1/128
    if N > 2:
        v[2, :] = 0                                          # an all-zero block
    codes, scales = nf4.quantize(v)
    bc, bs = _brute_quantize(v)
    assert np.array_equal(codes, bc)
    assert np.array_equal(scales, bs)
    assert np.all(codes[2] == nf4.ZERO_CODE) if N > 2 else True


def test_no_bf16_value_is_equidistant_from_two_levels():
    """The tie rule (lower index) never decides a code: for every finite
    bf16 value v and bf16 scales s in [1, 2) (so, scaling by powers of two,
    any normal scale), float32 |v/s - level| has a unique minimum.  Checked
    on every 8th scale mantissa here (all 128 were checked once)."""
    L = nf4.nf4_levels()
    pos = np.arange(0x0000, 0x7F80, dtype=np.uint32).astype(np.uint16)
    vb = np.concatenate([pos, pos | np.uint16(0x8000)])
    v = ob.bits_to_f64(vb).astype(np.float32)
    for sb in range(0x3F80, 0x4000, 8):
        s = np.float32(ob.bits_to_f64(np.array([sb], dtype=np.uint16))[0])
        x = v[np.abs(v) <= s] / s
        d = np.abs(x[:, None] - L[None, :])
        assert np.all((d == d.min(axis=1, keepdims=True)).sum(axis=1) == 1), hex(sb)


def test_level_points_round_trip_exactly():
    rng = np.random.default_rng(9)
    N, n = 5, 200
    codes = rng.integers(0, 16, size=(N, n)).astype(np.uint8)
    codes[:, ::64] = 15                                     # every block holds +1 * s
    s = ob.f64_to_bits(np.exp(rng.uniform(-9, 0, size=(N, -(-n // 64)))))
    vals = nf4.dequantize(codes, s)
    c2, s2 = nf4.quantize(vals)
    assert np.array_equal(s2, s)
    assert np.array_equal(c2, codes)
    assert np.array_equal(nf4.unpack_codes(nf4.pack_codes(codes), n), codes)


def test_quantization_error_bound():
    """|dequant(quant(v)) - v| <= s * (largest half gap between levels) plus
    the bf16 rounding of the product (half an ulp: |.| * 2^-8)."""
    L = nf4.nf4_levels().astype(np.float64)
    half_gap = np.max(np.diff(L)) / 2
    W = synth.make_w(64, 512, seed=4, dist="t3")
    vals = osl.pack_values(W, osl.select_keep(W, 256), 256)
    codes, scales = nf4.quantize(vals)
    back = ob.bits_to_f64(nf4.dequantize(codes, scales))
    v = ob.bits_to_f64(vals)
    s = np.repeat(ob.bits_to_f64(scales), 64, axis=1)[:, :256]
    assert np.all(np.abs(back - v) <= s * (half_gap * (1 + 1e-6)) + np.abs(back) * 2.0 ** -8)
    # the per-block maximum is reproduced exactly (code +-1)
    assert np.all(np.max(np.abs(back).reshape(64, 4, 64), axis=2) == ob.bits_to_f64(scales))


def test_pack_layout_hand_example():
    codes = np.array([[1, 2, 3, 15, 0]], dtype=np.uint8)
    p = nf4.pack_codes(codes)
    assert p.shape == (1, 32)
    assert list(p[0, :3]) == [0x21, 0xF3, 0x00]
    assert np.all(p[0, 3:] == 0)


def test_forward_on_exact_values_equals_salr_forward():
    """Values that are level points stay bit-exact through the codec, so the
    QSALR forward equals the SALR forward on them."""
    rng = np.random.default_rng(2)
    N, K, n_keep, M = 24, 128, 64, 3
    codes = rng.integers(0, 16, size=(N, n_keep)).astype(np.uint8)
    codes[:, 0] = 0                                           # -1 * s in every block
    scales = ob.f64_to_bits(np.full((N, 1), 0.03125))
    vals = nf4.dequantize(codes, scales)
    keep = np.zeros((N, K), dtype=bool)
    for r in range(N):
        keep[r, np.sort(rng.choice(K, n_keep, replace=False))] = True
    masks = osl.pack_masks(keep)
    X = ob.f64_to_bits(rng.standard_normal((M, K)))
    A = ob.f64_to_bits(rng.standard_normal((K, 4)) * 0.01)
    B = ob.f64_to_bits(rng.standard_normal((4, N)) * 0.01)
    c2, s2 = nf4.quantize(vals)
    Y = nf4.forward(X, masks, nf4.pack_codes(c2), s2, K, n_keep, A, B)
    assert np.array_equal(Y, osl.forward(X, masks, vals, K, A, B))


def test_bytes_per_weight_at_half_sparsity():
    """Bitmap (1/8 B) + codes (1/2 B per kept value) + scales (2 B per 64
    kept values) per weight element at s = 0.5: about 0.39 B, vs 1.125 B
    for bf16 values."""
    K, n_keep = 4096, 2048
    b = K / 8 + n_keep / 2 + 2 * nf4.blocks_per_row(n_keep)
    assert abs(b / K - 0.3906) < 1e-3
