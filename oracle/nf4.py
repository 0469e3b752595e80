"""QSALR value codec oracle: 4-bit NormalFloat (NF4) quantization of the
packed kept values of W_s.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module; the product path never
imports, calls or links it.

Sources, cited by page title and section:
  [summary]  gist.science technical summary of "Sparsity-Aware Low-Rank
             Representation for Efficient Fine-Tuning of Large Language
             Models", Experimental Results -> Ablation Studies,
             "Quantization": SALR combined with NF4 quantization (QSALR)
             shrinks large models about 5x.
  NF4        the NormalFloat data type of Dettmers et al., "QLoRA: Efficient
             Finetuning of Quantized LLMs" (2023): 16 levels placed at
             quantiles of the standard normal distribution, with an exact
             zero, scaled into [-1, 1], applied per block with the block's
             absolute maximum as scale.  Restated here from that definition.

Readings of what the summary leaves open (each listed in the design doc):
  * What is quantized: the kept values of the frozen base weight (the
    compact value array); the bitmap, lookup table and the trainable
    adapters are unchanged.
  * Levels: 8 positive quantiles at probabilities evenly spaced from
    1 - delta down to 1/2 (1/2 itself, i.e. zero, dropped), 7 negative ones
    at probabilities evenly spaced from 1 - delta to 1/2 (mirrored), and an
    exact 0, where delta = (1/30 + 1/32) / 2; divided by the largest, so the
    extremes are exactly -1 and +1.  Stored as float32 (computed in
    float64).
  * Blocks: 64 consecutive kept values of one row (a row's last block may be
    shorter); scale = the largest |value| of the block, which is a bf16
    value itself and is stored exactly as bf16.
  * Code of a value v with block scale s: the index of the level nearest to
    v / s, everything in float32 (IEEE division and subtraction), ties to
    the lower index; a block whose scale is 0 codes every value as the
    level 0.0.
  * Decoded value: bf16 (round to nearest even) of the float32 product
    level[code] * s.
  * Storage: codes nibble-packed, value 2b in the low and 2b + 1 in the high
    nibble of byte b, each row padded to whole blocks (32 bytes per block);
    scales bf16 [N][blocks per row].
"""

from __future__ import annotations

import numpy as np

from .bf16 import bits_to_f64, f64_to_bits

BLOCK = 64           # kept values per scale block
ZERO_CODE = 7        # index of the level 0.0


def nf4_delta() -> float:
    """Probability mass left beyond the outermost level on each side."""
    return 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels, ascending, float32 (NF4 definition above)."""
    from scipy.stats import norm

    top = 1.0 - nf4_delta()
    pos = norm.ppf(np.linspace(top, 0.5, 9)[:-1])          # 8 positive quantiles
    neg = -norm.ppf(np.linspace(top, 0.5, 8)[:-1])         # 7 negative quantiles
    levels = np.sort(np.concatenate([neg, [0.0], pos]))
    return (levels / levels.max()).astype(np.float32)


def blocks_per_row(n_keep: int) -> int:
    return -(-n_keep // BLOCK)


def block_scales(values: np.ndarray) -> np.ndarray:
    """bf16 scales [N x blocks]: the largest |value| of each block."""
    values = np.asarray(values, dtype=np.uint16)
    N, n = values.shape
    nb = blocks_per_row(n)
    mag = np.zeros((N, nb * BLOCK), dtype=np.float64)
    mag[:, :n] = bits_to_f64(values & np.uint16(0x7FFF))
    return f64_to_bits(mag.reshape(N, nb, BLOCK).max(axis=2))


def quantize(values: np.ndarray):
    """Codes uint8 [N x n_keep] (one per value, unpacked) and bf16 scales
    [N x blocks] of the packed kept values (bf16 bit patterns)."""
    values = np.asarray(values, dtype=np.uint16)
    N, n = values.shape
    levels = nf4_levels()
    scales = block_scales(values)
    s = bits_to_f64(scales).astype(np.float32)
    s_per_value = np.repeat(s, BLOCK, axis=1)[:, :n]
    v = bits_to_f64(values).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = v / s_per_value                                   # float32 division
        dist = np.abs(x[:, :, None] - levels[None, None, :])  # float32
    codes = np.argmin(dist, axis=2).astype(np.uint8)          # first minimum: lower index
    codes[s_per_value == 0] = ZERO_CODE
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [N x n_keep]: round(level[code] * scale) in float32."""
    codes = np.asarray(codes)
    N, n = codes.shape
    levels = nf4_levels()
    s = np.repeat(bits_to_f64(scales).astype(np.float32), BLOCK, axis=1)[:, :n]
    prod = levels[codes.astype(np.int64)] * s                 # float32 product
    return f64_to_bits(prod.astype(np.float64))


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Nibble-packed codes uint8 [N x 32*blocks]: byte b holds value 2b in
    its low nibble and value 2b + 1 in its high nibble; padding codes 0."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, n = codes.shape
    width = blocks_per_row(n) * BLOCK
    full = np.zeros((N, width), dtype=np.uint8)
    full[:, :n] = codes
    return (full[:, 0::2] | (full[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n_keep: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    lo, hi = packed & 0x0F, packed >> 4
    out = np.empty((packed.shape[0], 2 * packed.shape[1]), dtype=np.uint8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out[:, :n_keep]


def forward(X_bits, masks, packed_codes, scales, K: int, n_keep: int, A_cat_bits, B_cat_bits) -> np.ndarray:
    """QSALR forward: the SALR forward on the dequantized values (float64,
    no intermediate rounding)."""
    from . import salr

    values = dequantize(unpack_codes(packed_codes, n_keep), scales)
    return salr.forward(X_bits, masks, values, K, A_cat_bits, B_cat_bits)
