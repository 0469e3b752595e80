"""QSALR (NF4 values) on the GPU against the oracle (oracle/nf4.py).

salr_quantize_nf4: codes and scales bit for bit against the oracle's
quantization of the same kept values (signed zeros, subnormal and all-zero
blocks, ragged last blocks included).  Forward on NF4 layers: the oracle's
codes and scales uploaded, both token regimes (the few-row kernel with its
LDS dequantization, whole rows and column ranges, one and several rounds;
the many-row kernel on dequantized values), against the oracle's float64
forward of the dequantized layer; end to end GPU encode -> GPU quantize ->
GPU forward; the 4096 x 4096 layer at full size."""

import numpy as np
import pytest

from oracle import bf16 as ob
from oracle import nf4
from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits, upload_encoded, wait_error

pytestmark = pytest.mark.gpu


def _weights(N, K, seed, kind="normal"):
    if kind == "special":
        rng = np.random.default_rng(seed)
        W = synth.make_w(N, K, seed)
        W[0, : K // 2] = 0x8000                                    # -0.0 kept in row 0's first blocks
        W[1] = rng.integers(1, 0x80, size=K).astype(np.uint16)     # a row of subnormals
        W[2] = 0                                                   # an all-zero row
        return W
    return synth.make_w(N, K, seed, dist=kind)


def _encoded(N, K, n_keep, ranks, seed, kind="normal"):
    W = _weights(N, K, seed, kind)
    rng = np.random.default_rng(seed + 1)
    As = [ob.f64_to_bits(rng.standard_normal((q, K)) * 0.01) for q in ranks]
    Bs = [ob.f64_to_bits(rng.standard_normal((N, q)) * 0.01) for q in ranks]
    return W, osl.encode(W, n_keep, 0, As, Bs)


def _upload_nf4(enc, K, codes, scales):
    """An NF4 layer from the oracle's encoding and the oracle's codes."""
    import torch
    import sparse_rank_linear_amd as srl

    layer = upload_encoded(enc, K, 0)
    sz = srl.query_sizes(layer.N, K, layer.n_keep, 0, layer.r_cat, 0)
    packed = nf4.pack_codes(codes)
    layer.codes = torch.zeros(sz["codes_bytes"], dtype=torch.uint8, device="cuda")
    layer.codes[: packed.size].copy_(torch.from_numpy(packed.reshape(-1)))
    layer.scales = torch.zeros(sz["scales_bytes"] // 2, dtype=torch.int16, device="cuda")
    layer.scales[: scales.size].copy_(torch.from_numpy(scales.reshape(-1).view(np.int16)))
    layer.value_format = srl.binding.VALUES_NF4
    return layer


# N, K, n_keep, weight kind
QCASES = [(64, 512, 256, "normal"), (40, 1000, 333, "t3"), (16, 4096, 2048, "special"), (7, 200, 1, "normal"),
          (33, 1024, 1024, "normal")]


@pytest.mark.parametrize("case", QCASES, ids=lambda c: f"N{c[0]}_K{c[1]}_keep{c[2]}_{c[3]}")
def test_quantize_matches_oracle(case):
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep, kind = case
    say(f"quantize N={N} K={K} n_keep={n_keep} {kind}")
    _, enc = _encoded(N, K, n_keep, (), seed=N + K, kind=kind)
    layer = upload_encoded(enc, K, 0)
    srl.quantize_nf4(layer)
    torch.cuda.synchronize()
    codes, scales = nf4.quantize(enc.values)
    packed = nf4.pack_codes(codes)
    got_c = layer.codes.cpu().numpy()[: packed.size].reshape(packed.shape)
    got_s = layer.scales.cpu().numpy().view(np.uint16)[: scales.size].reshape(scales.shape)
    assert np.array_equal(got_s, scales)
    assert np.array_equal(got_c, packed)


# N, K, n_keep, LoRA ranks, token counts
FCASES = [
    (512, 512, 256, (24,), (1, 5, 16, 17, 64)),
    (100, 520, 260, (3, 5), (1, 16, 33)),
    (64, 9216, 4608, (32,), (1, 16, 20)),       # rows cut into 2048-column ranges
    (4200, 2056, 1028, (12,), (1, 16)),         # several rounds of whole rows
    (1100, 16384, 8192, (40,), (2, 16)),        # ranges in several rounds
    (16, 4096, 2048, (), (16, 300)),            # special values, no adapters
    (40, 1032, 0, (8,), (3, 70)),               # everything pruned
]


@pytest.mark.parametrize("case", FCASES, ids=lambda c: f"N{c[0]}_K{c[1]}_keep{c[2]}")
def test_nf4_forward_matches_oracle(case):
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep, ranks, Ms = case
    kind = "special" if N == 16 and K == 4096 else "normal"
    _, enc = _encoded(N, K, n_keep, ranks, seed=N * 3 + K, kind=kind)
    codes, scales = nf4.quantize(enc.values)
    layer = _upload_nf4(enc, K, codes, scales)
    packed = nf4.pack_codes(codes)
    for M in Ms:
        say(f"nf4 forward N={N} K={K} n_keep={n_keep} r_cat={layer.r_cat} M={M}")
        X = synth.make_x(K, M, seed=M + 3)
        ws = srl.forward_workspace(layer, M)
        Y = srl.linear_forward(layer, to_dev(X), ws=ws)
        torch.cuda.synchronize()
        assert wait_error(ws) == 0
        Yref = nf4.forward(X, enc.masks, packed, scales, K, n_keep, enc.A_cat, enc.B_cat)
        mr, nw = errors(to_host_bits(Y), Yref)
        say(f"  max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def test_nf4_end_to_end():
    """GPU encode -> GPU quantize -> GPU forward against oracle encode ->
    oracle quantize -> oracle forward (residual SVD omitted: the LoRA blocks
    are copied bit for bit)."""
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep = 512, 512, 256
    W, enc = _encoded(N, K, n_keep, (16,), seed=5)
    rng = np.random.default_rng(6)
    As = [ob.f64_to_bits(rng.standard_normal((16, K)) * 0.01)]
    Bs = [ob.f64_to_bits(rng.standard_normal((N, 16)) * 0.01)]
    enc = osl.encode(W, n_keep, 0, As, Bs)
    layer, _ = srl.encode(to_dev(W), n_keep, 0, [to_dev(a) for a in As], [to_dev(b) for b in Bs])
    srl.quantize_nf4(layer)
    codes, scales = nf4.quantize(enc.values)
    for M in (16, 100):
        X = synth.make_x(K, M, seed=M)
        Y = srl.linear_forward(layer, to_dev(X))
        torch.cuda.synchronize()
        Yref = nf4.forward(X, enc.masks, nf4.pack_codes(codes), scales, K, n_keep, enc.A_cat, enc.B_cat)
        mr, nw = errors(to_host_bits(Y), Yref)
        say(f"nf4 end to end M={M}: max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def test_nf4_full_size_attention_layer():
    """The 4096 x 4096 layer (50%, r_cat 80 with seeded adapters) in NF4 at
    1 and 16 tokens, every output against the oracle, plus 2048 tokens on
    sampled rows."""
    import torch
    import sparse_rank_linear_amd as srl

    wl = synth.WORKLOADS["llama7b_attn_4096"]
    inp = synth.make_inputs(wl, with_x=False)
    keep = osl.select_keep(inp.W, wl.n_keep)
    masks, values = osl.pack_masks(keep), osl.pack_values(inp.W, keep, wl.n_keep)
    codes, scales = nf4.quantize(values)
    packed = nf4.pack_codes(codes)
    a_cat = synth.make_w(wl.r_cat, wl.K, seed=301, scale=0.01)         # [r_cat][K]
    b_cat = synth.make_w(wl.N, wl.r_cat, seed=302, scale=0.01)         # [N][r_cat]
    enc = osl.Encoded(masks, values, osl.block_offsets(keep), a_cat.T.copy(), b_cat.T.copy(), keep,
                      np.zeros(0), 0.0, 0.0)
    layer = _upload_nf4(enc, wl.K, codes, scales)
    for M in (1, 16, 2048):
        X = synth.make_x(wl.K, M, seed=400 + M)
        ws = srl.forward_workspace(layer, M)
        Y = srl.linear_forward(layer, to_dev(X), ws=ws)
        torch.cuda.synchronize()
        assert wait_error(ws) == 0
        rows = np.arange(wl.N) if M <= 16 else np.sort(np.random.default_rng(M).choice(wl.N, 64, replace=False))
        Yref = nf4.forward(X, masks[rows], packed[rows], scales[rows], wl.K, wl.n_keep, a_cat.T, b_cat[rows].T)
        mr, nw = errors(to_host_bits(Y[:, torch.from_numpy(rows).cuda()]), Yref)
        say(f"nf4 full size M={M}: {len(rows)} rows max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE
