"""Backward pass on the GPU against the oracle (oracle/backward.py).

salr_transpose_layer: the encoding of W_s^T (bitmap, values padded with +0.0,
lookup table) bit for bit against the oracle's transposed encoding, and
salr_transpose_count against its largest column count; ragged N and K, more
than 1024 rows (several lookup entries per row of W_s^T), nothing kept,
everything kept.  salr_linear_backward: dX, dA_cat and dB_cat against the
oracle's float64 gradients in both token regimes (dX through the few-row and
many-row forward kernels of the transposed layer), with and without adapters,
an empty token sum, and the 4096 x 4096 layer at full size."""

import numpy as np
import pytest

from oracle import backward as obw
from oracle import bf16 as ob
from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits, upload_encoded, wait_error

pytestmark = pytest.mark.gpu


def _encoded(N, K, n_keep, ranks, seed, dist="normal"):
    W = synth.make_w(N, K, seed, dist=dist)
    rng = np.random.default_rng(seed + 1)
    As = [ob.f64_to_bits(rng.standard_normal((q, K)) * 0.01) for q in ranks]
    Bs = [ob.f64_to_bits(rng.standard_normal((N, q)) * 0.01) for q in ranks]
    return osl.encode(W, n_keep, 0, As, Bs)


def errors_f32(got, ref):
    """The forward's error measures for a float32 result."""
    got = np.asarray(got, dtype=np.float64)
    mr = osl.max_rel_err(got, ref)
    nrm = float(np.linalg.norm(ref))
    nw = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    return mr, nw


# N, K, n_keep, weight distribution
TCASES = [(64, 512, 256, "normal"), (104, 520, 260, "t3"), (2056, 200, 100, "normal"), (16, 1000, 0, "normal"),
          (48, 136, 136, "normal"), (1024, 4096, 2048, "normal")]


@pytest.mark.parametrize("case", TCASES, ids=lambda c: f"N{c[0]}_K{c[1]}_keep{c[2]}_{c[3]}")
def test_transpose_matches_oracle(case):
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep, dist = case
    say(f"transpose N={N} K={K} n_keep={n_keep} {dist}")
    enc = _encoded(N, K, n_keep, (), seed=N + 7 * K, dist=dist)
    masks_t, values_t, offsets_t, n_keep_t = obw.transpose_encoding(enc.masks, enc.values, K)
    layer = upload_encoded(enc, K, 0)
    assert srl.transpose_count(layer) == n_keep_t
    lt = srl.transpose_layer(layer)
    torch.cuda.synchronize()
    assert (lt.N, lt.K, lt.n_keep) == (K, N, n_keep_t)
    got = lt.to_numpy()
    assert np.array_equal(got["masks"], masks_t)
    assert np.array_equal(got["offsets"], offsets_t)
    assert np.array_equal(got["values"], values_t)
    # a roomier transposed layer: the same rows, each padded with +0.0 further
    if n_keep_t < N:
        wide = min(n_keep_t + 9, N)
        lt2 = srl.transpose_layer(layer, n_keep=wide)
        torch.cuda.synchronize()
        got2 = lt2.to_numpy()
        assert np.array_equal(got2["masks"], masks_t)
        assert np.array_equal(got2["values"][:, :n_keep_t], values_t)
        assert not got2["values"][:, n_keep_t:].any()


def test_transpose_rejects_small_n_keep():
    import sparse_rank_linear_amd as srl

    enc = _encoded(64, 256, 128, (), seed=3)
    layer = upload_encoded(enc, 256, 0)
    n = srl.transpose_count(layer)
    assert n > 0
    with pytest.raises(srl.SalrError):
        srl.transpose_layer(layer, n_keep=n - 1)


# N, K, n_keep, LoRA ranks, token counts
BCASES = [
    (512, 512, 256, (24,), (1, 5, 16, 17, 64)),
    (104, 520, 260, (3, 5), (1, 16, 33)),
    (64, 2048, 1024, (16,), (3, 100)),
    (1032, 1000, 500, (8,), (16, 20)),
    (40, 1032, 0, (8,), (3, 70)),              # everything pruned
    (256, 256, 128, (), (4, 40)),              # no adapters: dX only
    (4096, 136, 68, (40, 40), (2, 300)),       # W_s^T: 136 rows of 4096 columns
]


@pytest.mark.parametrize("case", BCASES, ids=lambda c: f"N{c[0]}_K{c[1]}_keep{c[2]}_r{sum(c[3])}")
def test_backward_matches_oracle(case):
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep, ranks, Ms = case
    enc = _encoded(N, K, n_keep, ranks, seed=N * 5 + K)
    layer = upload_encoded(enc, K, 0)
    lt = srl.transpose_layer(layer)
    for M in Ms:
        say(f"backward N={N} K={K} n_keep={n_keep} r_cat={layer.r_cat} M={M}")
        X = synth.make_x(K, M, seed=M + 11)
        dY = synth.make_x(N, M, seed=M + 12)
        ws = srl.backward_workspace(layer, lt, M)
        dX, dA, dB = srl.linear_backward(layer, lt, to_dev(X), to_dev(dY), ws=ws)
        torch.cuda.synchronize()
        assert wait_error(ws) == 0
        rX, rA, rB = obw.backward(X, dY, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
        mr, nw = errors(to_host_bits(dX), rX)
        say(f"  dX max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE
        if layer.r_cat:
            # stored layouts: dA [r_cat][K] = (dA_cat)^T, dB [N][r_cat] = (dB_cat)^T
            for name, got, ref in (("dA", dA, rA.T), ("dB", dB, rB.T)):
                mr, nw = errors_f32(got.cpu().numpy(), ref)
                say(f"  {name} max_rel={mr:.3e} normwise={nw:.3e}")
                assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE
        else:
            assert dA.numel() == 0 and dB.numel() == 0


def test_backward_without_dx_and_reused_workspace():
    """dX skipped (a first layer); one workspace over calls of different M
    gives the same gradients as fresh workspaces."""
    import torch
    import sparse_rank_linear_amd as srl

    N, K = 512, 512
    enc = _encoded(N, K, 256, (24,), seed=9)
    layer = upload_encoded(enc, K, 0)
    lt = srl.transpose_layer(layer)
    ws = srl.backward_workspace(layer, lt, 200)
    for M in (200, 7, 64):
        X, dY = to_dev(synth.make_x(K, M, seed=M)), to_dev(synth.make_x(N, M, seed=M + 1))
        dX0, dA0, dB0 = srl.linear_backward(layer, lt, X, dY)
        none, dA1, dB1 = srl.linear_backward(layer, lt, X, dY, ws=ws, need_dx=False)
        torch.cuda.synchronize()
        assert none is None
        assert torch.equal(dA0, dA1) and torch.equal(dB0, dB1)
    assert wait_error(ws) == 0


def test_backward_empty_token_sum():
    import torch
    import sparse_rank_linear_amd as srl

    enc = _encoded(64, 128, 64, (8,), seed=4)
    layer = upload_encoded(enc, 128, 0)
    lt = srl.transpose_layer(layer)
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dA = torch.full((8, 128), 7.0, device="cuda")
    dB = torch.full((64, 8), 7.0, device="cuda")
    dX, dA, dB = srl.linear_backward(layer, lt, X, dY, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert dX.shape == (0, 128)
    assert not dA.any() and not dB.any()


def test_backward_full_size_attention_layer():
    """The 4096 x 4096 layer (50%, r_cat 80) transposed on the GPU and
    differentiated at 16 and 2048 tokens, every gradient entry against the
    oracle."""
    import torch
    import sparse_rank_linear_amd as srl

    wl = synth.WORKLOADS["llama7b_attn_4096"]
    inp = synth.make_inputs(wl, with_x=False)
    keep = osl.select_keep(inp.W, wl.n_keep)
    masks, values = osl.pack_masks(keep), osl.pack_values(inp.W, keep, wl.n_keep)
    a_cat = synth.make_w(wl.r_cat, wl.K, seed=311, scale=0.01)         # [r_cat][K]
    b_cat = synth.make_w(wl.N, wl.r_cat, seed=312, scale=0.01)         # [N][r_cat]
    enc = osl.Encoded(masks, values, osl.block_offsets(keep), a_cat.T.copy(), b_cat.T.copy(), keep,
                      np.zeros(0), 0.0, 0.0)
    layer = upload_encoded(enc, wl.K, 0)
    lt = srl.transpose_layer(layer)
    for M in (16, 2048):
        say(f"backward full size 4096x4096 M={M}")
        X = synth.make_x(wl.K, M, seed=500 + M)
        dY = synth.make_x(wl.N, M, seed=600 + M)
        ws = srl.backward_workspace(layer, lt, M)
        dX, dA, dB = srl.linear_backward(layer, lt, to_dev(X), to_dev(dY), ws=ws)
        torch.cuda.synchronize()
        assert wait_error(ws) == 0
        rX, rA, rB = obw.backward(X, dY, masks, values, wl.K, a_cat.T, b_cat.T)
        for name, mr_nw in (("dX", errors(to_host_bits(dX), rX)), ("dA", errors_f32(dA.cpu().numpy(), rA.T)),
                            ("dB", errors_f32(dB.cpu().numpy(), rB.T))):
            say(f"  {name} max_rel={mr_nw[0]:.3e} normwise={mr_nw[1]:.3e}")
            assert mr_nw[0] <= TOL_MAX_REL and mr_nw[1] <= TOL_NORMWISE
