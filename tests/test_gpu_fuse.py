"""Multi-projection fusion on the GPU (salr_fuse_layers through the C ABI):
the fused encoding must equal the oracle's fusion of the same parts byte
for byte, and a forward on it must match the oracle's forward of the fused
encoding (which the CPU pins tie to the parts' separate forwards)."""

import numpy as np
import pytest

from oracle import bf16 as ob
from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits, upload_encoded, wait_error

pytestmark = pytest.mark.gpu

# (K, n_keep, [(N, r_svd, LoRA ranks) per part], token counts)
CASES = [
    (512, 256, [(64, 4, (4,)), (16, 2, ()), (48, 0, (3, 2))], (1, 16, 40)),      # ragged ranks, small
    (2048, 1024, [(1024, 16, (8,)), (256, 8, (8,)), (256, 8, (8,))], (1, 16, 300)),  # q/k/v-like
    (1032, 500, [(200, 0, (8,)), (200, 0, (8,))], (3, 16, 64)),                   # gate/up-like, ragged K
    (4096, 2048, [(80, 0, ()), (48, 0, ())], (16,)),                              # no adapters at all
    (1024, 400, [(256, 32, (8,)), (512, 0, (8,)), (128, 48, (8,)), (64, 0, ())], (1, 5, 16, 48)),  # rank windows
]


def _part(N, K, n_keep, r_svd, loras, seed):
    rng = np.random.default_rng(seed)
    W = synth.make_w(N, K, seed)
    As = [ob.f64_to_bits(rng.standard_normal((q, K)).astype(np.float32) * 0.01) for q in loras]
    Bs = [ob.f64_to_bits(rng.standard_normal((N, q)).astype(np.float32) * 0.01) for q in loras]
    return osl.encode(W, n_keep, r_svd, As, Bs)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"K{c[0]}_parts{len(c[2])}")
def test_fuse_matches_oracle(case):
    import sparse_rank_linear_amd as srl

    K, n_keep, specs, Ms = case
    parts = [_part(N, K, n_keep, rs, lr, seed=100 * i + N) for i, (N, rs, lr) in enumerate(specs)]
    layers = [upload_encoded(p, K, rs) for p, (N, rs, lr) in zip(parts, specs)]
    say(f"fuse K={K} n_keep={n_keep} parts={[(l.N, l.r_cat) for l in layers]}")
    fused = srl.fuse(layers)
    ref = osl.fuse(parts)
    got = fused.to_numpy()
    assert fused.N == sum(l.N for l in layers) and fused.r_cat == sum(l.r_cat for l in layers)
    assert np.array_equal(got["masks"], ref["masks"])
    assert np.array_equal(got["values"], ref["values"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["a_cat"], ref["A_cat"].T)
    assert np.array_equal(got["b_cat"], ref["B_cat"].T)
    assert fused.parts == tuple((l.N, l.r_cat) for l in layers)

    ws = srl.forward_workspace(fused, max(Ms))
    for M in Ms:
        say(f"fused forward K={K} N={fused.N} r_cat={fused.r_cat} M={M}")
        X = synth.make_x(K, M, seed=M + 3)
        Y = srl.linear_forward(fused, to_dev(X), ws=ws)
        Yref = osl.forward(X, ref["masks"], ref["values"], K, ref["A_cat"], ref["B_cat"])
        mr, nw = errors(to_host_bits(Y), Yref)
        assert wait_error(ws) == 0
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE, (M, mr, nw)


def test_fuse_of_a_fused_layer_records_the_inner_parts():
    """Fusing a fused layer keeps its parts: the record lists the innermost
    parts in row order, and the forward still matches the oracle."""
    import sparse_rank_linear_amd as srl

    K, n_keep = 512, 200
    specs = [(128, 8, ()), (64, 0, (8,)), (96, 16, (8,))]
    parts = [_part(N, K, n_keep, rs, lr, seed=7 + i) for i, (N, rs, lr) in enumerate(specs)]
    layers = [upload_encoded(p, K, rs) for p, (N, rs, lr) in zip(parts, specs)]
    inner = srl.fuse(layers[:2])
    outer = srl.fuse([inner, layers[2]])
    assert outer.parts == ((128, 8), (64, 8), (96, 24))
    ref = osl.fuse(parts)
    ws = srl.forward_workspace(outer, 16)
    X = synth.make_x(K, 16, seed=11)
    say(f"nested fuse K={K} N={outer.N} r_cat={outer.r_cat} M=16")
    Y = srl.linear_forward(outer, to_dev(X), ws=ws)
    Yref = osl.forward(X, ref["masks"], ref["values"], K, ref["A_cat"], ref["B_cat"])
    mr, nw = errors(to_host_bits(Y), Yref)
    assert wait_error(ws) == 0
    assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE, (mr, nw)


@pytest.mark.parametrize("M", [16, 2048])
def test_fused_qkv_full_size_against_the_parts(M):
    """The Llama-7B q/k/v projections (3 x 4096 x 4096, r_cat 3 x 80) fused
    at full size: every sampled output row must match the oracle's forward
    of its own part (the oracle's own encoding of that part's rows, seeded
    adapters), so the rank windows of the few-row (M = 16) and many-row
    (M = 2048) kernels are checked at the size the bench times."""
    import torch
    import sparse_rank_linear_amd as srl

    wl = synth.WORKLOADS["llama7b_attn_4096"]
    N, K, n_keep = wl.N, wl.K, wl.n_keep
    rng = np.random.default_rng(77)
    layers, refs = [], []
    for p in range(3):
        W = synth.make_w(N, K, seed=wl.seed + 30 + p)
        a_cat = synth.make_w(wl.r_cat, K, seed=wl.seed + 40 + p, scale=0.01)   # [r][K]
        b_cat = synth.make_w(N, wl.r_cat, seed=wl.seed + 50 + p, scale=0.01)   # [N][r]
        enc, _ = srl.encode(to_dev(W), n_keep, 0)
        layer = srl.SalrLayer.empty(N, K, n_keep, wl.r_svd, wl.r_cat)
        for f in ("masks", "values", "offsets"):
            getattr(layer, f).copy_(getattr(enc, f))
        layer.a_cat.view(torch.int16).copy_(torch.from_numpy(a_cat.view(np.int16)))
        layer.b_cat.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(b_cat).view(np.int16)))
        rows = np.unique(np.concatenate([rng.choice(N, 10, replace=False), [0, N - 1]]))
        keep = osl.select_keep(W[rows], n_keep)
        refs.append((rows, osl.pack_masks(keep), osl.pack_values(W[rows], keep, n_keep), a_cat, b_cat[rows]))
        layers.append(layer)
        del enc
    fused = srl.fuse(layers)
    assert fused.parts == ((N, wl.r_cat),) * 3
    del layers
    X = synth.make_x(K, M, seed=wl.seed + 60 + M)
    say(f"fused q/k/v full size: N={fused.N} K={K} r_cat={fused.r_cat} M={M}")
    ws = srl.forward_workspace(fused, M)
    Y = srl.linear_forward(fused, to_dev(X), ws=ws)
    torch.cuda.synchronize()
    assert wait_error(ws) == 0
    tok = np.arange(M) if M <= 256 else np.sort(np.random.default_rng(M).choice(M, 256, replace=False))
    for p, (rows, m_o, v_o, a_cat, b_rows) in enumerate(refs):
        cols = torch.from_numpy(p * N + rows).cuda()
        Yg = to_host_bits(Y[torch.from_numpy(tok).cuda()][:, cols])
        Yref = osl.forward(X[tok], m_o, v_o, K, a_cat.T, b_rows.T)
        mr, nw = errors(Yg, Yref)
        say(f"  part {p}: {len(tok)} tokens x {len(rows)} rows: max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE, (p, mr, nw)
