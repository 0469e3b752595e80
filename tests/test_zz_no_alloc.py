"""The allocation-free forward (salr_linear_forward_noalloc) against the
forward with a caller workspace (salr_linear_forward), through the C ABI:
same kernels and launch configurations, so the outputs must be equal bit
for bit, on two calls in a row with the second on a smaller input, in both
token regimes; a layer and token count whose workspace exceeds the fixed
array is rejected before any launch."""

import numpy as np
import pytest

from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits, upload_encoded

pytestmark = pytest.mark.gpu


def _layer(N, K, n_keep, r_svd, ranks, seed):
    rng = np.random.default_rng(seed)
    W = synth.make_w(N, K, seed)
    As = [synth._to_bf16_bits(rng.standard_normal((q, K), dtype=np.float32) * np.float32(0.01)) for q in ranks]
    Bs = [synth._to_bf16_bits(rng.standard_normal((N, q), dtype=np.float32) * np.float32(0.01)) for q in ranks]
    enc = osl.encode(W, n_keep, r_svd, As, Bs)
    return enc, upload_encoded(enc, K, r_svd)


# N, K, n_keep, r_svd, LoRA ranks, (first M, smaller second M)
CASES = [
    (512, 512, 256, 16, (8,), (16, 3)),          # few-row kernel
    (4200, 2056, 1028, 8, (4,), (16, 1)),        # few-row kernel, several rounds
    (3500, 8200, 4100, 0, (12,), (16, 5)),       # streaming kernel
    (300, 4096, 2048, 16, (16,), (300, 40)),     # many-row kernel
    (64, 4096, 2048, 4, (8,), (1000, 16)),       # many-row K splits, then few-row
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}_K{c[1]}_M{c[5][0]}-{c[5][1]}")
def test_noalloc_matches_workspace_forward(case):
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep, r_svd, ranks, (M1, M2) = case
    enc, layer = _layer(N, K, n_keep, r_svd, ranks, seed=N + K)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for M in (M1, M2):
        say(f"noalloc N={N} K={K} r_cat={layer.r_cat} M={M}")
        X = synth.make_x(K, M, seed=M + 1)
        Xd = to_dev(X)
        ws = srl.forward_workspace(layer, M)
        Y_ref = srl.linear_forward(layer, Xd, ws=ws)
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        srl.linear_forward_noalloc(layer, Xd, Y, wait_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0 and srl.wait_error(ws) == 0
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), "differs from salr_linear_forward"
        mr, nw = errors(to_host_bits(Y), osl.forward(X, enc.masks, enc.values, K, enc.A_cat, enc.B_cat))
        say(f"  equal to the workspace forward; vs oracle max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def test_noalloc_rejects_oversized_workspace():
    import torch
    import sparse_rank_linear_amd as srl

    # r_cat 256 at 70000 tokens: the many-row T partials alone exceed 64 MiB
    N, K = 64, 64
    layer = srl.SalrLayer.empty(N, K, 32, 0, 256)
    assert srl.query_sizes(N, K, 32, 0, 256, 70000)["forward_ws_bytes"] > srl.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((70000, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((70000, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(srl.SalrError, match="WORKSPACE"):
        srl.linear_forward_noalloc(layer, X, Y)
