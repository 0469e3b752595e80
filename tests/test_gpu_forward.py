"""Forward parity: the HIP forward (through the C ABI) against the oracle's
float64 forward on the same encoded layer, element by element.

Small shapes span several tiles and ragged tails in N, K and M on both the
few-row (M <= 16) and many-row kernels, plus the degenerate cases (no
adapters, nothing pruned, everything pruned, one row)."""

import numpy as np
import pytest

from oracle import bf16 as ob
from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits, upload_encoded, wait_error

pytestmark = pytest.mark.gpu

# N, K, n_keep, r_svd, LoRA ranks, token counts
CASES = [
    (512, 512, 256, 16, (8,), (1, 5, 16, 17, 64, 300)),
    (100, 520, 260, 4, (3, 5), (1, 16, 33, 257)),
    (48, 2056, 1000, 0, (), (1, 16, 40)),
    (33, 1024, 1024, 0, (16,), (2, 20)),
    (40, 1032, 0, 0, (8,), (3, 70)),
    (1, 64, 17, 1, (), (1, 30)),
    (200, 3072, 1536, 8, (4, 4, 4), (7, 16, 130)),
    (64, 9216, 4608, 8, (32,), (1, 16, 20)),      # T pieces of 2048 columns, ranges
    (16, 1024, 512, 0, (200,), (4, 16)),          # one workgroup computes 13 T pieces
    (30, 64, 32, 0, (256,), (16,)),               # the largest r_cat, tiny K
    # more than one round of 16-row work (> 256 tiles x ranges): whole rows
    # in several rounds of the one-round kernel (ragged last tile, r_cat not
    # a multiple of 8), and ranged rows on the streaming kernel
    (4200, 2056, 1028, 8, (4,), (1, 16)),
    (4110, 1000, 500, 0, (), (3, 16)),
    (4100, 1024, 0, 0, (8,), (2,)),               # everything pruned
    (1100, 16384, 8192, 0, (40,), (1, 16)),       # ranges in several rounds (too few tiles to stream)
    (3500, 8200, 4100, 0, (12,), (1, 16)),        # streaming: 5 chunks (the last of 8 columns), r_cat 12
    (7000, 4104, 2052, 0, (40,), (1, 16)),        # streaming: two tiles per workgroup, 3 chunks
    (3520, 6144, 6144, 0, (16,), (16,)),          # streaming, nothing pruned: whole chunks of values
    (3600, 5120, 0, 0, (), (5,)),                 # streaming, everything pruned, no adapters
    (4096, 520, 260, 0, (8,), (1, 16)),           # streaming, one-chunk tiles
    (4000, 3000, 1500, 8, (8,), (7, 16)),         # streaming, last chunk ends inside a bitmap word
    # many-token T = X A_cat: 208 padded ranks (16- and 32-token workgroups),
    # 128 ranks with 64-token workgroups over a ragged K
    (64, 1024, 512, 0, (200,), (300, 4100)),
    (64, 1000, 500, 0, (120,), (4100,)),
]


@pytest.fixture(scope="module")
def shared_ws():
    import sparse_rank_linear_amd as srl

    # one workspace for every call in this module: exercises the counter
    # protocol across layer shapes and both token regimes
    shapes = [(N, K, nk, rs, rs + sum(lr), max(ms)) for (N, K, nk, rs, lr, ms) in CASES]
    shapes.append((300, 4096, 2048, 16, 32, 100))  # test_forward_deterministic
    shapes.append((96, 4096, 2048, 8, 32, 16))  # test_forward_clustered_rows
    shapes.append((4096, 1024, 512, 0, 16, 16))  # test_forward_front_loaded_rows
    need = max(srl.query_sizes(*s)["forward_ws_bytes"] for s in shapes)
    return srl.workspace(need)


def _encode_case(N, K, n_keep, r_svd, loras, seed):
    rng = np.random.default_rng(seed)
    W = synth.make_w(N, K, seed)
    As = [ob.f64_to_bits(rng.standard_normal((q, K)).astype(np.float32) * 0.01) for q in loras]
    Bs = [ob.f64_to_bits(rng.standard_normal((N, q)).astype(np.float32) * 0.01) for q in loras]
    return osl.encode(W, n_keep, r_svd, As, Bs)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}_K{c[1]}_keep{c[2]}_r{c[3]}")
def test_forward_matches_oracle(case, shared_ws):
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep, r_svd, loras, Ms = case
    enc = _encode_case(N, K, n_keep, r_svd, loras, seed=N + K)
    layer = upload_encoded(enc, K, r_svd)
    for M in Ms:
        say(f"forward N={N} K={K} n_keep={n_keep} r_cat={layer.r_cat} M={M}")
        X = synth.make_x(K, M, seed=M + 7)
        Y = srl.linear_forward(layer, to_dev(X), ws=shared_ws)
        torch.cuda.synchronize()
        Yref = osl.forward(X, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
        mr, nw = errors(to_host_bits(Y), Yref)
        say(f"  max_rel={mr:.3e} normwise={nw:.3e}")
        assert wait_error(shared_ws) == 0
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


@pytest.mark.parametrize("M", [4, 16, 100])
def test_forward_deterministic(M, shared_ws):
    import torch
    import sparse_rank_linear_amd as srl

    enc = _encode_case(300, 4096, 2048, 16, (16,), seed=3)
    layer = upload_encoded(enc, 4096, 16)
    X = to_dev(synth.make_x(4096, M, seed=5))
    Y1 = srl.linear_forward(layer, X, ws=shared_ws)
    Y2 = srl.linear_forward(layer, X, ws=shared_ws)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


def test_forward_zero_rows_is_noop(shared_ws):
    import torch
    import sparse_rank_linear_amd as srl

    enc = _encode_case(16, 64, 32, 0, (), seed=1)
    layer = upload_encoded(enc, 64, 0)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Y = srl.linear_forward(layer, X, ws=shared_ws)
    assert Y.shape == (0, 16)


def test_forward_rejects_small_workspace():
    import torch
    import sparse_rank_linear_amd as srl

    enc = _encode_case(16, 64, 32, 0, (), seed=1)
    layer = upload_encoded(enc, 64, 0)
    X = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(srl.SalrError, match="WORKSPACE"):
        srl.linear_forward(layer, X, ws=ws)


@pytest.mark.parametrize("M", [1, 16])
def test_forward_clustered_rows(M, shared_ws):
    """Rows whose kept values crowd into one or two 1024-column blocks (very
    uneven counts per block), mixed with ordinary rows in the same tiles."""
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep = 96, 4096, 2048
    W = ob.bits_to_f64(synth.make_w(N, K, seed=21))
    W[1::2, :1024] *= 50.0  # odd rows: every value of block 0 outranks the rest
    W[3::8, 2048:3072] *= 50.0  # some rows: two crowded blocks
    rng = np.random.default_rng(22)
    A = ob.f64_to_bits(rng.standard_normal((24, K)).astype(np.float32) * 0.01)
    B = ob.f64_to_bits(rng.standard_normal((N, 24)).astype(np.float32) * 0.01)
    enc = osl.encode(ob.f64_to_bits(W), n_keep, 8, [A], [B])
    per_block = np.array([[bin(int(w)).count("1") for w in row[:16]] for row in enc.masks[:4]]).sum(axis=1)
    assert per_block[1] >= 900  # block 0 of an odd row is nearly all kept
    layer = upload_encoded(enc, K, 8)
    say(f"forward clustered N={N} K={K} M={M}")
    X = synth.make_x(K, M, seed=23)
    Y = srl.linear_forward(layer, to_dev(X), ws=shared_ws)
    torch.cuda.synchronize()
    Yref = osl.forward(X, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
    mr, nw = errors(to_host_bits(Y), Yref)
    say(f"  max_rel={mr:.3e} normwise={nw:.3e}")
    assert wait_error(shared_ws) == 0
    assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


@pytest.mark.parametrize("M", [1, 16])
def test_forward_front_loaded_rows(M, shared_ws):
    """Whole-row tiles (4096 rows, one round of workgroups) in which every
    seventh row keeps all its values in the first half of the columns, mixed
    with ordinary rows: the waves of the first columns read far more of
    those rows' values than of the others."""
    import torch
    import sparse_rank_linear_amd as srl

    N, K, n_keep = 4096, 1024, 512
    W = ob.bits_to_f64(synth.make_w(N, K, seed=31))
    # every seventh row: the first 512 columns outrank the rest
    W[5::7, :512] = np.sign(W[5::7, :512]) * (np.abs(W[5::7, :512]) + 1.0)
    rng = np.random.default_rng(32)
    A = ob.f64_to_bits(rng.standard_normal((16, K)).astype(np.float32) * 0.01)
    B = ob.f64_to_bits(rng.standard_normal((N, 16)).astype(np.float32) * 0.01)
    enc = osl.encode(ob.f64_to_bits(W), n_keep, 0, [A], [B])
    first = np.array([sum(bin(int(w)).count("1") for w in row[:8]) for row in enc.masks[5:13]])
    assert first[0] == n_keep and first[1] < n_keep  # row 5 front-loaded, row 6 not
    layer = upload_encoded(enc, K, 0)
    say(f"forward front-loaded N={N} K={K} M={M}")
    X = synth.make_x(K, M, seed=33)
    Y = srl.linear_forward(layer, to_dev(X), ws=shared_ws)
    torch.cuda.synchronize()
    Yref = osl.forward(X, enc.masks, enc.values, K, enc.A_cat, enc.B_cat)
    mr, nw = errors(to_host_bits(Y), Yref)
    say(f"  max_rel={mr:.3e} normwise={nw:.3e}")
    assert wait_error(shared_ws) == 0
    assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE
