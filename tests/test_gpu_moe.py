"""Grouped (mixture-of-experts) forward on the GPU against the oracle
(oracle/moe.py).

Each expert's encoding comes from the oracle and is uploaded into the
stacked buffers at the library's strides; the expert row boundaries live on
the device.  Cases: empty experts, one-token groups, more than 64 rows for
one expert (two passes over its tiles), ragged N (a partial row tile) and K
(a partial 1024-column chunk, a partial bitmap word), everything pruned,
nothing pruned, no adapters, a rank that is not a multiple of 8, one
expert; then the Mixtral-8x7B expert shape (8 x 14336 x 4096, 32 routed rows)
and the DeepSeek-V2-Lite expert shape (64 x 1408 x 2048, 96 routed rows) at
full size."""

import numpy as np
import pytest

from oracle import bf16 as ob
from oracle import moe as omoe
from oracle import salr as osl
from sparse_rank_linear_amd import synth
from tests.gpu_util import TOL_MAX_REL, TOL_NORMWISE, errors, say, to_dev, to_host_bits

pytestmark = pytest.mark.gpu


def _experts(E, N, K, n_keep, r, seed, scale=0.02):
    """E oracle encodings (each its own weight and LoRA pair)."""
    rng = np.random.default_rng(seed)
    out = []
    for e in range(E):
        W = synth.make_w(N, K, seed * 100 + e, scale=scale)
        As = [ob.f64_to_bits(rng.standard_normal((r, K)) * 0.01)] if r else []
        Bs = [ob.f64_to_bits(rng.standard_normal((N, r)) * 0.01)] if r else []
        out.append(osl.encode(W, n_keep, 0, As, Bs))
    return out


def _upload(encs, N, K, n_keep, r):
    import sparse_rank_linear_amd as srl

    moe = srl.SalrMoE.empty(len(encs), N, K, n_keep, r)
    for e, en in enumerate(encs):
        moe.set_expert(e, en.masks, en.values, en.offsets, en.A_cat.T.copy(), en.B_cat.T.copy())
    return moe


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _run(moe, X, off, m_cap=0):
    import torch
    import sparse_rank_linear_amd as srl

    d_off = torch.from_numpy(off).cuda()
    Y = srl.moe_forward(moe, to_dev(X), d_off, m_cap=m_cap)
    torch.cuda.synchronize()
    return to_host_bits(Y)


# E, N, K, n_keep, rank, rows per expert
CASES = [
    (4, 128, 512, 256, 24, (3, 0, 17, 64)),
    (8, 200, 1000, 500, 8, (1, 2, 3, 4, 0, 0, 70, 5)),
    (3, 64, 3072, 0, 16, (5, 5, 5)),
    (2, 96, 2048, 2048, 0, (16, 33)),
    (3, 48, 256, 100, 12, (7, 20, 1)),
    (1, 520, 1088, 544, 32, (40,)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"E{c[0]}_N{c[1]}_K{c[2]}_keep{c[3]}_r{c[4]}")
def test_moe_forward_matches_oracle(case):
    E, N, K, n_keep, r, counts = case
    say(f"moe E={E} N={N} K={K} n_keep={n_keep} r={r} rows={counts}")
    encs = _experts(E, N, K, n_keep, r, seed=E + N + K)
    moe = _upload(encs, N, K, n_keep, r)
    off = _offsets(counts)
    X = synth.make_x(K, int(off[-1]), seed=N)
    experts = [(en.masks, en.values, en.A_cat, en.B_cat) for en in encs]
    Yref = omoe.grouped_forward(X, off, experts, K)
    for m_cap in (0, 1):  # (the low-rank grid from T, or one 64-row block per expert and a grid-stride loop)
        Y = _run(moe, X, off, m_cap)
        mr, nw = errors(Y, Yref)
        say(f"  m_cap={m_cap} max_rel={mr:.3e} normwise={nw:.3e}")
        assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def test_moe_expert_view_runs_the_single_layer_forward():
    """salr_moe_expert's descriptor is a working layer: the single-layer
    forward on expert 1's view matches the oracle on that expert."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import binding as B

    E, N, K, n_keep, r = 3, 256, 1024, 512, 16
    encs = _experts(E, N, K, n_keep, r, seed=5)
    moe = _upload(encs, N, K, n_keep, r)
    view = moe.expert(1)
    X = synth.make_x(K, 20, seed=3)
    Xd = to_dev(X)
    Y = torch.empty((20, N), dtype=torch.bfloat16, device="cuda")
    ws = srl.workspace(srl.query_sizes(N, K, n_keep, 0, r, 20)["forward_ws_bytes"])
    st = srl.lib().salr_linear_forward(B.C.byref(view), B.C.c_void_p(Xd.data_ptr()), 20,
                                       B.C.c_void_p(Y.data_ptr()), B.C.c_void_p(ws.data_ptr()), ws.numel(),
                                       B._stream_ptr(None))
    assert st == 0
    torch.cuda.synchronize()
    en = encs[1]
    mr, nw = errors(to_host_bits(Y), osl.forward(X, en.masks, en.values, K, en.A_cat, en.B_cat))
    assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def test_moe_malformed_offsets_stay_in_bounds():
    """Boundaries outside [0, T] are clamped on the device: the groups they
    still describe are right, and nothing is written outside Y (also when
    decreasing boundaries make two groups overlap)."""
    import torch
    import sparse_rank_linear_amd as srl

    E, N, K, n_keep, r = 3, 64, 512, 256, 8
    encs = _experts(E, N, K, n_keep, r, seed=8)
    moe = _upload(encs, N, K, n_keep, r)
    T = 10
    X = synth.make_x(K, T, seed=4)
    experts = [(en.masks, en.values, en.A_cat, en.B_cat) for en in encs]
    for bad, good in (((-5, 4, 4, 1000), (0, 4, 4, T)), ((0, 6, 4, 1000), None)):
        guard = torch.full((T + 8, N), 3.0, dtype=torch.bfloat16, device="cuda")
        Y = guard[4:4 + T]
        srl.moe_forward(moe, to_dev(X), torch.tensor(bad, dtype=torch.int32, device="cuda"), Y=Y)
        torch.cuda.synchronize()
        assert torch.all(guard[:4] == 3.0) and torch.all(guard[4 + T:] == 3.0)
        if good is not None:
            mr, nw = errors(to_host_bits(Y), omoe.grouped_forward(X, good, experts, K))
            assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def _full_size(E, N, K, counts, rows_checked, seed):
    wl_keep = synth.n_keep_for(K, 0.5)
    rng = np.random.default_rng(seed)
    encs = []
    for e in range(E):
        W = synth.make_w(N, K, seed * 1000 + e)
        keep = osl.select_keep(W, wl_keep)
        A = synth.make_w(80, K, seed * 1000 + 500 + e, scale=0.01)    # [r][K]
        B = synth.make_w(N, 80, seed * 1000 + 700 + e, scale=0.01)    # [N][r]
        encs.append(osl.Encoded(osl.pack_masks(keep), osl.pack_values(W, keep, wl_keep), osl.block_offsets(keep),
                                A.T.copy(), B.T.copy(), keep, np.zeros(0), 0.0, 0.0))
    moe = _upload(encs, N, K, wl_keep, 80)
    off = _offsets(counts)
    X = synth.make_x(K, int(off[-1]), seed=seed)
    Y = _run(moe, X, off)
    rows = np.arange(N) if rows_checked is None else np.sort(rng.choice(N, rows_checked, replace=False))
    experts = [(en.masks, en.values, en.A_cat, en.B_cat) for en in encs]
    Yref = omoe.grouped_forward_rows(X, off, experts, K, rows)
    mr, nw = errors(Y[:, rows], Yref)
    say(f"moe full size E={E} {N}x{K}: {len(rows)} rows max_rel={mr:.3e} normwise={nw:.3e}")
    assert mr <= TOL_MAX_REL and nw <= TOL_NORMWISE


def test_moe_full_size_mixtral_experts():
    """8 experts of 14336 x 4096 (50%, r_cat 80), 16 tokens routed top-2 =
    32 rows; 512 sampled output columns of every row."""
    _full_size(8, 14336, 4096, (5, 3, 4, 6, 2, 4, 5, 3), 512, seed=71)


def test_moe_full_size_deepseek_lite_experts():
    """64 experts of 1408 x 2048 (50%, r_cat 80), 16 tokens routed top-6 =
    96 rows (some experts idle); every output."""
    counts = np.random.default_rng(5).multinomial(96, np.full(64, 1 / 64))
    _full_size(64, 1408, 2048, tuple(int(c) for c in counts), None, seed=72)
