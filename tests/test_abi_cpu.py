"""C-ABI checks that need no GPU: the library loads, exports every function
include/salr.h declares, sizes are what the layout says, and argument
validation rejects bad calls before any device work (so these calls are
safe without a GPU)."""

import ctypes as C
import os
import re

import pytest

import sparse_rank_linear_amd as srl
from sparse_rank_linear_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    """Every function declared in include/*.h."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, fn)).read(), flags=re.S)
            names.update(re.findall(r"\b(salr_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = srl.lib()
    declared = _header_functions()
    assert set(declared) == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_probe_validation_paths():
    lib = srl.lib()
    buf = C.create_string_buffer(64)
    p = C.cast(buf, C.c_void_p)
    # null, misaligned, zero or ragged sizes, bad grid / shape / iteration count
    assert lib.salr_probe_stream_read(None, 16, p, 1, None) == -1
    assert lib.salr_probe_stream_read(p, 0, p, 1, None) == -1
    assert lib.salr_probe_stream_read(p, 24, p, 1, None) == -1
    assert lib.salr_probe_stream_read(p, 16, None, 1, None) == -1
    assert lib.salr_probe_stream_read(p, 16, p, 0, None) == -1
    assert lib.salr_probe_stream_read(p, 16, p, 65537, None) == -1
    assert lib.salr_probe_mfma(None, 1, 1, 0, None) == -1
    assert lib.salr_probe_mfma(p, 0, 1, 0, None) == -1
    assert lib.salr_probe_mfma(p, 1, 0, 0, None) == -1
    assert lib.salr_probe_mfma(p, 1, 1, 2, None) == -1


def test_nf4_levels_equal_the_oracle():
    """The library's level table (normal quantiles by bisection on erfc)
    equals the oracle's (scipy quantiles), bit for bit."""
    import numpy as np
    from oracle import nf4

    got = np.array(srl.nf4_levels(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), nf4.nf4_levels().view(np.uint32))
    assert srl.lib().salr_nf4_levels(None) == -1


def test_nf4_sizes_and_quantize_validation():
    sz = srl.query_sizes(100, 520, 260, 4, 12, 300)
    assert sz["codes_bytes"] >= 100 * 5 * 32 and sz["scales_bytes"] >= 100 * 5 * 2
    assert sz["forward_ws_nf4_bytes"] >= sz["forward_ws_bytes"] + 100 * 260 * 2   # dequantized values
    lib = srl.lib()
    assert lib.salr_quantize_nf4(None, None) == -1
    d = _layer()
    assert lib.salr_quantize_nf4(C.byref(d), None) == -1          # no codes / scales
    d.codes, d.scales = 0x50000000, 0x60000008                   # misaligned scales
    assert lib.salr_quantize_nf4(C.byref(d), None) == -1
    d.scales, d.value_format = 0x60000000, 1                      # already NF4
    assert lib.salr_quantize_nf4(C.byref(d), None) == -1
    d = _layer()
    d.value_format = 2                                            # unknown format
    assert _fwd(d) == -1
    d.value_format = 1                                            # NF4 without codes
    assert _fwd(d) == -1


def test_status_strings_and_version():
    lib = srl.lib()
    for code in B.STATUS_NAMES:
        assert lib.salr_status_string(code)
    assert lib.salr_status_string(12345) == b"unknown status"
    assert lib.salr_version() == 10000


def test_query_sizes_layout():
    N, K, n_keep, r_svd, r_cat = 4096, 4096, 2048, 64, 80
    sz = srl.query_sizes(N, K, n_keep, r_svd, r_cat, 16)
    assert sz["masks_bytes"] == N * K // 8
    assert sz["values_bytes"] >= N * n_keep * 2 + 256
    assert sz["offsets_bytes"] == N * (K // 1024) * 4
    assert sz["a_cat_bytes"] == r_cat * K * 2
    assert sz["b_cat_bytes"] >= N * r_cat * 2 + 256  # tail padding, like values
    assert sz["forward_ws_bytes"] >= 512 * 1024
    assert sz["encode_ws_bytes"] >= N * K * 2
    # ragged shapes round up
    sz = srl.query_sizes(3, 520, 7, 0, 0, 0)
    assert sz["masks_bytes"] == 3 * 9 * 8 and sz["offsets_bytes"] == 3 * 1 * 4
    # the many-row workspace grows with M_max
    a = srl.query_sizes(N, K, n_keep, r_svd, r_cat, 16)["forward_ws_bytes"]
    b = srl.query_sizes(N, K, n_keep, r_svd, r_cat, 4096)["forward_ws_bytes"]
    assert b > a


@pytest.mark.parametrize("args", [
    (0, 64, 1, 0, 0, 1),        # N < 1
    (4, 0, 0, 0, 0, 1),         # K < 1
    (4, 60, 1, 0, 0, 1),        # K % 8
    (4, 64, 65, 0, 0, 1),       # n_keep > K
    (4, 64, -1, 0, 0, 1),       # n_keep < 0
    (4, 64, 8, 5, 4, 1),        # r_svd > r_cat
    (4, 64, 8, 5, 8, 1),        # r_svd > min(N, K)
    (4, 64, 8, 0, 300, 1),      # r_cat > 256
    (4, 64, 8, 0, 0, -1),       # M_max < 0
    (4, 1 << 21, 8, 0, 0, 1),   # K too large
])
def test_query_sizes_rejects(args):
    out = B.salr_sizes_t()
    assert srl.lib().salr_query_sizes(*args, C.byref(out)) == -1
    assert srl.lib().salr_query_sizes(4, 64, 8, 0, 0, 1, None) == -1


def _layer(N=64, K=64, n_keep=32, r_cat=0, base=0x10000000):
    d = B.salr_layer_t()
    d.N, d.K, d.n_keep, d.r_cat = N, K, n_keep, r_cat
    d.masks, d.values, d.offsets = base, base + 0x100000, base + 0x200000
    d.a_cat = base + 0x300000 if r_cat else None
    d.b_cat = base + 0x400000 if r_cat else None
    return d


def _fwd(d, X=0x20000000, M=4, Y=0x30000000, ws=0x40000000, ws_bytes=1 << 30):
    return srl.lib().salr_linear_forward(C.byref(d) if d is not None else None, C.c_void_p(X), M, C.c_void_p(Y),
                                         C.c_void_p(ws), ws_bytes, None)


def test_forward_validation_paths():
    # These return before any HIP call, so they run without a GPU.
    assert _fwd(_layer(), M=0) == 0                       # M == 0 is a no-op
    assert _fwd(None) == -1                               # null layer
    assert _fwd(_layer(), M=-1) == -1
    assert _fwd(_layer(), X=0) == -1                      # null X
    assert _fwd(_layer(), Y=0) == -1                      # null Y
    assert _fwd(_layer(), X=0x20000008) == -1             # misaligned X
    assert _fwd(_layer(), X=0x30000000, Y=0x30000000) == -1  # X aliases Y
    assert _fwd(_layer(K=60)) == -1                       # K % 8
    assert _fwd(_layer(n_keep=65)) == -1
    d = _layer(r_cat=8)
    d.a_cat = None
    assert _fwd(d) == -1                                  # adapters missing
    d = _layer()
    d.masks = 0x10000004
    assert _fwd(d) == -1                                  # misaligned masks
    assert _fwd(_layer(), ws=0) == -3                     # null workspace
    assert _fwd(_layer(), ws_bytes=1024) == -3            # workspace too small
    assert _fwd(_layer(), ws=0x40000008) == -3            # misaligned workspace
    d = _layer(N=64, r_cat=16)
    d.n_parts = 9
    assert _fwd(d) == -1                                  # more parts than recorded slots
    d.n_parts = 2
    d.part_rows[0], d.part_rows[1], d.part_ranks[0], d.part_ranks[1] = 32, 16, 8, 8
    assert _fwd(d) == -1                                  # parts' rows do not sum to N
    d.part_rows[1], d.part_ranks[1] = 32, 16
    assert _fwd(d) == -1                                  # parts' ranks do not sum to r_cat
    d.part_rows[0], d.part_rows[1], d.part_ranks[0], d.part_ranks[1] = 64, 0, 16, 0
    assert _fwd(d) == -1                                  # an empty part


def _enc(W=0x50000000, N=64, K=64, n_keep=32, r_svd=4, out=None, ws=0x60000000, ws_bytes=1 << 30, opts=None,
         loras=()):
    if out is None:
        out = _layer(N, K, n_keep, r_svd + sum(loras), base=0x70000000)
    nl = len(loras)
    ap = (C.c_void_p * max(nl, 1))(*[0x80000000 + 0x100000 * i for i in range(nl)])
    bp = (C.c_void_p * max(nl, 1))(*[0x90000000 + 0x100000 * i for i in range(nl)])
    rr = (C.c_int32 * max(nl, 1))(*loras)
    return srl.lib().salr_encode(
        C.c_void_p(W), N, K, n_keep, r_svd, nl,
        C.cast(ap, C.POINTER(C.c_void_p)) if nl else None, C.cast(bp, C.POINTER(C.c_void_p)) if nl else None,
        C.cast(rr, C.POINTER(C.c_int32)) if nl else None, C.byref(opts) if opts else None,
        C.byref(out) if out is not None else None, None, C.c_void_p(ws), ws_bytes, None)


def _fwd_noalloc(d, X=0x20000000, M=4, Y=0x30000000, err=None):
    return srl.lib().salr_linear_forward_noalloc(C.byref(d) if d is not None else None, C.c_void_p(X), M,
                                                 C.c_void_p(Y), C.c_void_p(err) if err else None, None)


def test_forward_noalloc_validation_paths():
    # Argument errors are reported before the device (and the library's
    # fixed array) is touched, so these run without a GPU.
    assert _fwd_noalloc(_layer(), M=0) == 0
    assert _fwd_noalloc(None) == -1
    assert _fwd_noalloc(_layer(), M=-1) == -1
    assert _fwd_noalloc(_layer(), X=0) == -1
    assert _fwd_noalloc(_layer(), X=0x20000008) == -1
    assert _fwd_noalloc(_layer(), X=0x30000000, Y=0x30000000) == -1
    assert _fwd_noalloc(_layer(K=60)) == -1
    d = _layer(N=64, r_cat=16)
    d.n_parts = 9
    assert _fwd_noalloc(d) == -1
    assert _fwd_noalloc(_layer(), err=0x50000002) == -1   # misaligned wait-error word


def test_encode_validation_paths():
    assert _enc(W=0) == -1
    d = _layer(64, 64, 32, 4, base=0x70000000)
    d.n_keep = 31
    assert _enc(out=d) == -1                              # descriptor disagrees with n_keep
    assert _enc(r_svd=70) == -1                           # r_svd > min(N, K)
    d = _layer(64, 64, 32, 5, base=0x70000000)
    assert _enc(out=d, r_svd=4) == -1                     # r_cat != r_svd + sum(lora)
    assert _enc(loras=(0,)) == -1                         # LoRA rank < 1
    assert _enc(opts=B.salr_encode_opts_t(65, 4, 0)) == -1  # oversample too large
    assert _enc(opts=B.salr_encode_opts_t(8, -1, 0)) == -1  # iters < 0
    assert _enc(ws=0) == -3
    assert _enc(ws_bytes=4096) == -3


def _fuse(parts, out):
    arr = (C.POINTER(B.salr_layer_t) * max(len(parts), 1))(*[C.pointer(p) for p in parts])
    return srl.lib().salr_fuse_layers(arr if parts else None, len(parts), C.byref(out) if out is not None else None,
                                      None)


def test_fuse_validation_paths():
    # Every case fails validation, which happens before any HIP call.
    a = _layer(64, 64, 32, 8, base=0x10000000)
    b = _layer(32, 64, 32, 4, base=0x20000000)
    out = _layer(96, 64, 32, 12, base=0x30000000)
    assert _fuse([], out) == -1                           # no parts
    assert _fuse([a, b], None) == -1                      # null output
    assert _fuse([a, b], _layer(95, 64, 32, 12, base=0x30000000)) == -1   # N != sum
    assert _fuse([a, b], _layer(96, 64, 32, 11, base=0x30000000)) == -1   # r_cat != sum
    assert _fuse([a, _layer(32, 72, 36, 4, base=0x20000000)], out) == -1  # K differs
    assert _fuse([a, _layer(32, 64, 31, 4, base=0x20000000)], out) == -1  # n_keep differs
    big = [_layer(16, 64, 32, 200, base=0x10000000 * (i + 1)) for i in range(2)]
    assert _fuse(big, _layer(32, 64, 32, 400, base=0x50000000)) == -1    # sum of ranks > 256
    c = _layer(32, 64, 32, 4, base=0x20000000)
    c.b_cat = None
    assert _fuse([a, c], out) == -1                       # adapters missing
    d = _layer(96, 64, 32, 12, base=0x30000000)
    d.values = 0x30100008
    assert _fuse([a, b], d) == -1                         # misaligned output
    nine = [_layer(16, 64, 32, 0, base=0x10000000 * (i + 1)) for i in range(9)]
    assert _fuse(nine, _layer(144, 64, 32, 0, base=0xa0000000)) == -1   # more than 8 parts
    f = _layer(96, 64, 32, 12, base=0x30000000)
    f.n_parts = 8
    for p in range(8):
        f.part_rows[p], f.part_ranks[p] = 12, 0
    f.part_ranks[0] = 12
    assert _fuse([a, f], _layer(160, 64, 32, 20, base=0x50000000)) == -1  # 1 + 8 recorded parts


def test_python_wrapper_requires_library(monkeypatch, tmp_path):
    """With the shared library missing, the product path raises instead of
    falling back to anything else."""
    monkeypatch.setattr(B, "_LIB", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.query_sizes(4, 64, 8, 0, 0, 1)


def _bwd(L, LT, X=0x20000000, dY=0x21000000, M=4, dX=0x30000000, dA=0x31000000, dB=0x32000000, ws=0x40000000,
         ws_bytes=1 << 30):
    vp = lambda a: C.c_void_p(a) if a else None
    return srl.lib().salr_linear_backward(C.byref(L) if L is not None else None,
                                          C.byref(LT) if LT is not None else None, vp(X), vp(dY), M, vp(dX), vp(dA),
                                          vp(dB), vp(ws), ws_bytes, None)


def test_backward_sizes():
    # the transposed-encoding build: row counts, block column counts, max word
    assert srl.transpose_ws_bytes(4096, 4096) >= 4096 * 64 * 4 + 64 * 4096 * 4
    with pytest.raises(srl.SalrError):
        srl.transpose_ws_bytes(4, 60)
    # the backward workspace grows with M and holds the transposed forward's
    a = srl.backward_ws_bytes(4096, 4096, 2100, 80, 16)
    b = srl.backward_ws_bytes(4096, 4096, 2100, 80, 2048)
    assert b > a >= srl.query_sizes(4096, 4096, 2100, 0, 80, 16)["forward_ws_bytes"]
    # operands of the gradient GEMMs at 2048 tokens: X^T, dY^T, G^T, T^T
    assert b >= 2 * 2048 * (4096 + 4096 + 2 * 80)
    with pytest.raises(srl.SalrError):
        srl.backward_ws_bytes(4100, 4096, 2048, 80, 16)    # N % 8: W_s^T's column count
    with pytest.raises(srl.SalrError):
        srl.backward_ws_bytes(4096, 4096, 4097, 80, 16)    # n_keep_t > N


def test_transpose_validation_paths():
    # These return before any HIP call, so they run without a GPU.
    lib = srl.lib()
    n = C.c_int32()
    L = _layer(N=64, K=128, n_keep=32)
    assert lib.salr_transpose_count(None, C.byref(n), C.c_void_p(0x40000000), 1 << 30, None) == -1
    assert lib.salr_transpose_count(C.byref(L), None, C.c_void_p(0x40000000), 1 << 30, None) == -1
    assert lib.salr_transpose_count(C.byref(_layer(N=60, K=128)), C.byref(n), C.c_void_p(0x40000000), 1 << 30,
                                    None) == -2                    # N % 8
    assert lib.salr_transpose_count(C.byref(L), C.byref(n), None, 1 << 30, None) == -3
    assert lib.salr_transpose_count(C.byref(L), C.byref(n), C.c_void_p(0x40000000), 64, None) == -3
    LT = _layer(N=128, K=64, n_keep=40, base=0x11000000)
    ws = C.c_void_p(0x40000000)
    assert lib.salr_transpose_layer(C.byref(L), None, ws, 1 << 30, None) == -1
    bad = _layer(N=120, K=64, n_keep=40, base=0x11000000)
    assert lib.salr_transpose_layer(C.byref(L), C.byref(bad), ws, 1 << 30, None) == -1   # LT.N != K
    bad = _layer(N=128, K=64, n_keep=65, base=0x11000000)
    assert lib.salr_transpose_layer(C.byref(L), C.byref(bad), ws, 1 << 30, None) == -1   # n_keep > N
    bad = _layer(N=128, K=64, n_keep=40, base=0x11000000)
    bad.values = 0x11100008
    assert lib.salr_transpose_layer(C.byref(L), C.byref(bad), ws, 1 << 30, None) == -1   # misaligned
    q = _layer(N=64, K=128, n_keep=32)
    q.value_format = B.VALUES_NF4
    assert lib.salr_transpose_layer(C.byref(q), C.byref(LT), ws, 1 << 30, None) == -2    # NF4 layer
    assert lib.salr_transpose_layer(C.byref(L), C.byref(LT), ws, 64, None) == -3


def test_backward_validation_paths():
    L = _layer(N=64, K=128, n_keep=32, r_cat=16)
    LT = _layer(N=128, K=64, n_keep=40, r_cat=16, base=0x11000000)
    assert _bwd(None, LT) == -1
    assert _bwd(L, None) == -1
    assert _bwd(L, _layer(N=120, K=64, n_keep=40, r_cat=16, base=0x11000000)) == -1   # LT.N != K
    assert _bwd(L, _layer(N=128, K=64, n_keep=40, r_cat=8, base=0x11000000)) == -1    # ranks differ
    assert _bwd(_layer(N=60, K=128, n_keep=32, r_cat=16),
                _layer(N=128, K=60, n_keep=30, r_cat=16, base=0x11000000)) == -2       # N % 8
    t = _layer(N=128, K=64, n_keep=40, r_cat=16, base=0x11000000)
    t.n_parts = 1
    assert _bwd(L, t) == -1                                     # a transposed layer has no parts
    t = _layer(N=128, K=64, n_keep=40, r_cat=16, base=0x11000000)
    t.value_format = B.VALUES_NF4
    assert _bwd(L, t) == -1                                     # nor NF4 values
    assert _bwd(L, LT, M=-1) == -1
    assert _bwd(L, LT, X=0) == -1
    assert _bwd(L, LT, dY=0) == -1
    assert _bwd(L, LT, dA=0) == -1                              # adapters need both gradients
    assert _bwd(L, LT, dB=0) == -1
    assert _bwd(L, LT, dY=0x21000008) == -1                     # misaligned
    assert _bwd(L, LT, dX=0x21000000) == -1                     # dX aliases dY
    d = _layer(N=64, K=128, n_keep=32, r_cat=16)
    d.b_cat = None
    assert _bwd(d, LT) == -1
    assert _bwd(L, LT, ws=0) == -3
    assert _bwd(L, LT, ws_bytes=4096) == -3


def _moe(E=4, N=64, K=128, n_keep=64, r_cat=8, base=0x10000000):
    d = B.salr_moe_layer_t()
    d.E, d.N, d.K, d.n_keep, d.r_cat = E, N, K, n_keep, r_cat
    d.masks, d.values, d.offsets = base, base + 0x1000000, base + 0x2000000
    d.a_cat = base + 0x3000000 if r_cat else None
    d.b_cat = base + 0x4000000 if r_cat else None
    return d


def test_moe_sizes_and_expert_views():
    E, N, K, n_keep, r = 8, 14336, 4096, 2048, 80
    sz = srl.moe_query_sizes(E, N, K, n_keep, r, 32)
    assert sz["masks_stride"] == N * K // 64 and sz["values_stride"] == N * n_keep
    assert sz["masks_bytes"] == E * N * K // 8
    assert sz["values_bytes"] >= E * N * n_keep * 2 + 256          # tail padding
    assert sz["b_cat_bytes"] >= E * N * r * 2 + 256
    assert sz["forward_ws_bytes"] >= 32 * 96 * 2                    # bf16 T, ranks padded to 32
    for name in ("masks", "values", "offsets", "a_cat", "b_cat"):   # 256-byte aligned expert slices
        esize = {"masks": 8, "values": 2, "offsets": 4, "a_cat": 2, "b_cat": 2}[name]
        assert (sz[name + "_stride"] * esize) % 256 == 0
    # ragged shapes keep every slice aligned
    sz = srl.moe_query_sizes(3, 7, 520, 9, 5, 1)
    assert sz["values_stride"] % 128 == 0 and sz["masks_stride"] % 32 == 0 and sz["offsets_stride"] % 64 == 0
    # expert views
    d = _moe(E=3, N=7, K=520, n_keep=9, r_cat=5)
    out = B.salr_layer_t()
    assert srl.lib().salr_moe_expert(C.byref(d), 2, C.byref(out)) == 0
    assert (out.N, out.K, out.n_keep, out.r_cat, out.n_parts) == (7, 520, 9, 5, 0)
    assert out.values == d.values + 2 * sz["values_stride"] * 2
    assert out.masks == d.masks + 2 * sz["masks_stride"] * 8
    assert out.offsets == d.offsets + 2 * sz["offsets_stride"] * 4
    assert out.a_cat == d.a_cat + 2 * sz["a_cat_stride"] * 2
    assert out.b_cat == d.b_cat + 2 * sz["b_cat_stride"] * 2
    assert srl.lib().salr_moe_expert(C.byref(d), 3, C.byref(out)) == -1
    assert srl.lib().salr_moe_expert(C.byref(d), -1, C.byref(out)) == -1


def test_moe_validation_paths():
    lib = srl.lib()
    out = B.salr_moe_sizes_t()
    assert lib.salr_moe_query_sizes(0, 64, 128, 64, 8, 1, C.byref(out)) == -1      # E < 1
    assert lib.salr_moe_query_sizes(4097, 64, 128, 64, 8, 1, C.byref(out)) == -1   # too many experts
    assert lib.salr_moe_query_sizes(4, 64, 128, 129, 8, 1, C.byref(out)) == -1     # n_keep > K
    assert lib.salr_moe_query_sizes(4, 64, 60, 8, 8, 1, C.byref(out)) == -1        # K % 8

    def fwd(d, X=0x20000000, T=4, off=0x21000000, m_cap=0, Y=0x30000000, ws=0x40000000, ws_bytes=1 << 30):
        vp = lambda a: C.c_void_p(a) if a else None
        return lib.salr_moe_forward(C.byref(d) if d is not None else None, vp(X), T, vp(off), m_cap, vp(Y), vp(ws),
                                    ws_bytes, None)

    assert fwd(_moe(), T=0) == 0                     # no rows: a no-op
    assert fwd(None) == -1
    assert fwd(_moe(), T=-1) == -1
    assert fwd(_moe(), m_cap=-1) == -1
    assert fwd(_moe(), X=0) == -1
    assert fwd(_moe(), Y=0) == -1
    assert fwd(_moe(), off=0) == -1
    assert fwd(_moe(), off=0x21000002) == -1         # misaligned offsets
    assert fwd(_moe(), X=0x20000008) == -1
    assert fwd(_moe(), X=0x30000000, Y=0x30000000) == -1
    d = _moe()
    d.b_cat = None
    assert fwd(d) == -1
    assert fwd(_moe(K=60)) == -1
    assert fwd(_moe(), ws=0) == -3
    assert fwd(_moe(), ws_bytes=64) == -3
