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
    text = open(os.path.join(ROOT, "include", "salr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(salr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = srl.lib()
    declared = _header_functions()
    assert set(declared) == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


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
