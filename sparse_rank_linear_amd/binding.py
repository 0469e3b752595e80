"""ctypes binding of libsalr.so (include/salr.h).

Argument marshalling only: every step of encode and forward runs in the HIP
library.  torch supplies device memory and streams.  There is no fallback:
if libsalr.so is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsalr.so")

SALR_OK = 0
STATUS_NAMES = {
    0: "SALR_OK",
    -1: "SALR_ERR_INVALID_ARG",
    -2: "SALR_ERR_UNSUPPORTED",
    -3: "SALR_ERR_WORKSPACE",
    -4: "SALR_ERR_NONFINITE",
    -5: "SALR_ERR_NUMERICAL",
    -6: "SALR_ERR_HIP",
}

# Every symbol include/salr.h declares.
EXPORTS = (
    "salr_query_sizes",
    "salr_encode",
    "salr_linear_forward",
    "salr_fuse_layers",
    "salr_status_string",
    "salr_version",
)


class SalrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib().salr_status_string(status).decode() if _LIB is not None else ""
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({text})")


class salr_layer_t(C.Structure):
    _fields_ = [
        ("N", C.c_int64),
        ("K", C.c_int64),
        ("n_keep", C.c_int32),
        ("r_cat", C.c_int32),
        ("masks", C.c_void_p),
        ("values", C.c_void_p),
        ("offsets", C.c_void_p),
        ("a_cat", C.c_void_p),
        ("b_cat", C.c_void_p),
        ("n_parts", C.c_int32),
        ("part_rows", C.c_int32 * 8),
        ("part_ranks", C.c_int32 * 8),
    ]


class salr_sizes_t(C.Structure):
    _fields_ = [
        ("masks_bytes", C.c_size_t),
        ("values_bytes", C.c_size_t),
        ("offsets_bytes", C.c_size_t),
        ("a_cat_bytes", C.c_size_t),
        ("b_cat_bytes", C.c_size_t),
        ("encode_ws_bytes", C.c_size_t),
        ("forward_ws_bytes", C.c_size_t),
    ]


class salr_encode_opts_t(C.Structure):
    _fields_ = [("oversample", C.c_int32), ("iters", C.c_int32), ("seed", C.c_uint64)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_rank_linear_amd.build`")
        lib = C.CDLL(LIB_PATH)
        lib.salr_query_sizes.argtypes = [C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                         C.POINTER(salr_sizes_t)]
        lib.salr_query_sizes.restype = C.c_int
        lib.salr_encode.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                                    C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.POINTER(C.c_int32),
                                    C.POINTER(salr_encode_opts_t), C.POINTER(salr_layer_t),
                                    C.POINTER(C.c_double), C.c_void_p, C.c_size_t, C.c_void_p]
        lib.salr_encode.restype = C.c_int
        lib.salr_linear_forward.argtypes = [C.POINTER(salr_layer_t), C.c_void_p, C.c_int64, C.c_void_p,
                                            C.c_void_p, C.c_size_t, C.c_void_p]
        lib.salr_linear_forward.restype = C.c_int
        lib.salr_fuse_layers.argtypes = [C.POINTER(C.POINTER(salr_layer_t)), C.c_int32, C.POINTER(salr_layer_t),
                                         C.c_void_p]
        lib.salr_fuse_layers.restype = C.c_int
        lib.salr_status_string.argtypes = [C.c_int]
        lib.salr_status_string.restype = C.c_char_p
        lib.salr_version.argtypes = []
        lib.salr_version.restype = C.c_int
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises if libsalr.so is missing)."""
    return _lib()


def _check(status: int, where: str):
    if status != SALR_OK:
        raise SalrError(status, where)


def query_sizes(N: int, K: int, n_keep: int, r_svd: int, r_cat: int, M_max: int) -> dict:
    out = salr_sizes_t()
    _check(_lib().salr_query_sizes(N, K, n_keep, r_svd, r_cat, M_max, C.byref(out)), "salr_query_sizes")
    return {f: getattr(out, f) for f, _ in salr_sizes_t._fields_}


def _stream_ptr(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev_ptr(t, name):
    import torch

    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _as_bf16_bits(t, name):
    import torch

    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t.view(torch.bfloat16)
    raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")


@dataclass
class SalrLayer:
    """An encoded layer: five device tensors plus its shape (include/salr.h
    layout: masks [N][ceil(K/64)] uint64 (held as int64), values bf16
    [N*n_keep + padding], offsets [N][ceil(K/1024)] uint32 (held as int32),
    a_cat bf16 [r_cat][K], b_cat bf16 [N][r_cat])."""

    N: int
    K: int
    n_keep: int
    r_svd: int
    r_cat: int
    masks: object
    values: object
    offsets: object
    a_cat: object
    b_cat: object
    parts: tuple = ()  # ((rows, ranks), ...) of a fused layer (salr_fuse_layers)

    @classmethod
    def empty(cls, N, K, n_keep, r_svd, r_cat, device="cuda"):
        import torch

        sz = query_sizes(N, K, n_keep, r_svd, r_cat, 0)
        kw, ng = -(-K // 64), -(-K // 1024)
        return cls(
            N, K, n_keep, r_svd, r_cat,
            masks=torch.zeros((N, kw), dtype=torch.int64, device=device),
            values=torch.zeros(sz["values_bytes"] // 2, dtype=torch.bfloat16, device=device),
            offsets=torch.zeros((N, ng), dtype=torch.int32, device=device),
            a_cat=torch.zeros((max(r_cat, 0), K), dtype=torch.bfloat16, device=device),
            # [N][r_cat] view of a buffer with the tail padding the kernels need
            b_cat=torch.zeros(sz["b_cat_bytes"] // 2, dtype=torch.bfloat16,
                              device=device)[: N * max(r_cat, 0)].view(N, max(r_cat, 0)),
        )

    @classmethod
    def from_arrays(cls, masks, values, offsets, a_cat, b_cat, K, r_svd, device="cuda"):
        """Upload an encoding held in numpy arrays (uint64 masks, uint16
        values [N][n_keep], uint32 offsets, uint16 a_cat [r_cat][K] and
        b_cat [N][r_cat], all in the library's stored layout)."""
        import numpy as np
        import torch

        N, n_keep = values.shape
        r_cat = a_cat.shape[0]
        lay = cls.empty(N, K, n_keep, r_svd, r_cat, device)
        lay.masks.copy_(torch.from_numpy(np.ascontiguousarray(masks).view(np.int64)))
        flat = torch.from_numpy(np.ascontiguousarray(values).reshape(-1).view(np.int16))
        lay.values.view(torch.int16)[: flat.numel()].copy_(flat)
        lay.offsets.copy_(torch.from_numpy(np.ascontiguousarray(offsets).view(np.int32)))
        if r_cat:
            lay.a_cat.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(a_cat).view(np.int16)))
            lay.b_cat.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(b_cat).view(np.int16)))
        return lay

    def descriptor(self) -> salr_layer_t:
        d = salr_layer_t()
        d.N, d.K, d.n_keep, d.r_cat = self.N, self.K, self.n_keep, self.r_cat
        d.masks = self.masks.data_ptr()
        d.values = self.values.data_ptr()
        d.offsets = self.offsets.data_ptr()
        d.a_cat = self.a_cat.data_ptr() if self.r_cat else None
        d.b_cat = self.b_cat.data_ptr() if self.r_cat else None
        d.n_parts = len(self.parts)
        for p, (rows, ranks) in enumerate(self.parts):
            d.part_rows[p], d.part_ranks[p] = rows, ranks
        return d

    def clone(self) -> "SalrLayer":
        c = SalrLayer.empty(self.N, self.K, self.n_keep, self.r_svd, self.r_cat, self.masks.device)
        c.parts = self.parts
        for name in ("masks", "values", "offsets", "a_cat", "b_cat"):
            getattr(c, name).copy_(getattr(self, name))
        return c

    def to_numpy(self) -> dict:
        """Device tensors back as numpy arrays in the stored layout."""
        import numpy as np

        vals = self.values.view(self.values.dtype).cpu().view(__import__("torch").int16).numpy().view(np.uint16)
        return {
            "masks": self.masks.cpu().numpy().view(np.uint64),
            "values": vals[: self.N * self.n_keep].reshape(self.N, self.n_keep),
            "offsets": self.offsets.cpu().numpy().view(np.uint32),
            "a_cat": self.a_cat.cpu().view(__import__("torch").int16).numpy().view(np.uint16),
            "b_cat": self.b_cat.cpu().view(__import__("torch").int16).numpy().view(np.uint16),
        }

    def compressed_bytes(self) -> int:
        """Bytes of the encoding (masks + values + offsets + a_cat + b_cat),
        without the values buffer's tail padding."""
        kw, ng = -(-self.K // 64), -(-self.K // 1024)
        return (self.N * kw * 8 + self.N * self.n_keep * 2 + self.N * ng * 4
                + 2 * self.r_cat * self.K + 2 * self.N * self.r_cat)


def workspace(nbytes: int, device="cuda"):
    """A zero-filled workspace buffer (uint8)."""
    import torch

    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def encode(W, n_keep: int, r_svd: int, lora_A=(), lora_B=(), oversample: int | None = None,
           iters: int | None = None, seed: int = 0, ws=None, stream=None):
    """SALR encode on the GPU.  W bf16 [N][K]; lora_A[i] bf16 [r_i][K];
    lora_B[i] bf16 [N][r_i].  Returns (SalrLayer, sigma list)."""
    W = _as_bf16_bits(W, "W")
    N, K = W.shape
    ranks = [int(a.shape[0]) for a in lora_A]
    r_cat = r_svd + sum(ranks)
    layer = SalrLayer.empty(N, K, n_keep, r_svd, r_cat, W.device)
    sz = query_sizes(N, K, n_keep, r_svd, r_cat, 0)
    if ws is None:
        ws = workspace(sz["encode_ws_bytes"], W.device)
    nl = len(ranks)
    a_ptrs = (C.c_void_p * max(nl, 1))(*[_dev_ptr(_as_bf16_bits(a, "lora_A"), "lora_A") for a in lora_A])
    b_ptrs = (C.c_void_p * max(nl, 1))(*[_dev_ptr(_as_bf16_bits(b, "lora_B"), "lora_B") for b in lora_B])
    r_arr = (C.c_int32 * max(nl, 1))(*ranks)
    opts = None
    if oversample is not None or iters is not None or seed:
        opts = salr_encode_opts_t(32 if oversample is None else oversample, 24 if iters is None else iters, seed)
    sig = (C.c_double * max(r_svd, 1))()
    desc = layer.descriptor()
    st = _lib().salr_encode(
        C.c_void_p(_dev_ptr(W, "W")), N, K, n_keep, r_svd, nl,
        C.cast(a_ptrs, C.POINTER(C.c_void_p)) if nl else None,
        C.cast(b_ptrs, C.POINTER(C.c_void_p)) if nl else None,
        C.cast(r_arr, C.POINTER(C.c_int32)) if nl else None,
        C.byref(opts) if opts is not None else None, C.byref(desc), sig,
        C.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_encode")
    return layer, [sig[i] for i in range(r_svd)]


def forward_workspace(layer: SalrLayer, M_max: int, device="cuda"):
    sz = query_sizes(layer.N, layer.K, layer.n_keep, layer.r_svd, layer.r_cat, M_max)
    return workspace(sz["forward_ws_bytes"], device)


def linear_forward(layer: SalrLayer, X, Y=None, ws=None, stream=None):
    """Y = X W_s^T + (X A_cat) B_cat on the GPU (asynchronous on `stream`).
    X bf16 [M][K]; returns Y bf16 [M][N]."""
    import torch

    X = _as_bf16_bits(X, "X")
    M = X.shape[0]
    if X.dim() != 2 or X.shape[1] != layer.K:
        raise ValueError("X must be [M][K]")
    if Y is None:
        Y = torch.empty((M, layer.N), dtype=torch.bfloat16, device=X.device)
    if ws is None:
        ws = forward_workspace(layer, M, X.device)
    desc = layer.descriptor()
    st = _lib().salr_linear_forward(C.byref(desc), C.c_void_p(_dev_ptr(X, "X")), M, C.c_void_p(_dev_ptr(Y, "Y")),
                                    C.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_linear_forward")
    return Y


def fuse(layers, stream=None) -> SalrLayer:
    """One encoded layer computing every layer in `layers` (same K and
    n_keep) in a single forward: rows stacked along N, ranks stacked along
    r_cat, B_cat block diagonal (include/salr.h, salr_fuse_layers)."""
    layers = list(layers)
    if not layers:
        raise ValueError("fuse needs at least one layer")
    K, n_keep = layers[0].K, layers[0].n_keep
    N = sum(l.N for l in layers)
    r_cat = sum(l.r_cat for l in layers)
    out = SalrLayer.empty(N, K, n_keep, 0, r_cat, layers[0].masks.device)
    descs = [l.descriptor() for l in layers]
    arr = (C.POINTER(salr_layer_t) * len(descs))(*[C.pointer(d) for d in descs])
    od = out.descriptor()
    st = _lib().salr_fuse_layers(arr, len(descs), C.byref(od), _stream_ptr(stream))
    _check(st, "salr_fuse_layers")
    out.parts = tuple((od.part_rows[p], od.part_ranks[p]) for p in range(od.n_parts))
    return out
