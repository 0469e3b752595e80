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
    "salr_linear_forward_noalloc",
    "salr_fuse_layers",
    "salr_status_string",
    "salr_version",
    "salr_nf4_levels",
    "salr_quantize_nf4",
    "salr_transpose_ws_bytes",
    "salr_transpose_count",
    "salr_transpose_layer",
    "salr_backward_ws_bytes",
    "salr_linear_backward",
    "salr_moe_query_sizes",
    "salr_moe_expert",
    "salr_moe_forward",
    # include/salr_probe.h
    "salr_probe_stream_read",
    "salr_probe_mfma",
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
        ("value_format", C.c_int32),
        ("codes", C.c_void_p),
        ("scales", C.c_void_p),
    ]

VALUES_BF16 = 0
VALUES_NF4 = 1


class salr_sizes_t(C.Structure):
    _fields_ = [
        ("masks_bytes", C.c_size_t),
        ("values_bytes", C.c_size_t),
        ("offsets_bytes", C.c_size_t),
        ("a_cat_bytes", C.c_size_t),
        ("b_cat_bytes", C.c_size_t),
        ("encode_ws_bytes", C.c_size_t),
        ("forward_ws_bytes", C.c_size_t),
        ("codes_bytes", C.c_size_t),
        ("scales_bytes", C.c_size_t),
        ("forward_ws_nf4_bytes", C.c_size_t),
    ]


class salr_moe_layer_t(C.Structure):
    _fields_ = [
        ("E", C.c_int32),
        ("N", C.c_int64),
        ("K", C.c_int64),
        ("n_keep", C.c_int32),
        ("r_cat", C.c_int32),
        ("masks", C.c_void_p),
        ("values", C.c_void_p),
        ("offsets", C.c_void_p),
        ("a_cat", C.c_void_p),
        ("b_cat", C.c_void_p),
    ]


class salr_moe_sizes_t(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "masks_bytes", "values_bytes", "offsets_bytes", "a_cat_bytes", "b_cat_bytes",
        "masks_stride", "values_stride", "offsets_stride", "a_cat_stride", "b_cat_stride",
        "forward_ws_bytes")]


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
        lib.salr_linear_forward_noalloc.argtypes = [C.POINTER(salr_layer_t), C.c_void_p, C.c_int64, C.c_void_p,
                                                    C.c_void_p, C.c_void_p]
        lib.salr_linear_forward_noalloc.restype = C.c_int
        lib.salr_fuse_layers.argtypes = [C.POINTER(C.POINTER(salr_layer_t)), C.c_int32, C.POINTER(salr_layer_t),
                                         C.c_void_p]
        lib.salr_fuse_layers.restype = C.c_int
        lib.salr_status_string.argtypes = [C.c_int]
        lib.salr_status_string.restype = C.c_char_p
        lib.salr_version.argtypes = []
        lib.salr_version.restype = C.c_int
        lib.salr_nf4_levels.argtypes = [C.POINTER(C.c_float)]
        lib.salr_nf4_levels.restype = C.c_int
        lib.salr_quantize_nf4.argtypes = [C.POINTER(salr_layer_t), C.c_void_p]
        lib.salr_quantize_nf4.restype = C.c_int
        lib.salr_transpose_ws_bytes.argtypes = [C.c_int64, C.c_int64, C.POINTER(C.c_size_t)]
        lib.salr_transpose_ws_bytes.restype = C.c_int
        lib.salr_transpose_count.argtypes = [C.POINTER(salr_layer_t), C.POINTER(C.c_int32), C.c_void_p, C.c_size_t,
                                             C.c_void_p]
        lib.salr_transpose_count.restype = C.c_int
        lib.salr_transpose_layer.argtypes = [C.POINTER(salr_layer_t), C.POINTER(salr_layer_t), C.c_void_p,
                                             C.c_size_t, C.c_void_p]
        lib.salr_transpose_layer.restype = C.c_int
        lib.salr_backward_ws_bytes.argtypes = [C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int64,
                                               C.POINTER(C.c_size_t)]
        lib.salr_backward_ws_bytes.restype = C.c_int
        lib.salr_linear_backward.argtypes = [C.POINTER(salr_layer_t), C.POINTER(salr_layer_t), C.c_void_p,
                                             C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                             C.c_void_p, C.c_size_t, C.c_void_p]
        lib.salr_linear_backward.restype = C.c_int
        lib.salr_moe_query_sizes.argtypes = [C.c_int32, C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int64,
                                             C.POINTER(salr_moe_sizes_t)]
        lib.salr_moe_query_sizes.restype = C.c_int
        lib.salr_moe_expert.argtypes = [C.POINTER(salr_moe_layer_t), C.c_int32, C.POINTER(salr_layer_t)]
        lib.salr_moe_expert.restype = C.c_int
        lib.salr_moe_forward.argtypes = [C.POINTER(salr_moe_layer_t), C.c_void_p, C.c_int64, C.c_void_p,
                                         C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        lib.salr_moe_forward.restype = C.c_int
        lib.salr_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_void_p]
        lib.salr_probe_stream_read.restype = C.c_int
        lib.salr_probe_mfma.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]
        lib.salr_probe_mfma.restype = C.c_int
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
    value_format: int = VALUES_BF16
    codes: object = None   # NF4: uint8 [N][32 * ceil(n_keep/64)] (+ padding)
    scales: object = None  # NF4: bf16 [N][ceil(n_keep/64)] (+ padding)

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
        d.value_format = self.value_format
        d.codes = self.codes.data_ptr() if self.codes is not None else None
        d.scales = self.scales.data_ptr() if self.scales is not None else None
        return d

    def clone(self) -> "SalrLayer":
        c = SalrLayer.empty(self.N, self.K, self.n_keep, self.r_svd, self.r_cat, self.masks.device)
        c.parts = self.parts
        for name in ("masks", "values", "offsets", "a_cat", "b_cat"):
            getattr(c, name).copy_(getattr(self, name))
        if self.codes is not None:
            c.codes, c.scales = self.codes.clone(), self.scales.clone()
            c.value_format = self.value_format
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
        """Bytes of the encoding (masks + values, or NF4 codes + scales, +
        offsets + a_cat + b_cat), without tail padding."""
        kw, ng = -(-self.K // 64), -(-self.K // 1024)
        if self.value_format == VALUES_NF4:
            nblk = -(-self.n_keep // 64)
            vbytes = self.N * nblk * 32 + self.N * nblk * 2
        else:
            vbytes = self.N * self.n_keep * 2
        return (self.N * kw * 8 + vbytes + self.N * ng * 4
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
    sig = _encode_into(layer.descriptor(), W, n_keep, r_svd, lora_A, lora_B, oversample, iters, seed, ws, stream)
    return layer, sig


def _encode_into(desc, W, n_keep, r_svd, lora_A, lora_B, oversample, iters, seed, ws, stream):
    """salr_encode into the buffers of an existing descriptor."""
    N, K = W.shape
    ranks = [int(a.shape[0]) for a in lora_A]
    r_cat = r_svd + sum(ranks)
    sz = query_sizes(N, K, n_keep, r_svd, r_cat, 0)
    if ws is None:
        ws = workspace(sz["encode_ws_bytes"], W.device)
    nl = len(ranks)
    a_ptrs = (C.c_void_p * max(nl, 1))(*[_dev_ptr(_as_bf16_bits(a, "lora_A"), "lora_A") for a in lora_A])
    b_ptrs = (C.c_void_p * max(nl, 1))(*[_dev_ptr(_as_bf16_bits(b, "lora_B"), "lora_B") for b in lora_B])
    r_arr = (C.c_int32 * max(nl, 1))(*ranks)
    opts = None
    if oversample is not None or iters is not None or seed:
        opts = salr_encode_opts_t(32 if oversample is None else oversample, 40 if iters is None else iters, seed)
    sig = (C.c_double * max(r_svd, 1))()
    st = _lib().salr_encode(
        C.c_void_p(_dev_ptr(W, "W")), N, K, n_keep, r_svd, nl,
        C.cast(a_ptrs, C.POINTER(C.c_void_p)) if nl else None,
        C.cast(b_ptrs, C.POINTER(C.c_void_p)) if nl else None,
        C.cast(r_arr, C.POINTER(C.c_int32)) if nl else None,
        C.byref(opts) if opts is not None else None, C.byref(desc), sig,
        C.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_encode")
    return [sig[i] for i in range(r_svd)]


def forward_workspace(layer: SalrLayer, M_max: int, device="cuda"):
    sz = query_sizes(layer.N, layer.K, layer.n_keep, layer.r_svd, layer.r_cat, M_max)
    key = "forward_ws_nf4_bytes" if layer.value_format == VALUES_NF4 else "forward_ws_bytes"
    return workspace(sz[key], device)


def nf4_levels():
    """The 16 NF4 levels of the library (salr_nf4_levels), as floats."""
    out = (C.c_float * 16)()
    _check(_lib().salr_nf4_levels(out), "salr_nf4_levels")
    return [out[i] for i in range(16)]


def quantize_nf4(layer: SalrLayer, stream=None) -> SalrLayer:
    """QSALR: code the layer's kept values as NF4 on the GPU
    (salr_quantize_nf4).  Allocates the codes and scales and switches the
    layer to them; the bf16 values stay allocated (the forward does not read
    them)."""
    import torch

    sz = query_sizes(layer.N, layer.K, layer.n_keep, layer.r_svd, layer.r_cat, 0)
    dev = layer.masks.device
    layer.codes = torch.zeros(sz["codes_bytes"], dtype=torch.uint8, device=dev)
    layer.scales = torch.zeros(sz["scales_bytes"] // 2, dtype=torch.int16, device=dev)
    d = layer.descriptor()
    _check(_lib().salr_quantize_nf4(C.byref(d), _stream_ptr(stream)), "salr_quantize_nf4")
    layer.value_format = d.value_format
    return layer


# Byte offset of the forward workspace's wait-error word (include/salr.h).
WAIT_ERROR_OFFSET = 8


class WaitTimeout(RuntimeError):
    """A bounded cross-workgroup wait of a forward call timed out (Y is
    unreliable)."""


def wait_error(ws, stream=None) -> int:
    """The forward workspace's wait-error word (uint32 at byte 8): nonzero
    once any call on this workspace had a bounded wait time out.  Waits for
    the work queued on `stream` (default: torch's current stream)."""
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    s.synchronize()
    word = ws[WAIT_ERROR_OFFSET:WAIT_ERROR_OFFSET + 4].cpu()
    return int(word.view(torch.int32).item())


def linear_forward(layer: SalrLayer, X, Y=None, ws=None, stream=None, check: bool = False):
    """Y = X W_s^T + (X A_cat) B_cat on the GPU (asynchronous on `stream`).
    X bf16 [M][K]; returns Y bf16 [M][N].  With check=True the call
    synchronizes the stream and raises WaitTimeout if the workspace's
    wait-error word is set."""
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
    if check and wait_error(ws, stream):
        raise WaitTimeout("salr_linear_forward: a bounded wait timed out (workspace error word set)")
    return Y


# Bytes of the library's fixed forward array (SALR_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def linear_forward_noalloc(layer: SalrLayer, X, Y, wait_err=None, stream=None):
    """salr_linear_forward_noalloc: the forward with the library's fixed
    per-GPU workspace (nothing allocated by the call).  Y bf16 [M][N] must
    be given; wait_err is an optional device int32 tensor of one element
    that a timed-out wait sets nonzero."""
    X = _as_bf16_bits(X, "X")
    Y = _as_bf16_bits(Y, "Y")
    M = X.shape[0]
    if X.dim() != 2 or X.shape[1] != layer.K or tuple(Y.shape) != (M, layer.N):
        raise ValueError("X must be [M][K] and Y [M][N]")
    desc = layer.descriptor()
    err = C.c_void_p(_dev_ptr(wait_err, "wait_err")) if wait_err is not None else None
    st = _lib().salr_linear_forward_noalloc(C.byref(desc), C.c_void_p(_dev_ptr(X, "X")), M,
                                            C.c_void_p(_dev_ptr(Y, "Y")), err, _stream_ptr(stream))
    _check(st, "salr_linear_forward_noalloc")
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


def transpose_ws_bytes(N: int, K: int) -> int:
    out = C.c_size_t()
    _check(_lib().salr_transpose_ws_bytes(N, K, C.byref(out)), "salr_transpose_ws_bytes")
    return out.value


def transpose_count(layer: SalrLayer, ws=None, stream=None) -> int:
    """The largest number of kept entries in one column of W_s (the n_keep
    of the transposed layer).  Synchronous."""
    if ws is None:
        ws = workspace(transpose_ws_bytes(layer.N, layer.K), layer.masks.device)
    out = C.c_int32()
    desc = layer.descriptor()
    st = _lib().salr_transpose_count(C.byref(desc), C.byref(out), C.c_void_p(ws.data_ptr()),
                                     ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_transpose_count")
    return out.value


def transpose_layer(layer: SalrLayer, n_keep: int | None = None, ws=None, stream=None) -> SalrLayer:
    """The encoding of W_s^T (K rows of N columns) built on the GPU, for
    the backward pass; n_keep defaults to the largest column count.
    Synchronous.  Its adapters are not allocated (the backward supplies the
    transposed adapters)."""
    dev = layer.masks.device
    if ws is None:
        ws = workspace(transpose_ws_bytes(layer.N, layer.K), dev)
    if n_keep is None:
        n_keep = transpose_count(layer, ws, stream)
    lt = SalrLayer.empty(layer.K, layer.N, n_keep, 0, 0, dev)
    lt.r_cat = layer.r_cat
    desc = layer.descriptor()
    tdesc = lt.descriptor()
    tdesc.a_cat = tdesc.b_cat = None
    st = _lib().salr_transpose_layer(C.byref(desc), C.byref(tdesc), C.c_void_p(ws.data_ptr()),
                                     ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_transpose_layer")
    return lt


def backward_ws_bytes(N: int, K: int, n_keep_t: int, r_cat: int, M_max: int) -> int:
    out = C.c_size_t()
    _check(_lib().salr_backward_ws_bytes(N, K, n_keep_t, r_cat, M_max, C.byref(out)), "salr_backward_ws_bytes")
    return out.value


def backward_workspace(layer: SalrLayer, lt: SalrLayer, M_max: int, device="cuda"):
    return workspace(backward_ws_bytes(layer.N, layer.K, lt.n_keep, layer.r_cat, M_max), device)


def linear_backward(layer: SalrLayer, lt: SalrLayer, X, dY, dX=None, dA=None, dB=None, ws=None,
                    need_dx: bool = True, stream=None, check: bool = False):
    """dX = dY W_s + (dY B_cat^T) A_cat^T (bf16 [M][K], or None when
    need_dx is False), dA = grad of a_cat as stored (float [r_cat][K]) and
    dB = grad of b_cat as stored (float [N][r_cat]) on the GPU
    (asynchronous on `stream`).  lt is transpose_layer(layer)."""
    import torch

    X = _as_bf16_bits(X, "X")
    dY = _as_bf16_bits(dY, "dY")
    M = X.shape[0]
    if X.dim() != 2 or X.shape[1] != layer.K or tuple(dY.shape) != (M, layer.N):
        raise ValueError("X must be [M][K] and dY [M][N]")
    dev = X.device
    if need_dx and dX is None:
        dX = torch.empty((M, layer.K), dtype=torch.bfloat16, device=dev)
    r = layer.r_cat
    if dA is None:
        dA = torch.empty((r, layer.K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((layer.N, r), dtype=torch.float32, device=dev)
    if ws is None:
        ws = backward_workspace(layer, lt, M, dev)
    desc = layer.descriptor()
    tdesc = lt.descriptor()
    tdesc.a_cat = tdesc.b_cat = None
    ptr = lambda t, n: C.c_void_p(_dev_ptr(t, n)) if (t is not None and t.numel()) else None
    st = _lib().salr_linear_backward(C.byref(desc), C.byref(tdesc), ptr(X, "X"), ptr(dY, "dY"), M,
                                     ptr(dX, "dX") if need_dx else None, ptr(dA, "dA"), ptr(dB, "dB"),
                                     C.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_linear_backward")
    if check and wait_error(ws, stream):
        raise WaitTimeout("salr_linear_backward: a bounded wait timed out (workspace error word set)")
    return (dX if need_dx else None), dA, dB


def moe_query_sizes(E: int, N: int, K: int, n_keep: int, r_cat: int, T_max: int) -> dict:
    out = salr_moe_sizes_t()
    _check(_lib().salr_moe_query_sizes(E, N, K, n_keep, r_cat, T_max, C.byref(out)), "salr_moe_query_sizes")
    return {f: getattr(out, f) for f, _ in salr_moe_sizes_t._fields_}


@dataclass
class SalrMoE:
    """E experts of one shape, each its own encoding, in five stacked device
    buffers at the library's per-expert strides (include/salr.h,
    salr_moe_layer_t)."""

    E: int
    N: int
    K: int
    n_keep: int
    r_cat: int
    masks: object
    values: object
    offsets: object
    a_cat: object
    b_cat: object

    @classmethod
    def empty(cls, E, N, K, n_keep, r_cat, device="cuda"):
        import torch

        sz = moe_query_sizes(E, N, K, n_keep, r_cat, 0)
        z = lambda nbytes: torch.zeros(max(int(nbytes), 256) // 2, dtype=torch.int16, device=device)
        return cls(E, N, K, n_keep, r_cat, masks=z(sz["masks_bytes"]), values=z(sz["values_bytes"]),
                   offsets=z(sz["offsets_bytes"]), a_cat=z(sz["a_cat_bytes"]), b_cat=z(sz["b_cat_bytes"]))

    def descriptor(self) -> salr_moe_layer_t:
        d = salr_moe_layer_t()
        d.E, d.N, d.K, d.n_keep, d.r_cat = self.E, self.N, self.K, self.n_keep, self.r_cat
        d.masks, d.values, d.offsets = self.masks.data_ptr(), self.values.data_ptr(), self.offsets.data_ptr()
        d.a_cat = self.a_cat.data_ptr() if self.r_cat else None
        d.b_cat = self.b_cat.data_ptr() if self.r_cat else None
        return d

    def expert(self, e: int) -> salr_layer_t:
        """Expert e's layer descriptor (views into the stacked buffers)."""
        out = salr_layer_t()
        d = self.descriptor()
        _check(_lib().salr_moe_expert(C.byref(d), e, C.byref(out)), "salr_moe_expert")
        return out

    def set_expert(self, e: int, masks, values, offsets, a_cat, b_cat):
        """Upload expert e's encoding from numpy arrays in the stored layout
        (uint64 masks, uint16 values [N][n_keep], uint32 offsets, uint16 a_cat
        [r_cat][K], b_cat [N][r_cat])."""
        import numpy as np

        sz = moe_query_sizes(self.E, self.N, self.K, self.n_keep, self.r_cat, 0)
        for buf, arr, stride, esize in ((self.masks, masks, sz["masks_stride"], 8),
                                        (self.values, values, sz["values_stride"], 2),
                                        (self.offsets, offsets, sz["offsets_stride"], 4),
                                        (self.a_cat, a_cat, sz["a_cat_stride"], 2),
                                        (self.b_cat, b_cat, sz["b_cat_stride"], 2)):
            flat = np.ascontiguousarray(arr).reshape(-1).view(np.int16)
            if flat.size == 0:
                continue
            start = e * stride * esize // 2
            import torch
            buf[start:start + flat.size].copy_(torch.from_numpy(flat))


def moe_encode_expert(moe: SalrMoE, e: int, W, r_svd: int, lora_A=(), lora_B=(), ws=None, stream=None):
    """salr_encode expert e's weight W (bf16 [N][K]) in place into the
    stacked buffers (r_svd + the LoRA ranks must equal moe.r_cat)."""
    W = _as_bf16_bits(W, "W")
    if tuple(W.shape) != (moe.N, moe.K):
        raise ValueError("W must be [N][K]")
    return _encode_into(moe.expert(e), W, moe.n_keep, r_svd, lora_A, lora_B, None, None, 0, ws, stream)


def moe_workspace(moe: SalrMoE, T_max: int, device="cuda"):
    return workspace(moe_query_sizes(moe.E, moe.N, moe.K, moe.n_keep, moe.r_cat, T_max)["forward_ws_bytes"], device)


def moe_forward(moe: SalrMoE, X, expert_offsets, Y=None, m_cap: int = 0, ws=None, stream=None):
    """Grouped forward: rows [off[e], off[e+1]) of X (bf16 [T][K]) through
    expert e; expert_offsets is a device int32 tensor [E + 1].  Returns Y
    bf16 [T][N] (asynchronous on `stream`)."""
    import torch

    X = _as_bf16_bits(X, "X")
    T = X.shape[0]
    if X.dim() != 2 or X.shape[1] != moe.K:
        raise ValueError("X must be [T][K]")
    if expert_offsets.dtype != torch.int32 or expert_offsets.numel() != moe.E + 1:
        raise ValueError("expert_offsets must be int32 [E + 1]")
    if Y is None:
        Y = torch.empty((T, moe.N), dtype=torch.bfloat16, device=X.device)
    if ws is None:
        ws = moe_workspace(moe, T, X.device)
    d = moe.descriptor()
    st = _lib().salr_moe_forward(C.byref(d), C.c_void_p(_dev_ptr(X, "X")) if T else None, T,
                                 C.c_void_p(_dev_ptr(expert_offsets, "expert_offsets")), m_cap,
                                 C.c_void_p(_dev_ptr(Y, "Y")) if T else None, C.c_void_p(ws.data_ptr()),
                                 ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "salr_moe_forward")
    return Y


def probe_stream_read(src, sink, workgroups: int, stream=None):
    """Read all of the device tensor `src` once (include/salr_probe.h);
    `sink` is a device tensor of at least `workgroups` int32."""
    nbytes = src.numel() * src.element_size()
    _check(_lib().salr_probe_stream_read(C.c_void_p(_dev_ptr(src, "src")), nbytes,
                                         C.c_void_p(_dev_ptr(sink, "sink")), workgroups, _stream_ptr(stream)),
           "salr_probe_stream_read")
    return nbytes


def probe_mfma(out, workgroups: int, iters: int, shape: int, stream=None):
    """Matrix-core peak loop (include/salr_probe.h); returns its flop count.
    `out` is a device float tensor of at least `workgroups` entries."""
    _check(_lib().salr_probe_mfma(C.c_void_p(_dev_ptr(out, "out")), workgroups, iters, shape, _stream_ptr(stream)),
           "salr_probe_mfma")
    return workgroups * 4 * iters * 131072
