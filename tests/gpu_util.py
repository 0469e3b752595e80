"""Helpers shared by the GPU tests: moving bf16 bit arrays between numpy and
the device, uploading an oracle encoding in the library's stored layout,
and the forward tolerance."""

import sys

import numpy as np

from oracle import bf16 as ob
from oracle import salr as osl

# Y tolerance: max_ij |Y_gpu - Y| / max(|Y_ij|, rms(Y)) (bf16 inputs, fp32
# accumulation, bf16 T and Y).
TOL_MAX_REL = 2e-2
# normwise ||Y_gpu - Y|| / ||Y||: bf16 rounding of Y (2^-9 relative at
# worst, ~1.1e-3 rms) plus bf16 rounding of X A_cat.
TOL_NORMWISE = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_host_bits(t):
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def upload_encoded(enc: "osl.Encoded", K: int, r_svd: int):
    import sparse_rank_linear_amd as srl

    return srl.SalrLayer.from_arrays(enc.masks, enc.values, enc.offsets, enc.A_cat.T.copy(), enc.B_cat.T.copy(),
                                     K, r_svd)


def errors(Y_gpu_bits, Y_ref):
    Yg = ob.bits_to_f64(Y_gpu_bits)
    mr = osl.max_rel_err(Yg, Y_ref)
    nrm = float(np.linalg.norm(Y_ref))
    nw = float(np.linalg.norm(Yg - Y_ref) / nrm) if nrm > 0 else float(np.linalg.norm(Yg))
    return mr, nw


def wait_error(ws) -> int:
    """The forward workspace's wait-timeout word (uint32 at byte offset 8)."""
    import torch

    return int(ws[8:12].cpu().view(torch.int32).item())
