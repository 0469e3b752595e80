"""CPU oracle for the SALR linear layer (encode, decode, forward).

TEST INFRASTRUCTURE ONLY: a plain, slow, float64 NumPy definition of what the
SALR hot path computes, used to check the HIP path.  Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it; the
product library never does, and this package imports nothing from the
product package.

Parity status of each function (what pins it, see tests/test_oracle_*.py):
  bf16.f64_to_bits / bits_to_f64   pinned: torch conversion, hand cases
  salr.select_keep                 pinned: brute-force pairwise ranking
  salr.pack_masks / pack_values / block_offsets / decode_dense
                                   pinned: bitwise round trip, per-bit loop
  salr.truncated_svd / residual_factors
                                   pinned: Eckart-Young, the per-entry MSE
                                   bound (1 - r/min(N,K)), full-rank case
  salr.encode R_energy / tail_energy
                                   pinned two-sided: a residual whose
                                   singular values are known in closed form
                                   (total and discarded energy at several
                                   ranks), nothing pruned, a planted
                                   undiscounted tail
  salr.forward                     pinned: per-set-bit triple loop, X = I
  salr.fuse                        pinned: fused forward = the parts', a
                                   planted misplaced block
  nf4.nf4_levels / quantize / dequantize / pack_codes
                                   pinned: normal-CDF spacing of the levels,
                                   brute-force nearest level, exact round
                                   trips, the per-block error bound, planted
                                   mistakes
  backward.backward                pinned: exact finite differences of the
                                   forward, a planted missing term
  backward.transpose_encoding      pinned: the dense transpose, bit for bit
  moe.grouped_forward              pinned: per-token brute force from the
                                   original weights, planted boundary shift
                                   and expert swap
  The pages print no worked example and no intermediate values, so no
  function is pinned to a number printed on the pages.
"""

from . import backward, bf16, moe, nf4, salr  # noqa: F401
