"""Write the residual-spectrum fixtures used by the full-size encode tests.

For each full-size workload: draw W (the seeded generator shared by both
sides), select the kept set with the oracle (magnitude, ties to the lower
column), form the pruning residual R = W - W_s, and record LAPACK's singular
values of R: the top r_svd of them, the discarded tail energy
sum_{i > r_svd} sigma_i^2 (the Eckart-Young optimum of the rank-r_svd
factorization) and ||R||_F^2.  Source: gist.science summary of
"Sparsity-Aware Low-Rank Representation for Efficient Fine-Tuning of Large
Language Models", Methodology 2 (residual and its truncated SVD).

Only the oracle and the input generator are called.  Usage (from the
repository root): python tests/golden/make_svd_golden.py [workload ...]
"""

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import salr as osl  # noqa: E402
from sparse_rank_linear_amd import synth  # noqa: E402

FULL_SIZE = ["tiny_512", "llama7b_attn_4096", "llama7b_mlp_up_11008", "llama7b_mlp_down_11008",
             "llama3_8b_qo", "llama3_8b_kv", "llama3_8b_gate_up", "llama3_8b_down",
             "l70b_up_s50", "l70b_up_s60", "l70b_up_s70", "l70b_down_s50", "l70b_down_s60", "l70b_down_s70"]


def spectrum(name):
    wl = synth.WORKLOADS[name]
    W = synth.make_inputs(wl, with_x=False).W
    keep = osl.select_keep(W, wl.n_keep)
    del W
    R = osl.residual(synth.make_inputs(wl, with_x=False).W, keep)
    del keep
    energy = float(np.sum(R * R))
    S = osl.singular_values(R)
    del R
    top = S[: wl.r_svd]
    return {
        "workload": name, "N": wl.N, "K": wl.K, "n_keep": wl.n_keep, "r_svd": wl.r_svd,
        "w_dist": wl.w_dist, "seed": wl.seed,
        "sigma_top": [float(x) for x in top],
        "tail_energy": float(np.sum(S[wl.r_svd:] ** 2)),
        "R_energy": energy,
    }


if __name__ == "__main__":
    names = sys.argv[1:] or FULL_SIZE
    for name in names:
        t = time.time()
        out = spectrum(name)
        with open(os.path.join(HERE, f"svd_{name}.json"), "w") as f:
            json.dump(out, f, indent=1)
        print(name, f"{time.time() - t:.1f} s", flush=True)
