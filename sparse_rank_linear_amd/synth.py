"""Seeded synthetic inputs for SALR linear layers.

This module draws random tensors and nothing else: it holds no step of the
method (no pruning, packing, SVD or product).  Both sides of every parity
check take their inputs from here, so it must stay free of anything either
side computes.

All tensors are bf16 and are returned as their raw 16-bit patterns in numpy
``uint16`` arrays.  Values are drawn in float32 (float64 for Student-t) from a
single ``numpy.random.default_rng(seed)`` and rounded to bf16 by torch's own
dtype conversion.  Draw order within one layer is fixed: W, then every LoRA
pair (A_i then B_i) in adapter order, then X.  Large matrices are drawn in
row chunks so that peak host memory stays near one bf16 copy.

Layouts (row-major):
  W        [N x K]   nn.Linear weight: N = out_features, K = in_features
  lora_A_i [r_i x K] nn.Linear weight of the adapter's down projection
  lora_B_i [N x r_i] nn.Linear weight of the adapter's up projection
  X        [M x K]   activations, one token per row

The workloads mirror the layer shapes on which SALR is evaluated in the
gist.science summary of "Sparsity-Aware Low-Rank Representation for Efficient
Fine-Tuning of Large Language Models" (Experimental Results: Llama2-7B,
Llama3-8B; Methodology part 1: 50% magnitude sparsity of the frozen weight)
and a 70B-shaped heavy-tailed stress layer.  Trained weights and datasets are
not used: Gaussian (or Student-t) values of the same shapes stand in.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_CHUNK_ELEMS = 1 << 23  # elements drawn per chunk


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) via torch's conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw(rng: np.random.Generator, shape, dist: str, scale: float) -> np.ndarray:
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        if dist == "normal":
            x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
            x *= np.float32(scale)
        elif dist == "t3":
            x = (scale * rng.standard_t(3, size=(r1 - r0, cols))).astype(np.float32)
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        out[r0:r1] = _to_bf16_bits(x)
    return out


def n_keep_for(K: int, sparsity: float) -> int:
    """Weights kept per row when a fraction `sparsity` of each row is pruned:
    K - floor(sparsity*K), evaluated in float64 with a 1e-6 guard so that
    e.g. 0.6*8192 = 4915.2 prunes 4915 and 0.5*K prunes exactly K/2."""
    return K - int(math.floor(sparsity * K + 1e-6))


@dataclass
class Workload:
    """One SALR layer workload: shapes, distributions and adapter ranks."""

    name: str
    N: int
    K: int
    M: int
    sparsity: float = 0.5
    r_svd: int = 64
    lora_ranks: tuple = (16,)
    w_dist: str = "normal"
    w_scale: float = 0.02
    lora_scale: float = 0.01
    x_scale: float = 1.0
    seed: int = 0

    @property
    def n_keep(self) -> int:
        return n_keep_for(self.K, self.sparsity)

    @property
    def r_cat(self) -> int:
        return self.r_svd + sum(self.lora_ranks)


@dataclass
class LayerInputs:
    W: np.ndarray                      # uint16 [N x K]
    lora_A: list = field(default_factory=list)  # uint16 [r_i x K]
    lora_B: list = field(default_factory=list)  # uint16 [N x r_i]
    X: np.ndarray | None = None        # uint16 [M x K]


def make_inputs(wl: Workload, M: int | None = None, with_x: bool = True) -> LayerInputs:
    """Draw W, the LoRA pairs and X for `wl` (X has M rows, default wl.M)."""
    rng = np.random.default_rng(wl.seed)
    W = _draw(rng, (wl.N, wl.K), wl.w_dist, wl.w_scale)
    As, Bs = [], []
    for r in wl.lora_ranks:
        As.append(_draw(rng, (r, wl.K), "normal", wl.lora_scale))
        Bs.append(_draw(rng, (wl.N, r), "normal", wl.lora_scale))
    X = None
    if with_x:
        m = wl.M if M is None else M
        X = _draw(rng, (m, wl.K), "normal", wl.x_scale)
    return LayerInputs(W=W, lora_A=As, lora_B=Bs, X=X)


def make_x(K: int, M: int, seed: int) -> np.ndarray:
    """Activations alone, N(0,1), from their own seed."""
    return _draw(np.random.default_rng(seed), (M, K), "normal", 1.0)


def make_w(N: int, K: int, seed: int, dist: str = "normal", scale: float = 0.02) -> np.ndarray:
    """A weight matrix alone, from its own seed."""
    return _draw(np.random.default_rng(seed), (N, K), dist, scale)


# Workloads.  "tiny" is the small case the oracle finishes in seconds; the
# 4096x4096 decode-regime layer is the headline; the others are parity cases.
WORKLOADS = {
    "tiny_512": Workload("tiny_512", N=512, K=512, M=16, r_svd=16, lora_ranks=(8,)),
    "llama7b_attn_4096": Workload("llama7b_attn_4096", N=4096, K=4096, M=16),
    "llama7b_mlp_up_11008": Workload("llama7b_mlp_up_11008", N=11008, K=4096, M=2048),
    "llama7b_mlp_down_11008": Workload("llama7b_mlp_down_11008", N=4096, K=11008, M=2048),
    "llama3_8b_qo": Workload("llama3_8b_qo", N=4096, K=4096, M=16, lora_ranks=(16, 16, 16)),
    "llama3_8b_kv": Workload("llama3_8b_kv", N=1024, K=4096, M=16, lora_ranks=(16, 16, 16)),
    "llama3_8b_gate_up": Workload("llama3_8b_gate_up", N=14336, K=4096, M=16, lora_ranks=(16, 16, 16)),
    "llama3_8b_down": Workload("llama3_8b_down", N=4096, K=14336, M=16, lora_ranks=(16, 16, 16)),
    "l70b_up_s50": Workload("l70b_up_s50", N=28672, K=8192, M=8192, sparsity=0.5, r_svd=128,
                            lora_ranks=(32,), w_dist="t3"),
    "l70b_down_s50": Workload("l70b_down_s50", N=8192, K=28672, M=8192, sparsity=0.5, r_svd=128,
                              lora_ranks=(32,), w_dist="t3"),
}
for _s in (0.6, 0.7):
    _tag = int(round(_s * 100))
    WORKLOADS[f"l70b_up_s{_tag}"] = Workload(f"l70b_up_s{_tag}", N=28672, K=8192, M=8192, sparsity=_s,
                                             r_svd=128, lora_ranks=(32,), w_dist="t3")
    WORKLOADS[f"l70b_down_s{_tag}"] = Workload(f"l70b_down_s{_tag}", N=8192, K=28672, M=8192,
                                               sparsity=_s, r_svd=128, lora_ranks=(32,), w_dist="t3")


# Mixture-of-experts expert layers in the decode regime (the MoE models of
# the same summary's Experimental Results: Mixtral-8x7B and
# DeepSeek-V2-Lite), each expert its own weight and adapters.
@dataclass
class MoeWorkload:
    name: str
    E: int          # experts
    N: int
    K: int
    tokens: int     # tokens in the batch
    top_k: int      # experts per token
    sparsity: float = 0.5
    r_svd: int = 64
    lora_ranks: tuple = (16,)
    seed: int = 0

    @property
    def n_keep(self) -> int:
        return n_keep_for(self.K, self.sparsity)

    @property
    def r_cat(self) -> int:
        return self.r_svd + sum(self.lora_ranks)

    def expert_workload(self, e: int) -> Workload:
        """Expert e's layer (its own seed)."""
        return Workload(f"{self.name}_e{e}", N=self.N, K=self.K, M=0, sparsity=self.sparsity, r_svd=self.r_svd,
                        lora_ranks=self.lora_ranks, seed=self.seed * 1000 + e + 1)


MOE_WORKLOADS = {
    # expert up/gate projection 14336 x 4096, 8 experts, top-2 of 16 tokens
    "mixtral_8x7b_w1": MoeWorkload("mixtral_8x7b_w1", E=8, N=14336, K=4096, tokens=16, top_k=2),
    # routed expert up projection 1408 x 2048, 64 experts, top-6 of 16 tokens
    "deepseek_v2_lite_up": MoeWorkload("deepseek_v2_lite_up", E=64, N=1408, K=2048, tokens=16, top_k=6),
}


def make_routing(E: int, tokens: int, top_k: int, seed: int):
    """A seeded random routing: each token picks top_k distinct experts
    uniformly.  Returns (counts per expert, int64 [tokens*top_k] token index
    of each grouped row: the rows of expert 0 first, then expert 1, ...)."""
    rng = np.random.default_rng(seed)
    picks = np.stack([rng.choice(E, top_k, replace=False) for _ in range(tokens)])  # [tokens x top_k]
    expert = picks.reshape(-1)
    token = np.repeat(np.arange(tokens), top_k)
    order = np.argsort(expert, kind="stable")
    counts = np.bincount(expert, minlength=E)
    return counts, token[order]
