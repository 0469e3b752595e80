"""SALR linear-layer benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: a Llama-7B attention projection in the decode regime --
W 4096x4096 bf16 ~N(0, 0.02^2), 50% per-row magnitude sparsity stored as
bitmap + packed values, residual truncated-SVD rank 64 + one LoRA of rank 16
(r_cat 80), X 16x4096 bf16 ~N(0, 1).  The layer is encoded on the GPU
(salr_encode), then cloned into 32 distinct copies (646 MB, more than twice
the 256 MB Infinity Cache) that the timed steps cycle through, so every step
streams its weights from HBM.

One step = one salr_linear_forward call over 16 tokens.  The K timed steps
(and, separately, the W warm-up steps) are captured in a HIP graph and
replayed, so the host's launch rate does not throttle the 3-6 us kernel;
HIP events on the launch stream bracket the timed replay.

Printed JSON fields beyond the common contract:
  roofline      the fused few-row kernel against HBM peak: algorithmic bytes
                per launch (compressed weight + X + Y) / mean launch time
  cpu_baseline  the float64 NumPy oracle's forward on the same layer shape
                (host cores), for context
  sweep         the same measurement at 1, 4 and 16 tokens
  prefill       a many-token case (11008x4096, 2048 tokens) against the bf16
                matrix-core peak (dense-equivalent flops), for context
  encode        wall time of salr_encode for the headline layer

    python bench.py --configs

prints instead one JSON line per workload and token count of the synthetic
workload table (sparse_rank_linear_amd/synth.py): the layer encoded on the
GPU, enough rotating copies to exceed the Infinity Cache, the graph-replayed
forward time, compressed-weight GB/s and the fraction of the roofline that
bounds the regime (HBM for <= 16 tokens, bf16 matrix cores above).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SALR linear fwd TFLOP/s (dense-equiv) + compressed-weight GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
COPIES = 32
# Sources that decide what the few-row forward kernel does and how it is
# launched; a stored counter measurement counts only while they are unchanged.
FWD_SMALL_SOURCES = ("fwd_small.hip", "salr_device.hpp", "salr_kernels.hpp", "salr_api.cpp")
PROFILE_JSON = os.path.join(ROOT, "profiles", "fwd_small_llama7b_attn_4096x4096_decode.json")


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    paths = [os.path.join(ROOT, "sparse_rank_linear_amd", "csrc", n) for n in FWD_SMALL_SOURCES]
    paths.append(os.path.join(ROOT, "sparse_rank_linear_amd", "build.py"))  # compile flags
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings), or None when the kernel
    sources changed since they were taken."""
    try:
        with open(PROFILE_JSON) as f:
            prof = json.load(f)
    except OSError:
        return None
    if prof.get("kernel_source_hash") != kernel_source_hash():
        return None
    return int(prof["traffic_bytes_per_launch"])


def _dev_bits(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _timed_graph(fn_list, steps: int):
    """Capture `steps` calls (cycling fn_list) into one graph; return a
    replay function and the graph."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(steps):
            fn_list[j % len(fn_list)]()
    return g


def _time_replay(g) -> float:
    import torch

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


def measure_decode(layers, X, ws, steps, warmup):
    """Mean seconds per forward call over `steps` graph-replayed calls."""
    import torch
    import sparse_rank_linear_amd as srl

    M = X.shape[0]
    Y = torch.empty((M, layers[0].N), dtype=torch.bfloat16, device=X.device)
    fns = [(lambda L=L: srl.linear_forward(L, X, Y=Y, ws=ws)) for L in layers]
    for j in range(warmup):  # eager warm-up steps
        fns[j % len(fns)]()
    torch.cuda.synchronize()
    g = _timed_graph(fns, steps)
    g.replay()  # first replay uploads the graph; untimed
    torch.cuda.synchronize()
    return _time_replay(g) / steps


def run_configs(dev):
    """One JSON line per (workload, token count) of the synthetic table."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    for name, wl in synth.WORKLOADS.items():
        inp = synth.make_inputs(wl, with_x=False)
        W = _dev_bits(inp.W, dev)
        As = [_dev_bits(a, dev) for a in inp.lora_A]
        Bs = [_dev_bits(b, dev) for b in inp.lora_B]
        layer, _ = srl.encode(W, wl.n_keep, wl.r_svd, As, Bs)  # (first call: warm-up)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        layer, _ = srl.encode(W, wl.n_keep, wl.r_svd, As, Bs)
        torch.cuda.synchronize()
        encode_ms = (time.perf_counter() - t0) * 1e3
        del W, As, Bs
        cbytes = layer.compressed_bytes()
        copies = max(2, -(-600_000_000 // cbytes))
        layers = [layer] + [layer.clone() for _ in range(copies - 1)]
        tokens = sorted({1, 16, wl.M}) if wl.M <= 16 else [wl.M]
        ws = srl.forward_workspace(layer, max(tokens))
        for M in tokens:
            X = _dev_bits(synth.make_x(wl.K, M, seed=11), dev)
            t = measure_decode(layers, X, ws, 32, 4)
            rec = {"workload": name, "N": wl.N, "K": wl.K, "n_keep": wl.n_keep, "r_cat": wl.r_cat, "M": M,
                   "us": round(t * 1e6, 2), "compressed_GBs": round(cbytes / t / 1e9, 1),
                   "tflops_dense_equiv": round(2 * M * wl.N * wl.K / t / 1e12, 2), "encode_ms": round(encode_ms, 1)}
            if M <= 16:
                rec["hbm_frac"] = round((cbytes + 2 * M * (wl.K + wl.N)) / t / 1e9 / HBM_PEAK_GBS, 4)
            else:
                rec["mfma_frac_dense_equiv"] = round(2 * M * wl.N * wl.K / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
            print(json.dumps(rec), flush=True)
        del layers, layer, ws
        torch.cuda.empty_cache()


# Projections that read the same input, fused into one call (salr_fuse_layers):
# name -> [(workload, rows)].  Parts of one group share K, sparsity and ranks;
# a part with fewer rows than its workload takes the workload's first rows
# (the Llama-7B attention block's k/v projections are 4096 x 4096 too; the
# Llama-3-8B ones are 1024 x 4096).
FUSED_GROUPS = {
    "llama7b_qkv": [("llama7b_attn_4096", 4096)] * 3,
    "llama3_8b_kv": [("llama3_8b_kv", 1024)] * 2,
    "llama3_8b_gate_up": [("llama3_8b_gate_up", 14336)] * 2,
}


def run_fused(dev, only=None, tokens=None):
    """One JSON line per (group, token count): the fused layer against the
    parts called one after another, same inputs, rotating copies."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    for gname, group in FUSED_GROUPS.items():
        if only and gname != only:
            continue
        parts = []
        for i, (wname, rows) in enumerate(group):
            wl = synth.WORKLOADS[wname]
            wl = synth.Workload(**{**wl.__dict__, "N": rows, "seed": wl.seed + i})
            inp = synth.make_inputs(wl, with_x=False)
            layer, _ = srl.encode(_dev_bits(inp.W, dev), wl.n_keep, wl.r_svd,
                                  [_dev_bits(a, dev) for a in inp.lora_A], [_dev_bits(b, dev) for b in inp.lora_B])
            parts.append(layer)
        fused = srl.fuse(parts)
        torch.cuda.synchronize()
        K = fused.K
        for M in (tokens,) if tokens else (1, 16, 2048):
            X = _dev_bits(synth.make_x(K, M, seed=11), dev)
            copies = 1 if M > 16 else max(2, -(-600_000_000 // fused.compressed_bytes()))
            sep = 0.0
            for p in parts:
                ls = [p] + [p.clone() for _ in range(copies - 1)]
                sep += measure_decode(ls, X, srl.forward_workspace(p, M), 32, 4)
                del ls
            fl = [fused] + [fused.clone() for _ in range(copies - 1)]
            t = measure_decode(fl, X, srl.forward_workspace(fused, M), 32, 4)
            del fl
            # algorithmic bytes: the parts' encodings (the zero blocks of the
            # fused B_cat are not needed), X and Y
            alg = sum(p.compressed_bytes() for p in parts) + 2 * M * K + 2 * M * fused.N
            line = {"fused": gname, "N": fused.N, "K": K, "r_cat": fused.r_cat, "M": M,
                    "separate_us": round(sep * 1e6, 2), "fused_us": round(t * 1e6, 2),
                    "speedup": round(sep / t, 3), "algorithmic_bytes": alg,
                    "fused_GBs": round(alg / t / 1e9, 1), "hbm_frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4)}
            if M > 16:
                tf = 2 * M * fused.N * K / t / 1e12
                line.update(tflops_dense_equiv=round(tf, 2), mfma_frac_dense_equiv=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
            print(json.dumps(line), flush=True)
            torch.cuda.empty_cache()
        del parts, fused


def run_layer(dev, name: str, M: int, steps: int, warmup: int):
    """One workload of the synthetic table at M tokens: GPU encode, then
    `steps` graph-replayed forward calls (for kernel traces and counters).
    One JSON line with the mean time per call."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, with_x=False)
    layer, _ = srl.encode(_dev_bits(inp.W, dev), wl.n_keep, wl.r_svd, [_dev_bits(a, dev) for a in inp.lora_A],
                          [_dev_bits(b, dev) for b in inp.lora_B])
    torch.cuda.synchronize()
    cbytes = layer.compressed_bytes()
    copies = 1 if M > 16 else max(2, -(-600_000_000 // cbytes))
    layers = [layer] + [layer.clone() for _ in range(copies - 1)]
    X = _dev_bits(synth.make_x(wl.K, M, seed=11), dev)
    t = measure_decode(layers, X, srl.forward_workspace(layer, M), steps, warmup)
    print(json.dumps({"workload": name, "N": wl.N, "K": wl.K, "r_cat": wl.r_cat, "M": M, "steps": steps,
                      "us": round(t * 1e6, 2), "tflops_dense_equiv": round(2 * M * wl.N * wl.K / t / 1e12, 2),
                      "compressed_GBs": round(cbytes / t / 1e9, 1)}), flush=True)


def cpu_baseline(wl, budget_s: float = 12.0):
    """The oracle's float64 forward on the headline shape, on host cores."""
    from oracle import salr as osl
    from sparse_rank_linear_amd import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    inp = synth.make_inputs(wl)
    # the residual adapter's place is taken by an extra LoRA of the same
    # rank: the forward's cost depends only on r_cat
    rng = np.random.default_rng(1)
    As = [synth._to_bf16_bits(rng.standard_normal((wl.r_cat, wl.K), dtype=np.float32) * np.float32(0.01))]
    Bs = [synth._to_bf16_bits(rng.standard_normal((wl.N, wl.r_cat), dtype=np.float32) * np.float32(0.01))]
    enc = osl.encode(inp.W, wl.n_keep, 0, As, Bs)
    reps, t0 = 0, time.perf_counter()
    while True:
        osl.forward(inp.X, enc.masks, enc.values, wl.K, enc.A_cat, enc.B_cat)
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 50:
            break
    per = (time.perf_counter() - t0) / reps
    kw, ng = -(-wl.K // 64), -(-wl.K // 1024)
    cbytes = wl.N * kw * 8 + wl.N * wl.n_keep * 2 + wl.N * ng * 4 + 2 * wl.r_cat * (wl.K + wl.N)
    return {
        "value": round(cbytes / per / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{reps} float64 oracle forwards (decode to dense + matmul) of the {wl.N}x{wl.K} layer, "
                  f"{wl.M} tokens, r_cat {wl.r_cat}; {per * 1e3:.1f} ms each",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-extra", action="store_true", help="headline line only (no sweep/prefill/cpu)")
    ap.add_argument("--layer", default=None,
                    help="time one workload of the synthetic table (with --tokens) and exit")
    ap.add_argument("--tokens", type=int, default=None,
                    help="token count for --layer (default 16) or --fused (default 1, 16 and 2048)")
    ap.add_argument("--group", default=None, choices=sorted(FUSED_GROUPS),
                    help="with --fused: only this projection group")
    ap.add_argument("--fused", action="store_true",
                    help="time fused projections (salr_fuse_layers) against separate calls, then exit")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload of the synthetic table instead of the headline line")
    ap.add_argument("--probe", choices=["copy"], default=None,
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer's multi-GPU "
              "sharding is described but not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    dev = torch.device("cuda:0")
    if args.probe == "copy":
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy", "bytes_read_per_launch": a.numel() * 2,
                          "bytes_written_per_launch": a.numel() * 2, "launches": 5}))
        return

    if args.layer:
        run_layer(dev, args.layer, args.tokens or 16, args.steps, args.warmup)
        return
    if args.fused:
        run_fused(dev, args.group, args.tokens)
        return
    if args.configs:
        run_configs(dev)
        return

    wl = synth.WORKLOADS["llama7b_attn_4096"]
    inp = synth.make_inputs(wl)
    W = _dev_bits(inp.W, dev)
    As = [_dev_bits(a, dev) for a in inp.lora_A]
    Bs = [_dev_bits(b, dev) for b in inp.lora_B]
    layer, _ = srl.encode(W, wl.n_keep, wl.r_svd, As, Bs)  # (first call also loads the code objects)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    layer, _ = srl.encode(W, wl.n_keep, wl.r_svd, As, Bs)
    torch.cuda.synchronize()
    encode_s = time.perf_counter() - t0
    layers = [layer] + [layer.clone() for _ in range(COPIES - 1)]
    ws = srl.forward_workspace(layer, 16384)
    cbytes = layer.compressed_bytes()

    def line_for(M, steps, warmup):
        X = _dev_bits(synth.make_x(wl.K, M, seed=11), dev)
        t = measure_decode(layers, X, ws, steps, warmup)
        algo = cbytes + 2 * M * (wl.K + wl.N)
        return t, algo

    t, algo = line_for(wl.M, args.steps, args.warmup)
    M = wl.M
    achieved = algo / t / 1e9
    out = {
        "metric": METRIC,
        "value": round(cbytes / t / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama7b_attn_4096x4096_decode", "N": wl.N, "K": wl.K, "M": M,
                   "sparsity": wl.sparsity, "n_keep": wl.n_keep, "r_svd": wl.r_svd, "r_cat": wl.r_cat,
                   "rotating_copies": COPIES, "compressed_weight_bytes": cbytes},
        "tflops_dense_equiv": round(2 * M * wl.N * wl.K / t / 1e12, 4),
        "tflops_effective": round(2 * M * (wl.N * wl.n_keep + wl.r_cat * (wl.K + wl.N)) / t / 1e12, 4),
        "roofline": {"bound": "hbm", "kernel": "fwd_small_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic()},
        "encode": {"seconds": round(encode_s, 4), "iters": 24, "oversample": 32, "call": "second"},
    }
    if not args.no_extra:
        sweep = []
        for m in (1, 4, 16):
            tm, al = line_for(m, 128, 16)
            sweep.append({"M": m, "us_per_step": round(tm * 1e6, 3), "compressed_GBs": round(cbytes / tm / 1e9, 1),
                          "hbm_frac": round(al / tm / 1e9 / HBM_PEAK_GBS, 4)})
        out["sweep"] = sweep
        # many-token context: 11008 x 4096, 2048 tokens (matrix-core bound)
        pw = synth.WORKLOADS["llama7b_mlp_up_11008"]
        pin = synth.make_inputs(pw, with_x=False)
        player, _ = srl.encode(_dev_bits(pin.W, dev), pw.n_keep, pw.r_svd, [_dev_bits(a, dev) for a in pin.lora_A],
                               [_dev_bits(b, dev) for b in pin.lora_B])
        del layers
        Xp = _dev_bits(synth.make_x(pw.K, pw.M, seed=12), dev)
        pws = srl.forward_workspace(player, pw.M)
        tp = measure_decode([player], Xp, pws, 20, 3)
        dense = 2 * pw.M * pw.N * pw.K
        out["prefill"] = {"workload": "llama7b_mlp_up_11008x4096_prefill", "M": pw.M, "ms_per_step": round(tp * 1e3, 4),
                          "tflops_dense_equiv": round(dense / tp / 1e12, 2),
                          "mfma_frac_dense_equiv": round(dense / tp / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
