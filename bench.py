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
  us_per_step_stats  median / p10 / p90 of the per-call mean over 10 more
                replays of the timed graph
  checks        the timed run checked: workspace wait-error word clear, the
                timed output equal to an eager call bit for bit, and the same
                launch configuration (with seeded adapters) against the
                oracle on sampled rows; the script exits non-zero if any fails
  measured_peaks  achievable HBM read rate and bf16 matrix-core rate from the
                library's probe kernels; every fraction is also given
                against them
  sweep         the same measurement at 1, 4 and 16 tokens
  prefill       a many-token case (11008x4096, 2048 tokens) against the bf16
                matrix-core peak (dense-equivalent and effective flops)
  l70b_up_s50   the 70B-shaped layer (28672x8192, Student-t, 50%, r_cat 160)
                at 8192 tokens, likewise
  encode        wall time of salr_encode for the headline layer
  qsalr_nf4     the headline layer with NF4 values (QSALR): bytes per weight
                element and the HBM fraction at 16 tokens
  backward      dX, dA_cat, dB_cat of the headline layer at 2048 tokens
                against the bf16 matrix-core peak, and the one-off build of
                the transposed encoding
  moe           grouped expert layers (Mixtral-8x7B and DeepSeek-V2-Lite
                expert shapes, seeded top-k routing of 16 tokens) against
                HBM peak on the routed experts' bytes

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


def measure_decode(layers, X, ws, steps, warmup, reps: int = 0, detail: bool = False):
    """Mean seconds per forward call over `steps` graph-replayed calls (one
    replay: the timed region).  With reps > 0, that many further replays
    give the spread of the per-call mean (median, p10, p90).  With detail,
    returns a dict with those, the output buffer and the last layer called."""
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
    t = _time_replay(g) / steps
    if not detail:
        return t
    extra = [_time_replay(g) / steps for _ in range(reps)]
    q = np.percentile(np.array(extra), [10, 50, 90]) if extra else [t, t, t]
    return {"mean": t, "p10": float(q[0]), "median": float(q[1]), "p90": float(q[2]), "replays": reps,
            "Y": Y, "last_layer": layers[(steps - 1) % len(layers)]}


def measure_peaks(dev):
    """Achievable HBM read rate and bf16 matrix-core rate of this GPU from
    the library's probe kernels (include/salr_probe.h): a 1 GiB buffer (four
    times the Infinity Cache) read once per launch at several grid sizes,
    and independent matrix-core chains in 4 waves per workgroup, 4
    workgroups per CU.  Best of each, timed with events on the launch
    stream."""
    import torch
    import sparse_rank_linear_amd as srl

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3
            best = t if best is None else min(best, t)
        return best

    buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    read = {}
    for wg in (256, 512, 1024, 2048, 4096):
        nbytes = buf.numel()
        t = timed(lambda: srl.probe_stream_read(buf, sink, wg), 5)
        read[wg] = nbytes / t / 1e9
    del buf
    # (the 32x32x16 loop: four accumulator chains, nothing else in the loop)
    out = torch.empty(4096, dtype=torch.float32, device=dev)
    flops = 1024 * 4 * 4000 * 131072
    t = timed(lambda: srl.probe_mfma(out, 1024, 4000, 1), 3)
    # the 16x16x32 form the forward kernels issue, with one wave per SIMD
    # (256 workgroups of 4 waves) as in their matrix-core waves, and with four
    t16 = {wg: flops / timed(lambda wg=wg: srl.probe_mfma(out, wg, 4000 * 1024 // wg, 0), 3) / 1e12
           for wg in (256, 1024)}
    best_wg = max(read, key=read.get)
    return {"hbm_read_GBs": round(read[best_wg], 1), "hbm_read_workgroups": best_wg,
            "hbm_read_by_grid": {str(k): round(v, 1) for k, v in read.items()},
            "mfma_bf16_TFLOPs": round(flops / t / 1e12, 1), "mfma_probe": "v_mfma_f32_32x32x16_bf16",
            "mfma_bf16_16x16x32_TFLOPs": {"1_wave_per_simd": round(t16[256], 1), "4_waves_per_simd": round(t16[1024], 1)}}


def measure_launch_floor(dev, nbytes: int, copies: int, steps: int):
    """What one launch that only reads `nbytes` once costs on this GPU: the
    stream-read probe (include/salr_probe.h) over `copies` rotating buffers of
    that size (more than the Infinity Cache together), graph-replayed and
    timed like the forward, at several grid sizes; and the same probe reading
    16 bytes (the per-launch cost of a graph node with nothing to read).
    Mean seconds per launch."""
    import torch
    import sparse_rank_linear_amd as srl

    nb = (nbytes + 15) // 16 * 16
    pool = torch.zeros(copies * nb, dtype=torch.uint8, device=dev)
    bufs = [pool[j * nb:(j + 1) * nb] for j in range(copies)]
    sink = torch.empty(65536, dtype=torch.int32, device=dev)

    def per_launch(grid, size):
        fns = [(lambda b=b: srl.probe_stream_read(b[:size], sink, grid)) for b in bufs]
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = _timed_graph(fns, steps)
        g.replay()
        torch.cuda.synchronize()
        return min(_time_replay(g) for _ in range(3)) / steps

    by_grid = {grid: per_launch(grid, nb) for grid in (256, 512, 1024, 2048, (nb + 8191) // 8192)}
    empty = per_launch(256, 16)
    del pool, bufs
    best = min(by_grid, key=by_grid.get)
    return {"bytes": nb, "rotating_copies": copies, "read_us_by_grid": {str(k): round(v * 1e6, 3) for k, v in by_grid.items()},
            "best_us": round(by_grid[best] * 1e6, 3), "best_grid": best,
            "best_GBs": round(nb / by_grid[best] / 1e9, 1), "empty_launch_us": round(empty * 1e6, 3)}


def check_timed_output(wl, inp, layer, X_bits, X, ws, Y_timed, last_layer, dev):
    """Checks of the timed run: (1) no bounded wait timed out (workspace
    error word); (2) the timed output equals an eager call on the layer the
    last timed step used, bit for bit (the kernels sum in a fixed order);
    (3) the same launch configuration on this layer's bitmap and values with
    seeded adapters of the same rank against the oracle's float64 forward
    from its own encoding of sampled rows.  Returns a dict of results."""
    import torch
    import sparse_rank_linear_amd as srl
    from oracle import bf16 as ob
    from oracle import salr as osl
    from sparse_rank_linear_amd import synth

    res = {"wait_error": srl.wait_error(ws)}
    Y2 = srl.linear_forward(last_layer, X, ws=ws)
    torch.cuda.synchronize()
    res["timed_equals_eager"] = bool(torch.equal(Y_timed.view(torch.int16), Y2.view(torch.int16)))
    probe = layer.clone()
    a_cat = synth.make_w(wl.r_cat, wl.K, seed=wl.seed + 201, scale=0.01)
    b_cat = synth.make_w(wl.N, wl.r_cat, seed=wl.seed + 202, scale=0.01)
    probe.a_cat.view(torch.int16).copy_(torch.from_numpy(a_cat.view(np.int16)))
    probe.b_cat.view(torch.int16).copy_(torch.from_numpy(b_cat.view(np.int16)))
    Y3 = srl.linear_forward(probe, X, ws=ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(wl.N, 14, replace=False), [0, wl.N - 1]]))
    keep = osl.select_keep(inp.W[rows], wl.n_keep)
    Yref = osl.forward(X_bits, osl.pack_masks(keep), osl.pack_values(inp.W[rows], keep, wl.n_keep), wl.K,
                       a_cat.T, b_cat[rows].T)
    Yg = ob.bits_to_f64(Y3[:, torch.from_numpy(rows).to(dev)].contiguous().view(torch.int16).cpu().numpy()
                        .view(np.uint16))
    res["oracle_max_rel_err"] = float(osl.max_rel_err(Yg, Yref))
    res["wait_error"] = max(res["wait_error"], srl.wait_error(ws))
    res["ok"] = res["wait_error"] == 0 and res["timed_equals_eager"] and res["oracle_max_rel_err"] <= 2e-2
    return res


def dense_context(dev, N, K, r_cat, M, steps, warmup, rotate_bytes=600_000_000):
    """Context only: the same shape computed densely with torch's bf16
    products, Y = X W^T + (X A_cat) B_cat, through the vendor GEMM library
    (not inspected).  With M <= 16 the dense weight rotates over copies
    totalling more than the Infinity Cache, as the compressed one does.
    Graph-replayed like the forward; mean seconds per call."""
    import torch

    copies = max(1, -(-rotate_bytes // (2 * N * K))) if M <= 16 else 1
    gen = torch.Generator(device=dev).manual_seed(21)
    rnd = lambda *shape: (torch.randn(shape, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    Ws = [rnd(N, K) for _ in range(copies)]
    A, B, X = rnd(K, r_cat), rnd(r_cat, N), rnd(M, K)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    T = torch.empty((M, r_cat), dtype=torch.bfloat16, device=dev)

    def call(W):
        torch.mm(X, W.t(), out=Y)
        torch.mm(X, A, out=T)
        Y.addmm_(T, B)

    fns = [(lambda W=W: call(W)) for W in Ws]
    for j in range(max(warmup, copies)):
        fns[j % len(fns)]()
    torch.cuda.synchronize()
    g = _timed_graph(fns, steps)
    g.replay()
    torch.cuda.synchronize()
    t = min(_time_replay(g) for _ in range(3)) / steps
    del g, Ws, A, B, X, Y, T
    torch.cuda.empty_cache()
    return {"us": round(t * 1e6, 3), "dense_weight_copies": copies,
            "dense_GBs": round((2 * N * K + 2 * r_cat * (K + N) + 2 * M * (K + N)) / t / 1e9, 1),
            "dense_tflops": round(2 * M * N * K / t / 1e12, 2)}


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
        if name.startswith("llama3_8b_"):
            tokens = [1, 16, 256, 4096]  # the Llama-3-8B block from decode to prefill
        ws = srl.forward_workspace(layer, max(tokens))
        for M in tokens:
            X = _dev_bits(synth.make_x(wl.K, M, seed=11), dev)
            steps = 32 if M <= 256 else 8
            t = measure_decode(layers if M <= 256 else [layer], X, ws, steps, 4)
            rec = {"workload": name, "N": wl.N, "K": wl.K, "n_keep": wl.n_keep, "r_cat": wl.r_cat, "M": M,
                   "us": round(t * 1e6, 2), "compressed_GBs": round(cbytes / t / 1e9, 1),
                   "tflops_dense_equiv": round(2 * M * wl.N * wl.K / t / 1e12, 2), "encode_ms": round(encode_ms, 1)}
            # bytes bound at few tokens, matrix cores at many; at 256 tokens the
            # arithmetic intensity sits near the ridge, so both fractions
            if M <= 256:
                rec["hbm_frac"] = round((cbytes + 2 * M * (wl.K + wl.N)) / t / 1e9 / HBM_PEAK_GBS, 4)
            if M >= 256:
                rec["mfma_frac_dense_equiv"] = round(2 * M * wl.N * wl.K / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                eff = 2 * M * (wl.N * wl.n_keep + wl.r_cat * (wl.K + wl.N))
                rec["mfma_frac_effective"] = round(eff / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
            d = dense_context(dev, wl.N, wl.K, wl.r_cat, M, steps, 4)
            rec["dense_bf16_us"] = d["us"]
            rec["speedup_vs_dense"] = round(d["us"] / (t * 1e6), 3)
            print(json.dumps(rec), flush=True)
            del X
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
    ap.add_argument("--line", default=None,
                    choices=["nf4", "backward", "prefill", "l70b_up_s50", "moe:mixtral_8x7b_w1",
                             "moe:deepseek_v2_lite_up"],
                    help="print one extra line of the default run alone (for profiling), then exit")
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
    if args.line:
        run_line(dev, args.line, args.steps, args.warmup)
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

    M = wl.M
    X = _dev_bits(inp.X, dev)
    r = measure_decode(layers, X, ws, args.steps, args.warmup, reps=10, detail=True)
    t = r["mean"]
    algo = cbytes + 2 * M * (wl.K + wl.N)
    achieved = algo / t / 1e9
    checks = check_timed_output(wl, inp, layer, inp.X, X, ws, r["Y"], r["last_layer"], dev)
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
        "us_per_step_stats": {"median": round(r["median"] * 1e6, 3), "p10": round(r["p10"] * 1e6, 3),
                              "p90": round(r["p90"] * 1e6, 3), "replays": r["replays"], "steps_per_replay": args.steps},
        "tflops_dense_equiv": round(2 * M * wl.N * wl.K / t / 1e12, 4),
        "tflops_effective": round(2 * M * (wl.N * wl.n_keep + wl.r_cat * (wl.K + wl.N)) / t / 1e12, 4),
        "roofline": {"bound": "hbm", "kernel": "fwd_small_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic()},
        "encode": {"seconds": round(encode_s, 4), "iters": 40, "oversample": 32, "call": "second"},
        "checks": {k: v for k, v in checks.items()},
    }
    if not args.no_extra:
        peaks = measure_peaks(dev)
        out["measured_peaks"] = peaks
        out["roofline"]["peak_measured"] = peaks["hbm_read_GBs"]
        out["roofline"]["frac_measured"] = round(achieved / peaks["hbm_read_GBs"], 4)
        # the floor for one launch that reads as many bytes as the forward
        floor = measure_launch_floor(dev, algo, COPIES, args.steps)
        out["launch_floor"] = floor
        out["roofline"]["frac_of_launch_floor"] = round(floor["best_us"] / (t * 1e6), 4)
        sweep = []
        for m in (1, 4, 16):
            Xm = _dev_bits(synth.make_x(wl.K, m, seed=11), dev)
            tm = measure_decode(layers, Xm, ws, 128, 16)
            al = cbytes + 2 * m * (wl.K + wl.N)
            sweep.append({"M": m, "us_per_step": round(tm * 1e6, 3), "compressed_GBs": round(cbytes / tm / 1e9, 1),
                          "hbm_frac": round(al / tm / 1e9 / HBM_PEAK_GBS, 4),
                          "hbm_frac_measured_peak": round(al / tm / 1e9 / peaks["hbm_read_GBs"], 4)})
        out["sweep"] = sweep
        del layers
        # many-token lines (matrix-core bound): 11008 x 4096 at 2048 tokens,
        # and the 70B-shaped 28672 x 8192 layer at 8192 tokens
        out["prefill"] = many_token_line(dev, "llama7b_mlp_up_11008", "llama7b_mlp_up_11008x4096_prefill", peaks,
                                         steps=20, warmup=3)
        # context: the same two shapes done densely in bf16 by the vendor GEMM library
        dh = dense_context(dev, wl.N, wl.K, wl.r_cat, M, 320, 32)
        dh["workload"] = "llama7b_attn_4096x4096_decode"
        dh["salr_speedup"] = round(dh["us"] / (t * 1e6), 3)
        wp = synth.WORKLOADS["llama7b_mlp_up_11008"]
        dp = dense_context(dev, wp.N, wp.K, wp.r_cat, wp.M, 20, 3)
        dp["workload"] = "llama7b_mlp_up_11008x4096_prefill"
        dp["salr_speedup"] = round(dp["us"] / (out["prefill"]["ms_per_step"] * 1e3), 3)
        out["dense_context"] = [dh, dp]
        out["l70b_up_s50"] = many_token_line(dev, "l70b_up_s50", "l70b_up_28672x8192_s50_m8192", peaks,
                                             steps=5, warmup=2)
        out["qsalr_nf4"] = nf4_line(dev, layer, wl, steps=128, warmup=16)
        out["backward"] = backward_line(dev, layer, wl, M=2048, steps=10, warmup=2)
        del layer
        torch.cuda.empty_cache()
        out["moe"] = [moe_line(dev, name, steps=64, warmup=8) for name in ("mixtral_8x7b_w1", "deepseek_v2_lite_up")]
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)
    if not checks["ok"]:
        print(f"bench.py: the timed run failed its checks: {checks}", file=sys.stderr)
        sys.exit(1)


def run_line(dev, line, steps, warmup):
    """One extra line of the default run alone, with the given step counts."""
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    if line.startswith("moe:"):
        print(json.dumps(moe_line(dev, line[4:], steps=steps, warmup=warmup)), flush=True)
        return
    if line in ("prefill", "l70b_up_s50"):
        name, label = (("llama7b_mlp_up_11008", "llama7b_mlp_up_11008x4096_prefill") if line == "prefill"
                       else ("l70b_up_s50", "l70b_up_28672x8192_s50_m8192"))
        peaks = {"mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS}
        print(json.dumps(many_token_line(dev, name, label, peaks, steps=steps, warmup=warmup)), flush=True)
        return
    wl = synth.WORKLOADS["llama7b_attn_4096"]
    inp = synth.make_inputs(wl, with_x=False)
    layer, _ = srl.encode(_dev_bits(inp.W, dev), wl.n_keep, wl.r_svd, [_dev_bits(a, dev) for a in inp.lora_A],
                          [_dev_bits(b, dev) for b in inp.lora_B])
    fn = nf4_line if line == "nf4" else backward_line
    kw = {"M": 2048} if line == "backward" else {}
    print(json.dumps(fn(dev, layer, wl, steps=steps, warmup=warmup, **kw)), flush=True)


def nf4_line(dev, layer, wl, steps, warmup):
    """The headline layer with its kept values in NF4 (QSALR): rotating
    quantized copies (> 512 MB), 16 tokens, against HBM peak."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    q = srl.quantize_nf4(layer.clone())
    cb = q.compressed_bytes()
    copies = max(2, -(-600_000_000 // cb))
    layers = [q] + [q.clone() for _ in range(copies - 1)]
    M = wl.M
    X = _dev_bits(synth.make_x(wl.K, M, seed=13), dev)
    ws = srl.forward_workspace(q, M)
    r = measure_decode(layers, X, ws, steps, warmup, reps=4, detail=True)
    t = r["mean"]
    algo = cb + 2 * M * (wl.K + wl.N)
    adapters = 2 * wl.r_cat * (wl.K + wl.N)
    line = {"workload": "llama7b_attn_4096x4096_decode_nf4", "M": M, "rotating_copies": copies,
            "compressed_weight_bytes": cb, "weight_bytes_per_element": round((cb - adapters) / (wl.N * wl.K), 4),
            "us_per_step": round(t * 1e6, 3), "us_median": round(r["median"] * 1e6, 3),
            "compressed_GBs": round(cb / t / 1e9, 1), "hbm_frac": round(algo / t / 1e9 / HBM_PEAK_GBS, 4),
            "wait_error": srl.wait_error(ws)}
    del layers, q, ws
    torch.cuda.empty_cache()
    return line


def backward_line(dev, layer, wl, M, steps, warmup):
    """One backward call of the headline layer (dX, dA_cat, dB_cat) at M
    tokens, graph-replayed, against the bf16 matrix-core peak; plus the
    one-off build of the transposed encoding."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    lt = srl.transpose_layer(layer)
    t_transpose = time.perf_counter() - t0
    X = _dev_bits(synth.make_x(wl.K, M, seed=14), dev)
    dY = _dev_bits(synth.make_x(wl.N, M, seed=15), dev)
    ws = srl.backward_workspace(layer, lt, M)
    dX = torch.empty((M, wl.K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((wl.r_cat, wl.K), dtype=torch.float32, device=dev)
    dB = torch.empty((wl.N, wl.r_cat), dtype=torch.float32, device=dev)
    call = lambda: srl.linear_backward(layer, lt, X, dY, dX=dX, dA=dA, dB=dB, ws=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    g = _timed_graph([call], steps)
    g.replay()
    torch.cuda.synchronize()
    t = _time_replay(g) / steps
    r = wl.r_cat
    dense = 2 * M * wl.N * wl.K + 2 * M * r * (wl.K + wl.N) * 3  # dX (dense-equiv, with its low-rank), G, T, dA, dB
    line = {"workload": "llama7b_attn_4096x4096_backward", "M": M, "r_cat": r, "ms_per_step": round(t * 1e3, 4),
            "tflops_dense_equiv": round(dense / t / 1e12, 2),
            "mfma_frac_dense_equiv": round(dense / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "transpose_build_ms": round(t_transpose * 1e3, 2), "n_keep_transposed": lt.n_keep,
            "wait_error": srl.wait_error(ws)}
    del lt, X, dY, ws, dX, dA, dB, g
    torch.cuda.empty_cache()
    return line


def moe_line(dev, name, steps, warmup):
    """A grouped expert layer in the decode regime: every expert encoded on
    the GPU (its own weight, residual SVD and LoRA), a seeded top-k routing
    of the batch, rotating copies of the whole expert set (> 512 MB), one
    salr_moe_forward per step; HBM fraction on the bytes the step must read
    (the routed experts' compressed weights, X and Y)."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    mw = synth.MOE_WORKLOADS[name]
    moe = srl.SalrMoE.empty(mw.E, mw.N, mw.K, mw.n_keep, mw.r_cat, dev)
    for e in range(mw.E):
        inp = synth.make_inputs(mw.expert_workload(e), with_x=False)
        srl.moe_encode_expert(moe, e, _dev_bits(inp.W, dev), mw.r_svd, [_dev_bits(a, dev) for a in inp.lora_A],
                              [_dev_bits(b, dev) for b in inp.lora_B])
    torch.cuda.synchronize()
    counts, _ = synth.make_routing(mw.E, mw.tokens, mw.top_k, seed=mw.seed + 3)
    T = int(counts.sum())
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
    kw, ng = -(-mw.K // 64), -(-mw.K // 1024)
    per_expert = mw.N * kw * 8 + mw.N * mw.n_keep * 2 + mw.N * ng * 4 + 2 * mw.r_cat * (mw.K + mw.N)
    copies = max(1, -(-600_000_000 // (per_expert * mw.E)))
    sets = [moe]
    for _ in range(copies - 1):
        c = srl.SalrMoE.empty(mw.E, mw.N, mw.K, mw.n_keep, mw.r_cat, dev)
        for f in ("masks", "values", "offsets", "a_cat", "b_cat"):
            getattr(c, f).copy_(getattr(moe, f))
        sets.append(c)
    X = _dev_bits(synth.make_x(mw.K, T, seed=16), dev)
    Y = torch.empty((T, mw.N), dtype=torch.bfloat16, device=dev)
    ws = srl.moe_workspace(moe, T, dev)
    fns = [(lambda m=m: srl.moe_forward(m, X, off, Y=Y, m_cap=int(counts.max()), ws=ws)) for m in sets]
    for j in range(warmup):
        fns[j % len(fns)]()
    torch.cuda.synchronize()
    g = _timed_graph(fns, steps)
    g.replay()
    torch.cuda.synchronize()
    t = _time_replay(g) / steps
    active = int((counts > 0).sum())
    algo = active * per_expert + 2 * T * (mw.K + mw.N)
    line = {"workload": f"{name}_{mw.E}x{mw.N}x{mw.K}_top{mw.top_k}_of_{mw.tokens}", "rows": T,
            "active_experts": active, "rotating_copies": copies, "us_per_step": round(t * 1e6, 3),
            "routed_weight_bytes": active * per_expert, "compressed_GBs": round(active * per_expert / t / 1e9, 1),
            "hbm_frac": round(algo / t / 1e9 / HBM_PEAK_GBS, 4)}
    del sets, moe, X, Y, ws, g
    torch.cuda.empty_cache()
    return line


def many_token_line(dev, name, label, peaks, steps, warmup):
    """One many-token workload: GPU encode, then graph-replayed forwards on
    one resident copy (the regime is matrix-core bound), against the bf16
    matrix-core peak on dense-equivalent and on the method's own flops."""
    import torch
    import sparse_rank_linear_amd as srl
    from sparse_rank_linear_amd import synth

    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, with_x=False)
    layer, _ = srl.encode(_dev_bits(inp.W, dev), wl.n_keep, wl.r_svd, [_dev_bits(a, dev) for a in inp.lora_A],
                          [_dev_bits(b, dev) for b in inp.lora_B])
    del inp
    X = _dev_bits(synth.make_x(wl.K, wl.M, seed=12), dev)
    ws = srl.forward_workspace(layer, wl.M)
    r = measure_decode([layer], X, ws, steps, warmup, reps=4, detail=True)
    werr = srl.wait_error(ws)
    t = r["mean"]
    dense = 2 * wl.M * wl.N * wl.K
    eff = 2 * wl.M * (wl.N * wl.n_keep + wl.r_cat * (wl.K + wl.N))
    line = {"workload": label, "N": wl.N, "K": wl.K, "M": wl.M, "n_keep": wl.n_keep, "r_cat": wl.r_cat,
            "ms_per_step": round(t * 1e3, 4), "ms_median": round(r["median"] * 1e3, 4),
            "ms_p10": round(r["p10"] * 1e3, 4), "ms_p90": round(r["p90"] * 1e3, 4),
            "tflops_dense_equiv": round(dense / t / 1e12, 2), "tflops_effective": round(eff / t / 1e12, 2),
            "mfma_frac_dense_equiv": round(dense / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_frac_effective": round(eff / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_frac_dense_equiv_measured_peak": round(dense / t / 1e12 / peaks["mfma_bf16_TFLOPs"], 4),
            "wait_error": werr}
    del layer, X, ws, r
    torch.cuda.empty_cache()
    return line


if __name__ == "__main__":
    main()
