"""Throughput of the KV-cache translation hot path on one MI355X.

One step = token alignment + layer map + translation of every receiver
layer, K and V, of the long-context cross-family workload: sender 36 layers,
receiver 32 layers, 8 KV heads x 128 on both sides, 32768 receiver tokens
over a shared synthetic string (sender tokens 1..8 characters, receiver
1..6), three sender taps per receiver layer flattened to 3072 features,
3072 -> 1024 maps per layer and role (dense + rank-16 folded, bf16), sender
keys stored rotated (base 5e5) and rotated back, outputs rotated at the
receiver position (base 1e6), 1% outlier channels x20.  Inputs are seeded
synthetic tensors resident in HBM before timing.

Prints one JSON line.  ``value`` = receiver tokens translated per second
(all layers, K+V).  ``roofline`` reports the dominant kernel (the grouped
GEMM with its fused epilogue) against the bf16/fp16 dense matrix-core peak,
timed with HIP events on the launch stream inside each timed step.
``cpu_baseline`` times the CPU oracle on a bounded row sample of the same
workload.  ``also`` reports the per-head workload (32 -> 80 layers, 4096
tokens, fp32 128 x 128 maps) against the HBM peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from cross_model_kv_kvx_amd import kvx, synth  # noqa: E402

PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flat_inputs(dev):
    c = synth.CONFIGS[4]
    seed = c["seed"]
    send_end, recv_end = synth.token_ends(c["recv_tokens"], seed)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    x = {}
    for r, role in enumerate(("k", "v")):
        x[f"{role}_send"] = synth.sender_cache(shp, seed * 100 + r, dev, outlier_frac=0.01, outlier_scale=20.0,
                                               outlier_pairs=(role == "k"))
        wt, u, v, b = synth.flat_maps(32, 3072, 1024, seed * 100 + 20 + r, dev, 16)
        x[f"fold_{role}"] = (wt, u, v)
        x[f"wt_{role}"] = kvx.fold_lowrank(wt, u, v, torch.bfloat16)
        x[f"b_{role}"] = b
    x["send_end"] = torch.as_tensor(send_end, device=dev)
    x["recv_end"] = torch.as_tensor(recv_end, device=dev)
    x["send_end_h"], x["recv_end_h"] = send_end, recv_end
    x["shp"] = shp
    return x


def run_step(x, taps, ws, outs, stage_ms=None):
    tmap = kvx.align_tokens(x["send_end"], x["recv_end"], out=outs["map"], workspace=outs["align_ws"])
    kvx.translate(x["k_send"], x["v_send"], tmap, taps, x["wt_k"], x["wt_v"], x["b_k"], x["b_v"],
                  send_rope_base=5e5, recv_rope_base=1e6, k_recv=outs["k"], v_recv=outs["v"], workspace=ws,
                  stage_ms=stage_ms)
    return tmap


def cpu_baseline(x, target_s=15.0):
    """The oracle as it stands on a bounded sample: token alignment of the
    whole string plus translation of sampled receiver rows (all layers, K
    and V), with maps folded by the oracle (untimed setup)."""
    from oracle import kvx_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the process CPU count
        threads = os.cpu_count() or 1
    wo = {}
    for role in ("k", "v"):
        wt, u, v = (t.cpu().numpy() for t in x[f"fold_{role}"])
        wo[role] = np.stack([O.bf16_bits_to_f64(O.fold_lowrank(wt[l], u[l], v[l])[1]) for l in range(32)])
    bo = {role: x[f"b_{role}"].cpu().numpy() for role in ("k", "v")}
    caches = {role: x[f"{role}_send"].cpu() for role in ("k", "v")}
    taps = O.layer_taps(36, 32, 3, 4)
    n_recv = x["recv_end_h"].size
    rng = np.random.default_rng(0)
    rows_done, t_total, n = 0, 0.0, 64
    t0 = time.perf_counter()
    tmap = O.token_align(x["send_end_h"], x["recv_end_h"])
    t_align = time.perf_counter() - t0
    while t_total < target_s and rows_done < n_recv:
        rows = np.sort(rng.choice(n_recv, size=n, replace=False))
        t0 = time.perf_counter()
        for role in ("k", "v"):
            O.translate_rows(caches[role], tmap, taps, wo[role], bo[role], rows, per_head=False,
                             recv_heads=8, recv_head_dim=128, send_rope_base=5e5 if role == "k" else 0.0,
                             recv_rope_base=1e6 if role == "k" else 0.0)
        t_total += time.perf_counter() - t0
        rows_done += n
    per_row = t_total / rows_done
    step_s = t_align + per_row * n_recv
    return {"value": n_recv / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"token alignment of all {n_recv} receiver tokens ({t_align:.3f} s) + translation of "
                      f"{rows_done} random receiver rows x 32 layers x K,V ({t_total:.1f} s), scaled to "
                      f"{n_recv} rows"}


def perhead_measure(dev, steps=10):
    """Per-head workload: sender 32 layers, receiver 80, 4096 tokens,
    8 x 128 heads, fp32 128 x 128 maps, identity token map."""
    shp = synth.CacheShape(32, 4096, 8, 128)
    x = {}
    for r, role in enumerate(("k", "v")):
        x[f"{role}_send"] = synth.sender_cache(shp, 200 + r, dev, channel_scale="loguniform")
        x[f"wt_{role}"], x[f"b_{role}"] = synth.perhead_maps(80, 8, 128, 220 + r, dev)
    taps = kvx.layer_map(32, 80, 1)
    ident = torch.arange(4096, dtype=torch.int32, device=dev)
    k = torch.empty((80, 4096, 8, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    ms = []
    for i in range(steps + 2):
        st = []
        kvx.translate(x["k_send"], x["v_send"], ident, taps, x["wt_k"], x["wt_v"], x["b_k"], x["b_v"],
                      per_head=True, k_recv=k, v_recv=v, stage_ms=st)
        if i >= 2:
            ms.append(st[1])
    t = float(np.mean(ms)) * 1e-3
    # algorithmic bytes: each sender row read once, each receiver row written
    # once, maps (fp32) and bias read once
    bytes_alg = 2 * (32 * 4096 * 1024 * 2 + 80 * 4096 * 1024 * 2 + 80 * 8 * 128 * 128 * 4 + 80 * 1024 * 4)
    return {"workload": "per-head 32->80 layers, 4096 tokens, 8x128 heads, fp32 maps, bf16 caches",
            "tokens_per_s": 4096 / t, "kernel_ms": t * 1e3,
            "roofline": {"bound": "hbm", "achieved": bytes_alg / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": bytes_alg / t / 1e9 / PEAK_HBM_GBS, "traffic": None}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the translation runs on a single device with no collectives; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log("bench: building inputs")
    x = flat_inputs(dev)
    taps = kvx.layer_map(36, 32, 3, 4)
    N_R = x["recv_end_h"].size
    send = kvx.cache_desc(x["k_send"], 5e5)
    recv = kvx.CacheDesc(32, N_R, 8, 128, kvx.BF16, 1e6)
    ws = torch.empty(kvx.translate_workspace_size(send, recv, 3, False), dtype=torch.uint8, device=dev)
    outs = {"map": torch.empty(N_R, dtype=torch.int32, device=dev),
            "align_ws": torch.empty(kvx.lib().kvx_align_workspace_size(N_R), dtype=torch.uint8, device=dev),
            "k": torch.empty((32, N_R, 8, 128), dtype=torch.bfloat16, device=dev)}
    outs["v"] = torch.empty_like(outs["k"])
    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        run_step(x, taps, ws, outs)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    stages = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st = []
        tmap = run_step(x, taps, ws, outs, stage_ms=st)
        stages.append(st)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    m = tmap.cpu().numpy()
    U = int(1 + np.count_nonzero(np.diff(m)))
    gemm_ms = float(np.mean([s[1] for s in stages]))
    prep_ms = float(np.mean([s[0] for s in stages]))
    flops = 2.0 * U * 3072 * 1024 * 32 * 2
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    res = {
        "metric": "translated KV tokens/sec (all layers, K+V) at 32k ctx; % of MFMA/HBM roofline",
        "value": N_R / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cross-family flattened translation with RoPE: 36->32 layers, 8x128 heads, "
                               "taps -4/0/+4, 3072->1024 bf16 maps, 32768 receiver tokens",
                   "recv_tokens": N_R, "send_tokens": int(x["send_end_h"].size), "distinct_sender_rows": U,
                   "global_batch": 1, "seq_len": N_R, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_BF16_TFLOPS, "traffic": None,
                     "kernel": "flat_gemm_kernel", "kernel_ms": gemm_ms, "prep_ms": prep_ms,
                     "flops_per_launch": flops},
    }
    if not args.no_also:
        log("bench: per-head workload")
        res["also"] = perhead_measure(dev)
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
