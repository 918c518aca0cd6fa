"""Benchmark: ms per CSA layer of the indexer-distillation hot path on one MI355X.

One step is the whole path over one V4-Flash-shaped CSA layer (B=1, S=4096, H=64, D=512,
pool N=1024, top-k K=512, window W=128; bf16 q / pool / window keys, fp32 sink and student
logits, uniform causal top-k slots), with every input resident in HBM before the timed
region: the window-LSE, the joint target, and the KL forward with its backward to the
student logits.  The default path runs distill_target_fused (window part and target in one
pass, nc_lse written as a by-product) -> distill_kl_fwd_bwd; --path 3call runs
window_lse -> distill_target -> distill_kl_fwd_bwd.  Both compute the same outputs.

Prints ONE JSON line.  `value` is the wall-clock ms per layer over the timed steps
(bracketed by device synchronisation).  Per-kernel durations come from HIP events recorded
on the stream the kernels run on (torch's current stream), and give each kernel's
achieved rate against its binding roofline (MI355X peaks: 2.5 PFLOP/s dense bf16 MFMA,
8 TB/s HBM).  `cpu_baseline` times the fp64 oracle on a strided quarter of the rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "ms per CSA layer (target+window_lse+KL fwd/bwd), % MFMA/HBM roofline"
KERNEL_SOURCES = {
    "distill_target": "sparse_attention_indexer_distill_amd/csrc/distill_target.hip",
    "distill_target_fused": "sparse_attention_indexer_distill_amd/csrc/distill_target.hip",
    "window_lse": "sparse_attention_indexer_distill_amd/csrc/window_lse.hip",
    "distill_kl_fwd_bwd": "sparse_attention_indexer_distill_amd/csrc/distill_kl.hip",
}


def src_hash(kernel: str) -> str:
    h = hashlib.sha256()
    # the kernel's source, the shared device header and the build flags
    for p in (KERNEL_SOURCES[kernel], "sparse_attention_indexer_distill_amd/csrc/sd_device.hpp",
              "sparse_attention_indexer_distill_amd/build.py"):
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def window_pairs(cfg, seg) -> int:
    """Number of (token, window key) pairs: sum_t |win(t)|."""
    S, W = cfg.S, cfg.W
    t = np.arange(S)
    if seg is None:
        return int(cfg.B * np.minimum(t + 1, W).sum())
    total = 0
    for b in range(cfg.B):
        s = seg[b].numpy()
        start = np.zeros(S, dtype=np.int64)       # first token of t's segment
        for i in range(1, S):
            start[i] = start[i - 1] if s[i] == s[i - 1] else i
        total += int(np.minimum(t - start + 1, W).sum())
    return total


def algorithmic_work(cfg, x) -> dict:
    B, S, H, D, N, K = cfg.B, cfg.S, cfg.H, cfg.D, cfg.N, cfg.K
    e = 2 if cfg.dtype == "bf16" else 4
    idx = x["idx"]
    valid = int(((idx >= 0) & (idx < N)).sum())
    wp = window_pairs(cfg, x["seg"])
    seg_b = 0 if x["seg"] is None else B * S * 4
    return {
        "window_lse": dict(flops=2 * H * D * wp, bytes=B * S * H * D * e + B * S * D * e + B * S * H * 4 + H * 4 + seg_b,
                           pairs=wp),
        "distill_target": dict(flops=2 * H * D * valid,
                               bytes=B * S * H * D * e + B * N * D * e + B * S * K * 4 + B * S * H * 4 + B * S * K * 4,
                               pairs=valid),
        "distill_kl_fwd_bwd": dict(flops=10 * valid, bytes=B * S * K * 4 * 4 + B * S * 4 + 8, pairs=valid),
        # window part and compressed part in one pass: q read once; kwin, pool, idx read; T and nc written
        "distill_target_fused": dict(flops=2 * H * D * (wp + valid),
                                     bytes=B * S * H * D * e + B * S * D * e + B * N * D * e + B * S * K * 4 +
                                     B * S * K * 4 + B * S * H * 4 + H * 4 + seg_b,
                                     pairs=wp + valid),
    }


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    summary is missing or was taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source sha256\[:16\]:\s*([0-9a-f]{16})", text)
    m_b = re.search(r"HBM bytes per launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != src_hash(kernel):
        return None
    return float(m_b.group(1))


def cpu_baseline(cfg, x, ms_per_step: float) -> dict:
    import oracle
    rows = np.arange(0, cfg.B * cfg.S, 4)          # strided quarter of the rows
    t0 = time.perf_counter()
    oracle.window_lse(x["q"], x["kwin"], x["sink"], x["seg"], cfg.W, cfg.scale, rows=rows)
    T = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=cfg.W, scale=cfg.scale,
                      rows=rows)
    oracle.kl(T.astype(np.float32), x["z"].reshape(-1, cfg.K).numpy()[rows],
              x["idx"].reshape(-1, cfg.K).numpy()[rows], cfg.N)
    dt = time.perf_counter() - t0
    ms_layer = dt * 1e3 * (cfg.B * cfg.S) / len(rows)
    # the same oracle on one core, over a smaller sample (every 64th row)
    nthreads = oracle.num_threads()
    rows1 = np.arange(0, cfg.B * cfg.S, 64)
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.window_lse(x["q"], x["kwin"], x["sink"], x["seg"], cfg.W, cfg.scale, rows=rows1)
        T1 = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=cfg.W, scale=cfg.scale,
                           rows=rows1)
        oracle.kl(T1.astype(np.float32), x["z"].reshape(-1, cfg.K).numpy()[rows1],
                  x["idx"].reshape(-1, cfg.K).numpy()[rows1], cfg.N)
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(nthreads)
    ms_layer_1core = dt1 * 1e3 * (cfg.B * cfg.S) / len(rows1)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(ms_layer, 3), "unit": "ms", "cores": nthreads, "kind": "oracle",
            "value_1core": round(ms_layer_1core, 3),
            "sample_1core": f"{len(rows1)} rows (every 64th), {dt1:.2f} s wall on one thread",
            "sample": f"{len(rows)} of {cfg.B * cfg.S} rows (every 4th), fp64 window_lse + joint target + KL; "
                      f"{dt:.2f} s wall, scaled by {cfg.B * cfg.S / len(rows):.0f}x",
            "cpu": cpu, "nproc": os.cpu_count(), "gpu_speedup": round(ms_layer / ms_per_step, 1)}


def time_launches(fn, steps: int, warmup: int, reps: int = 20) -> dict:
    """Mean/median/min per-launch duration of fn() (kernel launches only, on torch's current
    stream).  The launches are captured as one HIP graph of `reps` back-to-back calls and the
    graph is replayed between HIP events, so the host's per-call overhead (longer than these
    small kernels) never leaves the GPU idle inside the timed interval."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) / reps for a, b in evs]
    return {"ms": float(np.mean(t)), "ms_median": float(np.median(t)), "ms_min": float(np.min(t))}


def next_rows(cfg, sd, dev, steps: int, warmup: int) -> dict:
    """The steps next to the layer, at the workload's shape, each against its HBM roofline:
    the indexer's masked top-k (scores [B,S,N] -> idx, values) and its gradient scatter, and the
    CSA compressor (ratio 4, overlapping windows, kv/score [B,S,D] bf16 -> pool [B,N,D]) with its
    backward.  Algorithmic bytes: the visible part of the scores row (the blocks complete at t)
    plus the outputs; the scatter's inputs plus its dense [B,S,N] output; the compressor's kv and
    score once plus pool (and, backward, dpool plus dkv and dscore)."""
    B, S, N, K, D = cfg.B, cfg.S, cfg.N, cfg.K, cfg.D
    out = {}
    scores = synth.student_scores(cfg).to(dev)
    seg = synth.segment_ids(cfg)
    seg = None if seg is None else torch.from_numpy(seg).to(dev)
    idx = torch.empty(B, S, K, dtype=torch.int32, device=dev)
    val = torch.empty(B, S, K, device=dev)
    t = np.arange(S)
    vis = int(B * np.minimum(N, (t + 1) // 4).sum())
    r = time_launches(lambda: sd.indexer_topk(scores, seg, K=K, ratio=4, out_idx=idx, out_values=val), steps, warmup)
    r["algorithmic_bytes"] = vis * 4 + B * S * K * 8
    out["indexer_topk"] = r
    dv = torch.randn(B, S, K, device=dev)
    dsc = torch.empty(B, S, N, device=dev)
    r = time_launches(lambda: sd.indexer_topk_bwd(dv, idx, N, out=dsc), steps, warmup)
    r["algorithmic_bytes"] = B * S * K * 8 + B * S * N * 4
    out["indexer_topk_bwd"] = r
    x = synth.compressor_inputs(cfg, 4, True)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    pool = torch.empty(B, S // 4, D, device=dev)
    r = time_launches(lambda: sd.compressor_pool(g["kv"], g["score"], g["ape"], g["seg"], ratio=4, overlap=True,
                                                 out=pool), steps, warmup)
    e = g["kv"].element_size()
    r["algorithmic_bytes"] = 2 * B * S * D * e + 8 * D * 4 + B * (S // 4) * D * 4
    out["compressor_pool"] = r
    dkv = torch.empty(B, S, D, device=dev)
    dsco = torch.empty(B, S, D, device=dev)
    dape = torch.empty(8, D, device=dev)
    ws = torch.empty(max(16, sd.compressor_pool_bwd_workspace_bytes(B, S, D, 4, True)), dtype=torch.uint8, device=dev)
    r = time_launches(lambda: sd.compressor_pool_bwd(g["kv"], g["score"], g["ape"], g["dpool"], g["seg"], ratio=4,
                                                     overlap=True, dkv=dkv, dscore=dsco, dape=dape, workspace=ws),
                      steps, warmup)
    r["algorithmic_bytes"] = 2 * B * S * D * e + B * (S // 4) * D * 4 + 2 * B * S * D * 4 + 16 * D * 4
    out["compressor_pool_bwd"] = r
    for v in out.values():
        gbs = v["algorithmic_bytes"] / (v["ms"] * 1e-3) / 1e9
        v.update({"GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bound": "hbm",
                  "ms": round(v["ms"], 4), "ms_median": round(v["ms_median"], 4), "ms_min": round(v["ms_min"], 4)})
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 untimed steps (~50 ms): the GPU's clocks are still ramping over the first few
    # dozen steps, which inflates a short measurement by ~10%
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c3", choices=["c3", "c4", "c5"])
    ap.add_argument("--path", default="fused", choices=["3call", "fused"],
                    help="3call: window_lse -> distill_target -> KL; fused: distill_target_fused -> KL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing the indexer top-k and compressor steps next to the layer")
    ap.add_argument("--graph", action="store_true",
                    help="time whole steps as replays of one captured HIP graph of the step")
    ap.add_argument("--l2-cold", action="store_true",
                    help="also time each kernel with L2 flushed before every step (512 MB touched, untimed)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (the path runs on a single MI355X); got --gpus {args.gpus}. "
              "Multi-GPU sharding of this path is a design note, not a measured configuration.", file=sys.stderr)
        return 2

    import sparse_attention_indexer_distill_amd as sd
    sd.load_library()
    cfg = synth.CONFIGS[args.workload]
    x = synth.make_inputs(cfg)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    B, S, H, K = cfg.B, cfg.S, cfg.H, cfg.K
    bufs = dict(nc_lse=torch.empty(B, S, H, device=dev), target=torch.empty(B, S, K, device=dev),
                kl_rows=torch.empty(B, S, device=dev), dlogits=torch.empty(B, S, K, device=dev),
                stats=torch.empty(2, device=dev),
                workspace=torch.empty(sd.distill_kl_workspace_bytes(B, S, K), dtype=torch.uint8, device=dev))
    nonempty = int(((x["idx"] >= 0) & (x["idx"] < cfg.N)).any(-1).sum())
    grad_scale = 1e-2 / nonempty          # loss coefficient 1e-2, mean over non-empty rows

    fused = args.path == "fused"
    names = ["distill_target_fused", "distill_kl_fwd_bwd"] if fused else ["window_lse", "distill_target",
                                                                           "distill_kl_fwd_bwd"]

    def step(ev=None):
        j = 0
        if ev is not None:
            ev[j].record()
        if fused:
            sd.distill_target_fused(g["q"], g["kwin"], g["pool"], g["idx"], g["sink"], g["seg"], W=cfg.W,
                                    out=bufs["target"], nc_out=bufs["nc_lse"])
        else:
            sd.window_lse(g["q"], g["kwin"], g["sink"], g["seg"], W=cfg.W, out=bufs["nc_lse"])
            if ev is not None:
                j += 1
                ev[j].record()
            sd.distill_target(g["q"], g["pool"], g["idx"], bufs["nc_lse"], out=bufs["target"])
        if ev is not None:
            j += 1
            ev[j].record()
        sd.distill_kl_fwd_bwd(bufs["target"], g["z"], g["idx"], cfg.N, grad_scale=grad_scale,
                              kl_rows=bufs["kl_rows"], dlogits=bufs["dlogits"], stats=bufs["stats"],
                              workspace=bufs["workspace"])
        if ev is not None:
            ev[j + 1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # one step captured as a HIP graph (the library only launches kernels on the
        # capturing stream: no allocation, copy or memset inside the step)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        # the replay must reproduce the eager step bit for bit (every reduction has a fixed order)
        outs = ("nc_lse", "target", "kl_rows", "dlogits", "stats")
        step()
        torch.cuda.synchronize()
        ref = {k: bufs[k].clone() for k in outs}
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            if not torch.equal(bufs[k], ref[k]):
                raise SystemExit(f"bench: graph replay differs from the eager step in {k}")
    # timed region 1: whole steps, wall clock between device synchronisations
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # timed region 2: the same steps with HIP events between the kernels (per-kernel time)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    per_min = {n: float(np.min([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    per_med = {n: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    cold = None
    if args.l2_cold:
        # timed region 3 (reported separately): every step starts with a cold L2
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            step(evc[i])
        torch.cuda.synchronize()
        cold = {n: round(float(np.median([e[j].elapsed_time(e[j + 1]) for e in evc])), 4) for j, n in enumerate(names)}
        del flush

    work = algorithmic_work(cfg, x)
    kernels = {}
    for n in names:
        ms = per[n]
        tf = work[n]["flops"] / (ms * 1e-3) / 1e12
        gbs = work[n]["bytes"] / (ms * 1e-3) / 1e9
        kernels[n] = {"ms": round(ms, 4), "ms_median": round(per_med[n], 4), "ms_min": round(per_min[n], 4),
                      "TFLOP/s": round(tf, 1),
                      "GB/s": round(gbs, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                      "algorithmic_flops": work[n]["flops"], "algorithmic_bytes": work[n]["bytes"],
                      "src": src_hash(n)}
    dom = "distill_target_fused" if fused else "distill_target"
    ach = kernels[dom]["TFLOP/s"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": read_traffic(dom, args.workload)}
    out = {
        "metric": METRIC, "value": round(ms_per_step, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: V4-Flash-shaped CSA layer" if cfg.name == "c3" else cfg.name,
                   "B": B, "S": S, "H": H, "D": cfg.D, "N": cfg.N, "K": K, "W": cfg.W,
                   "global_batch": B, "seq_len": S, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": kernels,
        "path": args.path,
        "timing": "graph replay" if args.graph else "eager launches",
        **({"l2_cold_ms_median": cold} if cold is not None else {}),
        "layer_useful_TFLOP/s": round(sum(work[n]["flops"] for n in names) / (ms_per_step * 1e-3) / 1e12, 1),
    }
    if not args.no_next_rows:
        out["next_rows"] = next_rows(cfg, sd, dev, max(args.steps, 20), min(max(args.warmup, 5), 50))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, x, ms_per_step)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
