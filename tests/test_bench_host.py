"""Host-side logic of bench.py, checked on the CPU: the window-pair count behind the
window FLOP, the algorithmic FLOP and byte counts, and the rule that an HBM counter
summary is only used for the kernel source it was taken from."""
import os

import numpy as np
import pytest
import torch

import bench
import synth


def _pairs_bruteforce(cfg, seg):
    """sum over (b, t) of |{j : max(0, t-W+1) <= j <= t, seg[b,j] == seg[b,t]}|."""
    total = 0
    for b in range(cfg.B):
        s = np.zeros(cfg.S, dtype=np.int64) if seg is None else seg[b].numpy()
        for t in range(cfg.S):
            for j in range(max(0, t - cfg.W + 1), t + 1):
                total += int(s[j] == s[t])
    return total


@pytest.mark.parametrize("segments,W", [(1, 8), (2, 8), (4, 5), (2, 40)])
def test_window_pairs_match_bruteforce(segments, W):
    cfg = synth.Config("wp", 901, B=2, S=48, H=2, D=32, N=12, K=4, W=W, dtype="f32", segments=segments)
    x = synth.make_inputs(cfg)
    assert bench.window_pairs(cfg, x["seg"]) == _pairs_bruteforce(cfg, x["seg"])


def test_algorithmic_work_counts():
    cfg = synth.CONFIGS["c2"]
    x = synth.make_inputs(cfg)
    w = bench.algorithmic_work(cfg, x)
    valid = int(((x["idx"] >= 0) & (x["idx"] < cfg.N)).sum())
    # 2*H*D FLOP per valid (token, slot) pair and per (token, window key) pair
    assert w["distill_target"]["flops"] == 2 * cfg.H * cfg.D * valid
    assert w["window_lse"]["flops"] == 2 * cfg.H * cfg.D * bench.window_pairs(cfg, x["seg"])
    assert w["distill_target_fused"]["flops"] == w["distill_target"]["flops"] + w["window_lse"]["flops"]
    # the fused kernel reads q once: its bytes are below the two kernels' sum by one q stream
    q_bytes = cfg.B * cfg.S * cfg.H * cfg.D * 2
    assert (w["window_lse"]["bytes"] + w["distill_target"]["bytes"] - w["distill_target_fused"]["bytes"]
            == q_bytes + cfg.B * cfg.S * cfg.H * 4)
    # KL: T, z, idx read and dz written (4 bytes each per slot), kl rows, two stats floats
    assert w["distill_kl_fwd_bwd"]["bytes"] == cfg.B * cfg.S * cfg.K * 16 + cfg.B * cfg.S * 4 + 8


def test_traffic_is_ignored_for_another_kernel_source(tmp_path, monkeypatch):
    kernel, wl = "distill_target", "c9"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # src_hash reads the kernel sources relative to ROOT: give it copies of the real ones
    for rel in (bench.KERNEL_SOURCES[kernel], "sparse_attention_indexer_distill_amd/csrc/sd_device.hpp",
                "sparse_attention_indexer_distill_amd/build.py"):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(os.path.dirname(bench.__file__), rel), "rb").read())
    good = bench.src_hash(kernel)
    (prof / f"{kernel}_{wl}_counters.md").write_text(f"source sha256[:16]: {good}\nHBM bytes per launch: 1.5e+08\n")
    assert bench.read_traffic(kernel, wl) == pytest.approx(1.5e8)
    (prof / f"{kernel}_{wl}_counters.md").write_text("source sha256[:16]: 0123456789abcdef\n"
                                                     "HBM bytes per launch: 1.5e+08\n")
    assert bench.read_traffic(kernel, wl) is None
    assert bench.read_traffic(kernel, "none") is None


def test_multi_gpu_request_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
