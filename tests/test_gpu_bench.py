"""bench.py end to end on the GPU, a few steps: the one JSON line it prints carries the
fields the benchmark contract asks for, and its roofline and oracle baseline are
consistent with the kernel timings in the same line."""
import json

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_bench_prints_one_complete_json_line(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--steps", "3", "--warmup", "2"])
    assert bench.main() == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["unit"] == "ms" and d["value"] > 0 and d["ms_per_step"] == d["value"]
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["higher_is_better"] is False and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"] == "synthetic" and d["path"] == "fused"
    assert d["config"]["workload"].startswith("c3") and d["config"]["S"] == 4096 and d["config"]["K"] == 512

    k = d["kernels"]
    assert set(k) == {"distill_target_fused", "distill_kl_fwd_bwd"}
    assert all(v["ms"] > 0 for v in k.values())

    r = d["roofline"]
    assert r["bound"] == "mfma" and r["kernel"] == "distill_target_fused" and r["unit"] == "TFLOP/s"
    assert r["peak"] == 2500.0 and 0 < r["frac"] < 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # achieved = useful FLOP of one launch / its mean duration
    kt = k["distill_target_fused"]
    # (kt["ms"] is rounded to 4 decimals: up to ~3e-4 relative at 0.2 ms)
    assert abs(r["achieved"] - kt["algorithmic_flops"] / (kt["ms"] * 1e-3) / 1e12) <= 1e-3 * r["achieved"] + 0.1
    # HBM counters, when the committed summary matches this kernel source, cover at least
    # the compulsory bytes
    assert r["traffic"] is None or r["traffic"] >= 0.95 * kt["algorithmic_bytes"]

    nr = d["next_rows"]
    assert set(nr) == {"indexer_topk", "indexer_topk_bwd", "compressor_pool", "compressor_pool_bwd"}
    for v in nr.values():
        assert v["ms"] > 0 and v["bound"] == "hbm" and 0 < v["hbm_frac"] < 1.5

    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "ms" and c["value"] > 0 and c["cores"] >= 1
    assert isinstance(c["sample"], str) and "rows" in c["sample"]
