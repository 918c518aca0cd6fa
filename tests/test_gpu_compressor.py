"""GPU parity of the compressor pool and its analytic backward against the fp64 oracle
(needs an MI355X).

Tolerances: pool, dkv and dscore abs 1e-5 (each is a softmax-weighted combination of at
most 2 x 128 inputs of magnitude ~1, accumulated in fp32 with hardware exp2: errors of a few
ulps, ~1e-6); dape, a sum over every entry of the batch, max error <= 1e-4 * max|dape| + 1e-5.
Tokens past the last entry get exact zeros, compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-5


def _sd():
    import sparse_attention_indexer_distill_amd as sd
    sd.load_library()
    return sd


def run_case(cfg, ratio, overlap, dtype=None, seg=None, what=""):
    sd = _sd()
    dev = torch.device("cuda:0")
    x = synth.compressor_inputs(cfg, ratio, overlap, dtype)
    if seg is None:
        seg = x["seg"]
    B, S, D = x["kv"].shape
    print(f"[gpu] compressor {what}: B={B} S={S} D={D} ratio={ratio} overlap={overlap} {x['kv'].dtype} "
          f"seg={seg is not None}", flush=True)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    seg_d = None if seg is None else torch.as_tensor(seg).to(dev)
    pool = sd.compressor_pool(g["kv"], g["score"], g["ape"], seg_d, ratio=ratio, overlap=overlap)
    dkv, dsc, dape = sd.compressor_pool_bwd(g["kv"], g["score"], g["ape"], g["dpool"], seg_d, ratio=ratio,
                                            overlap=overlap)
    torch.cuda.synchronize()
    segn = None if seg is None else np.asarray(seg)
    p_ref = oracle.compressor_pool(x["kv"], x["score"], x["ape"], segn, ratio, overlap)
    dkv_ref, dsc_ref, dape_ref = oracle.compressor_pool_bwd(x["kv"], x["score"], x["ape"], segn, x["dpool"], ratio,
                                                            overlap)
    p = pool.cpu().numpy()
    assert np.isfinite(p).all()
    e = np.abs(p - p_ref).max()
    assert e <= ATOL, f"{what}: pool err {e:.3e}"
    for name, got, ref in (("dkv", dkv, dkv_ref), ("dscore", dsc, dsc_ref)):
        got = got.cpu().numpy()
        assert np.isfinite(got).all()
        e = np.abs(got - ref).max()
        assert e <= ATOL, f"{what}: {name} err {e:.3e}"
        N = S // ratio
        assert (got[:, N * ratio:] == 0).all(), f"{what}: {name} past the last entry not zero"
    da = dape.cpu().numpy()
    e = np.abs(da - dape_ref).max()
    assert e <= 1e-4 * np.abs(dape_ref).max() + 1e-5, f"{what}: dape err {e:.3e}"
    return pool, dkv, dsc, dape


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_csa_compressor_full_size(name):
    run_case(synth.CONFIGS[name], 4, True, what=name + " CSA")


def test_csa_compressor_two_segments():
    run_case(synth.CONFIGS["c4"], 4, True, what="c4 CSA, two documents")


def test_hca_compressor():
    run_case(synth.CONFIGS["c3"], 128, False, what="c3 HCA")


@pytest.mark.parametrize("case", [
    # (B, S, D, ratio, overlap, dtype, segment length)
    (2, 1003, 64, 4, True, "f32", 333),     # ragged tail, boundaries inside blocks
    (1, 514, 32, 2, True, "bf16", 0),
    (1, 640, 16, 16, True, "f32", 200),
    (2, 130, 8, 8, False, "bf16", 0),
    (1, 77, 12, 1, False, "f32", 0),
    (1, 1000, 128, 32, False, "bf16", 300),
    (1, 64, 4, 64, False, "f32", 0),
    (1, 700, 32, 8, True, "bf16", 250),     # 16-position windows: the largest held in registers
    (1, 520, 16, 16, False, "f32", 0),
], ids=lambda c: "-".join(map(str, c)))
def test_compressor_edge_shapes(case):
    B, S, D, r, ovl, dt, L = case
    cfg = synth.Config(f"cp_{S}_{D}_{r}", 890 + S % 53 + r, B=B, S=S, H=1, D=D, N=max(S // r, 1), K=1, W=1, dtype=dt)
    seg = None
    if L:
        seg = (np.arange(S) // L).astype(np.int32)[None].repeat(B, 0)
    run_case(cfg, r, ovl, seg=seg, what="edge")


def _random_compressor_cases(n=16, seed=51515):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        ovl = bool(rng.random() < 0.5)
        r = int(rng.choice([1, 2, 4, 8, 16] if ovl else [1, 2, 4, 8, 16, 32, 64, 128]))
        D = 4 * int(rng.integers(1, 129))
        S = int(rng.integers(r, 2500))
        B = int(rng.integers(1, 3))
        dt = "bf16" if rng.random() < 0.6 else "f32"
        L = int(rng.choice([0, int(rng.integers(1, S + 1))]))
        out.append((B, S, D, r, ovl, dt, L))
    return out


@pytest.mark.parametrize("case", _random_compressor_cases(), ids=lambda c: "-".join(map(str, c)))
def test_compressor_random_shapes(case):
    """Seeded random shapes: ratios 1..128 (up to 16 with overlap), D a multiple of 4 up to
    512, ragged S, bf16 and fp32, optional segments of arbitrary length."""
    B, S, D, r, ovl, dt, L = case
    cfg = synth.Config(f"cpr_{S}_{D}_{r}", 600 + (S + 3 * D + r) % 157, B=B, S=S, H=1, D=D, N=max(S // r, 1), K=1,
                       W=1, dtype=dt)
    seg = None
    if L:
        seg = (np.arange(S) // L).astype(np.int32)[None].repeat(B, 0)
    run_case(cfg, r, ovl, seg=seg, what="random")


def test_compressor_deterministic_and_segment_isolated():
    sd = _sd()
    dev = torch.device("cuda:0")
    c = synth.CONFIGS["c4"]
    x = synth.compressor_inputs(c, 4, True)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    print("[gpu] compressor: determinism and segment isolation", flush=True)
    a = [t.clone() for t in (sd.compressor_pool(g["kv"], g["score"], g["ape"], g["seg"], ratio=4, overlap=True),
                             *sd.compressor_pool_bwd(g["kv"], g["score"], g["ape"], g["dpool"], g["seg"], ratio=4,
                                                     overlap=True))]
    b = [sd.compressor_pool(g["kv"], g["score"], g["ape"], g["seg"], ratio=4, overlap=True),
         *sd.compressor_pool_bwd(g["kv"], g["score"], g["ape"], g["dpool"], g["seg"], ratio=4, overlap=True)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # the first document's tokens poisoned: the second document's entries are bitwise unchanged
    h = c.S // 2
    kv_p, sc_p = g["kv"].clone(), g["score"].clone()
    kv_p[:, :h] = float("nan")
    sc_p[:, :h] = float("inf")
    p2 = sd.compressor_pool(kv_p, sc_p, g["ape"], g["seg"], ratio=4, overlap=True)
    torch.cuda.synchronize()
    assert torch.equal(p2[:, h // 4:], a[0][:, h // 4:])
