"""GPU parity of the indexer's top-k selection and its gradient scatter (needs an MI355X).

Both are integer and index work, compared bit for bit with the oracle: the kept block
indices, their order and the -1 padding; the gathered values (copies of float32 scores);
and the scattered gradient, whose entries are copies of single slot gradients when a row's
slots are distinct (the sums of duplicate slots are compared within 1e-6 relative, since
the oracle adds them in double).  Shapes: the V4-Flash layer (c3: N=1024, K=512), the
long-context layer (c5: B=2, N=2048, K=1024), two packed segments (c4), heavy ties, NaN and
-inf scores, and HCA-like wide blocks.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _sd():
    import sparse_attention_indexer_distill_amd as sd
    sd.load_library()
    return sd


def _say(msg):
    print(msg, flush=True)


def check_topk(scores, seg, K, ratio, what, rows=None):
    sd = _sd()
    dev = torch.device("cuda:0")
    B, S, N = scores.shape
    seg_d = None if seg is None else torch.as_tensor(seg).to(dev)
    _say(f"[gpu] indexer_topk {what}: B={B} S={S} N={N} K={K} ratio={ratio} seg={seg is not None}")
    idx, val = sd.indexer_topk(torch.as_tensor(scores).to(dev), seg_d, K=K, ratio=ratio)
    torch.cuda.synchronize()
    i_ref, v_ref = oracle.indexer_topk(scores, seg, K, ratio, rows=rows)
    i_gpu = idx.reshape(-1, K).cpu().numpy()
    v_gpu = val.reshape(-1, K).cpu().numpy()
    if rows is not None:
        i_gpu, v_gpu = i_gpu[rows], v_gpu[rows]
    bad = np.flatnonzero((i_gpu != i_ref).any(-1))
    assert len(bad) == 0, f"{what}: {len(bad)} rows differ, first row {bad[0]}: {i_gpu[bad[0]][:12]} vs {i_ref[bad[0]][:12]}"
    np.testing.assert_array_equal(v_gpu.view(np.uint32), v_ref.view(np.uint32))   # bitwise, NaN payloads too
    return idx, val


@pytest.mark.parametrize("name", ["c3", "c5", "c4"])
def test_topk_full_size_bit_exact(name):
    c = synth.CONFIGS[name]
    seg = synth.segment_ids(c)             # two packed documents at c4, None otherwise
    scores = synth.student_scores(c).numpy()
    check_topk(scores, seg, c.K, 4, name)


@pytest.mark.parametrize("name", ["c3", "c2"])
def test_topk_ties_nan_and_inf(name):
    c = synth.CONFIGS[name]
    s = synth.student_scores(c, ties=True).numpy().copy()
    rng = np.random.default_rng(c.cid + 17)
    m = rng.random(s.shape)
    s[m < 0.02] = np.nan
    s[(m >= 0.02) & (m < 0.04)] = -np.inf
    s[(m >= 0.04) & (m < 0.05)] = np.inf
    s[(m >= 0.05) & (m < 0.06)] = -0.0
    check_topk(s, None, c.K, 4, name + " ties/nan/inf")


@pytest.mark.parametrize("case", [
    # (B, S, N, K, ratio, segments)
    (2, 300, 75, 40, 4, 1),       # K inside the visible count for late rows, ragged S
    (1, 520, 130, 130, 4, 2),     # K = N, two segments
    (1, 4096, 32, 8, 128, 1),     # wide (HCA-like) blocks
    (3, 70, 17, 1, 4, 1),         # top-1
    (1, 9000, 4096, 300, 2, 1),   # the largest N, E = 64 registers
    (1, 33, 2, 4096, 16, 1),      # K far above N: everything padded past the visible blocks
], ids=lambda c: "-".join(map(str, c)))
def test_topk_edge_shapes(case):
    B, S, N, K, ratio, segs = case
    cfg = synth.Config(f"topk_{S}_{N}", 880 + S % 97, B=B, S=S, H=1, D=32, N=N, K=min(K, 4096), W=1, dtype="f32",
                       segments=segs if S % (segs * 4) == 0 else 1)
    s = synth.student_scores(cfg).numpy()
    seg = None
    if segs > 1:
        L = S // segs
        seg = np.minimum(np.arange(S) // L, segs - 1).astype(np.int32)[None].repeat(B, 0)
        seg[:, L + 1] = 7                      # a lone token with its own id inside the second document
    rows = None if B * S <= 20000 else np.arange(0, B * S, 3)
    check_topk(s, seg, K, ratio, "edge", rows=rows)


def _random_topk_cases(n=16, seed=77031):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        ratio = int(rng.choice([1, 2, 4, 8, 16, 128]))
        N = int(rng.integers(1, 4097))
        S = int(min(max(ratio, N * ratio + int(rng.integers(-3 * ratio, 3 * ratio + 1))), 3000))
        K = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(1, N + 1)), int(rng.integers(1, 4097))]))
        B = int(rng.integers(1, 3))
        if B * S * max(N, K) > 12_000_000:  # the oracle's dense scatter stays small
            continue
        segs = int(rng.integers(1, 4))
        ties = bool(rng.random() < 0.4)
        out.append((B, S, N, K, ratio, segs, ties))
    return out


@pytest.mark.parametrize("case", _random_topk_cases(), ids=lambda c: "-".join(map(str, c)))
def test_topk_random_shapes_bit_exact(case):
    """Seeded random shapes (N up to 4096, K up to 4096, block ratios 1..128, up to three
    segments, optionally tied scores): every row bit-exact against the oracle, selection and
    scatter."""
    B, S, N, K, ratio, segs, ties = case
    cfg = synth.Config(f"topk_r_{S}_{N}", 700 + (S * 7 + N) % 211, B=B, S=S, H=1, D=32, N=N, K=K, W=1, dtype="f32")
    s = synth.student_scores(cfg, ties=ties).numpy()
    seg = None
    if segs > 1:
        seg = np.minimum(np.arange(S) * segs // S, segs - 1).astype(np.int32)[None].repeat(B, 0)
    idx, val = check_topk(s, seg, K, ratio, "random")
    sd = _sd()
    dv = torch.from_numpy(np.random.default_rng(S + N + K).standard_normal((B, S, K)).astype(np.float32))
    ds = sd.indexer_topk_bwd(dv.to(torch.device("cuda:0")), idx, N)
    torch.cuda.synchronize()
    ref = oracle.indexer_topk_bwd(dv, idx.cpu(), N).astype(np.float32)
    np.testing.assert_array_equal(ds.reshape(-1, N).cpu().numpy(), ref)


def test_topk_bwd_scatter_bit_exact_and_duplicates():
    sd = _sd()
    dev = torch.device("cuda:0")
    for name in ("c3", "c5"):
        c = synth.CONFIGS[name]
        scores = synth.student_scores(c)
        idx, val = sd.indexer_topk(scores.to(dev), None, K=c.K, ratio=4)
        dv = torch.from_numpy(np.random.default_rng(c.cid).standard_normal((c.B, c.S, c.K)).astype(np.float32))
        _say(f"[gpu] indexer_topk_bwd {name}")
        ds = sd.indexer_topk_bwd(dv.to(dev), idx, c.N)
        torch.cuda.synchronize()
        ref = oracle.indexer_topk_bwd(dv, idx.cpu(), c.N).astype(np.float32)
        np.testing.assert_array_equal(ds.reshape(-1, c.N).cpu().numpy(), ref)
    # arbitrary slots: -1, out of range, and duplicates (summed in slot order)
    c = synth.CONFIGS["c2"]
    rng = np.random.default_rng(3)
    # distinct blocks per row (a random permutation's head), some slots -1 or out of range
    idx = np.argsort(rng.random((c.B, c.S, c.N)), axis=-1)[..., : c.K].astype(np.int32)
    junk = rng.random(idx.shape)
    idx[junk < 0.05] = -1
    idx[(junk >= 0.05) & (junk < 0.08)] = c.N + 2
    dup_rows = rng.random(c.S) < 0.3
    idx[0, dup_rows, 1] = idx[0, dup_rows, 0]
    idx[0, dup_rows, 63] = idx[0, dup_rows, 0]
    dv = rng.standard_normal((c.B, c.S, c.K)).astype(np.float32)
    _say("[gpu] indexer_topk_bwd with duplicate slots")
    ds = sd.indexer_topk_bwd(torch.from_numpy(dv).to(dev), torch.from_numpy(idx).to(dev), c.N)
    torch.cuda.synchronize()
    ref = oracle.indexer_topk_bwd(dv, idx, c.N)
    got = ds.reshape(-1, c.N).cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)
    # rows whose valid slots happen to be distinct are plain copies, bit for bit
    valid = (idx[0] >= 0) & (idx[0] < c.N)
    nodup = np.array([len(np.unique(r[v])) == v.sum() for r, v in zip(idx[0], valid)])
    assert nodup.sum() > 10 and (~nodup).sum() > 10
    np.testing.assert_array_equal(got[nodup], ref[nodup].astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("K,N", [(1, 7), (37, 130), (100, 301), (200, 257), (333, 1000), (700, 1500),
                                 (1000, 1024), (1100, 2048), (2100, 4096), (4096, 4096)])
def test_topk_bwd_scatter_ragged_slot_counts(K, N):
    """Slot counts on both sides of every register width of the scatter and past it (K above 1024
    reads the slots from memory), 97 rows (a ragged last workgroup), invalid slots, and rows whose
    duplicate slots lie 64 or more slots apart (different register steps)."""
    sd = _sd()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1000 + K)
    S = 97
    if K <= N:
        idx = np.argsort(rng.random((1, S, N)), axis=-1)[..., :K].astype(np.int32)
    else:
        idx = rng.integers(0, N, size=(1, S, K)).astype(np.int32)
    junk = rng.random(idx.shape)
    idx[junk < 0.05] = -1
    idx[(junk >= 0.05) & (junk < 0.07)] = N + 5
    if K > 1:
        dup_rows = rng.random(S) < 0.3
        idx[0, dup_rows, K - 1] = idx[0, dup_rows, 0]
        idx[0, dup_rows, K // 2] = idx[0, dup_rows, 0]
    dv = rng.standard_normal((1, S, K)).astype(np.float32)
    _say(f"[gpu] indexer_topk_bwd ragged K={K} N={N}")
    ds = sd.indexer_topk_bwd(torch.from_numpy(dv).to(dev), torch.from_numpy(idx).to(dev), N)
    torch.cuda.synchronize()
    ref = oracle.indexer_topk_bwd(dv, idx, N)
    got = ds.reshape(-1, N).cpu().numpy().astype(np.float64)
    # m float32 additions in slot order err by at most m 2^-24 times the sum of the magnitudes
    mag = oracle.indexer_topk_bwd(np.abs(dv), idx, N)
    cnt = oracle.indexer_topk_bwd(np.ones_like(dv), idx, N)
    assert np.all(np.abs(got - ref) <= cnt * 2.0 ** -24 * mag)
    valid = (idx[0] >= 0) & (idx[0] < N)
    nodup = np.array([len(np.unique(r[v])) == v.sum() for r, v in zip(idx[0], valid)])
    np.testing.assert_array_equal(got[nodup], ref[nodup].astype(np.float32).astype(np.float64))


def test_selection_feeds_the_layer_and_its_gradient_reaches_the_scores():
    """The chain the loss runs: scores -> indexer_topk -> (idx, student logits) -> fused target
    and KL -> gradient on the logits -> indexer_topk_bwd -> gradient on the scores.  Checked
    against the oracle's composition of the same steps."""
    sd = _sd()
    dev = torch.device("cuda:0")
    x = synth.make_inputs("c2")
    c = x["cfg"]
    scores = synth.student_scores(c)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    _say("[gpu] c2: selection -> layer -> scatter")
    idx, z = sd.indexer_topk(scores.to(dev), None, K=c.K, ratio=4)
    out = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], idx, z, g["sink"], None, W=c.W, grad_scale=0.25,
                               fused=True)
    dscores = sd.indexer_topk_bwd(out["dlogits"], idx, c.N)
    torch.cuda.synchronize()
    i_ref, z_ref = oracle.indexer_topk(scores, None, c.K, 4)
    i_ref = i_ref.reshape(c.B, c.S, c.K)
    T_ref = oracle.target(x["q"], x["pool"], i_ref, x["kwin"], x["sink"], None, W=c.W, scale=c.scale)
    _, dz_ref, _ = oracle.kl(T_ref.astype(np.float32), z_ref.reshape(c.B, c.S, c.K), i_ref, c.N, grad_scale=0.25)
    ds_ref = oracle.indexer_topk_bwd(dz_ref.astype(np.float32).reshape(c.B, c.S, c.K), i_ref, c.N)
    got = dscores.reshape(-1, c.N).cpu().numpy()
    dT = np.abs(out["target"].reshape(-1, c.K).cpu().numpy() - T_ref).max(-1)
    err = np.abs(got - ds_ref).max(-1)
    scale = np.abs(ds_ref).max(-1)
    assert (err <= 1e-4 * scale + 1e-6 * 0.25 + 2 * 0.25 * dT).all(), err.max()
    assert ((got != 0) <= (ds_ref != 0)).all()          # no gradient outside the kept blocks
