"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Tolerances (stated once, used everywhere):
  target T           abs 1e-5                       (the accuracy bar for target probabilities)
  nc_lse             abs 1e-4 + rel 1e-5            (fp32 dot products over D <= 512 terms
                                                     of magnitude ~1, scaled by 1/sqrt(D): ~1e-6
                                                     typical error; the LSE adds |lse| * 2^-24)
  KL per row         rel 1e-4 + abs 2e-6            (rel 1e-4 on loss and gradient; the absolute
                                                     term covers rows whose KL is ~0, where fp32
                                                     rounding of log T and z, ~1e-7 * |log T| per
                                                     slot, is all that is left)
  dlogits            per row: max|d| <= 1e-4 * max|ref| + 1e-6 * |g| * max_k T_k
                                                    (norm-wise rel 1e-4; the absolute term is
                                                     ~16 fp32 ulps of the row's largest
                                                     probability, for rows where the student
                                                     matches the target and the gradient is a
                                                     difference of two nearly equal numbers)
  loss (mean over non-empty rows) rel 1e-4; non-empty row count exact
Masks and zero patterns are compared bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

T_ATOL = 1e-5
NC_ATOL, NC_RTOL = 1e-4, 1e-5
KL_RTOL, KL_ATOL = 1e-4, 2e-6
DZ_RTOL = 1e-4


def _sd():
    import sparse_attention_indexer_distill_amd as sd
    sd.load_library()
    return sd


def _say(msg):
    print(msg, flush=True)


def _dev():
    return torch.device("cuda:0")


def _to(x, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _np(t):
    return t.detach().cpu().numpy()


# ------------------------------------------------------------------ comparisons
def check_T(T_gpu, T_ref, idx_rows, N, what):
    """T_gpu, T_ref: [rows, K]; idx_rows [rows, K]."""
    valid = (idx_rows >= 0) & (idx_rows < N)
    # bit-exact zero pattern on invalid slots, and no NaN anywhere
    assert np.isfinite(T_gpu).all(), f"{what}: non-finite target"
    assert (T_gpu[~valid] == 0).all() and not np.signbit(T_gpu[~valid]).any(), f"{what}: invalid slot not +0"
    err = np.abs(T_gpu - T_ref).max(initial=0.0)
    assert err <= T_ATOL, f"{what}: max |T - T_ref| = {err:.3e}"
    return err


def check_nc(nc_gpu, nc_ref, what):
    assert np.isfinite(nc_gpu).all(), f"{what}: non-finite nc_lse"
    err = np.abs(nc_gpu - nc_ref)
    bad = err > NC_ATOL + NC_RTOL * np.abs(nc_ref)
    assert not bad.any(), f"{what}: nc_lse max err {err.max():.3e}"
    return err.max(initial=0.0)


def check_kl(kl_gpu, dz_gpu, kl_ref, dz_ref, idx_rows, N, what, T_rows, grad_scale=1.0, dT_rows=None):
    """dT_rows: per-row max |T_gpu - T_ref| when the GPU's KL ran on the GPU's target and the
    oracle's on the oracle's (the layer tests).  The gradient g((sum T) Q - T) then differs by
    up to 2 |g| max|dT| on top of the KL kernel's own error: on rows whose student matches
    the target the gradient is nothing but that difference."""
    valid = (idx_rows >= 0) & (idx_rows < N)
    assert np.isfinite(kl_gpu).all() and np.isfinite(dz_gpu).all(), f"{what}: non-finite KL/grad"
    assert (dz_gpu[~valid] == 0).all() and not np.signbit(dz_gpu[~valid]).any(), f"{what}: invalid slot grad not +0"
    empty = ~valid.any(-1)
    assert (kl_gpu[empty] == 0).all() and (dz_gpu[empty] == 0).all(), f"{what}: empty rows not zero"
    e_kl = np.abs(kl_gpu - kl_ref)
    assert (e_kl <= KL_RTOL * np.abs(kl_ref) + KL_ATOL).all(), f"{what}: KL err {e_kl.max():.3e}"
    e_dz = np.abs(dz_gpu - dz_ref).max(-1)
    scale = np.abs(dz_ref).max(-1)
    atol = 1e-6 * abs(grad_scale) * np.abs(T_rows).max(-1)
    if dT_rows is not None:
        atol = atol + 2.0 * abs(grad_scale) * dT_rows
    assert (e_dz <= DZ_RTOL * scale + atol).all(), f"{what}: grad err {(e_dz / np.maximum(scale, 1e-30)).max():.3e}"
    return e_kl.max(initial=0.0), (e_dz / np.maximum(scale, 1e-30)).max(initial=0.0)


# ------------------------------------------------------------------ the layer on a config
_ORACLE_CACHE = {}


def oracle_layer(name, x, rows, z, shuffle_pad):
    """Oracle nc_lse, target, KL and gradient on the given rows (cached per workload when every
    row is compared, so the two paths share one oracle pass)."""
    key = (name, shuffle_pad) if len(rows) == x["cfg"].B * x["cfg"].S else None
    if key is not None and key in _ORACLE_CACHE:
        return _ORACLE_CACHE[key]
    c = x["cfg"]
    idx_all = x["idx"].reshape(-1, c.K).numpy()
    nc_ref = oracle.window_lse(x["q"], x["kwin"], x["sink"], x["seg"], c.W, c.scale, rows=rows)
    T_ref = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=c.W, scale=c.scale,
                          rows=rows)
    z_rows = z.reshape(-1, c.K).numpy()[rows]
    kl_ref, dz_ref, _ = oracle.kl(T_ref.astype(np.float32), z_rows, idx_all[rows], c.N)
    res = (nc_ref, T_ref, kl_ref, dz_ref)
    if key is not None:
        _ORACLE_CACHE.clear()                # one full-size workload held at a time
        _ORACLE_CACHE[key] = res
    return res


def run_config(name, nsample=None, shuffle_pad=False, fused=False):
    sd = _sd()
    x = synth.make_inputs(name, shuffle_pad=shuffle_pad)
    c = x["cfg"]
    dev = _dev()
    rows = np.arange(c.B * c.S) if nsample is None else synth.sample_rows(c, nsample)
    idx_all = x["idx"].reshape(-1, c.K).numpy()
    # c4-style rows whose student logits equal log(target)
    z = x["z"].clone()
    if len(x["kl_zero_rows"]):
        Tz = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=c.W,
                           scale=c.scale, rows=x["kl_zero_rows"]).astype(np.float32)
        with np.errstate(divide="ignore"):
            zz = np.where(Tz > 0, np.log(np.where(Tz > 0, Tz, 1.0)), -60.0).astype(np.float32)
        z.reshape(-1, c.K)[torch.as_tensor(x["kl_zero_rows"])] = torch.from_numpy(zz)
    g = _to(x, dev)
    g["z"] = z.to(dev)
    _say(f"[gpu] {name}: layer B={c.B} S={c.S} H={c.H} D={c.D} N={c.N} K={c.K} W={c.W} {c.dtype} fused={fused}")
    out = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=c.W,
                               grad_scale=1.0, fused=fused)
    torch.cuda.synchronize()
    nc = _np(out["nc_lse"]).reshape(-1, c.H)[rows]
    T = _np(out["target"]).reshape(-1, c.K)[rows]
    kl = _np(out["kl_rows"]).reshape(-1)[rows]
    dz = _np(out["dlogits"]).reshape(-1, c.K)[rows]
    stats = _np(out["stats"])
    # oracle on the same rows
    nc_ref, T_ref, kl_ref, dz_ref = oracle_layer(name, x, rows, z, shuffle_pad)
    e_nc = check_nc(nc, nc_ref, name)
    e_T = check_T(T, T_ref, idx_all[rows], c.N, name)
    e_kl, e_dz = check_kl(kl, dz, kl_ref, dz_ref, idx_all[rows], c.N, name, T_ref,
                          dT_rows=np.abs(T - T_ref).max(-1))
    # loss statistics: the count is exact, the sum is checked when every row was compared
    nonempty = ((idx_all >= 0) & (idx_all < c.N)).any(-1)
    assert stats[1] == nonempty.sum()
    if nsample is None:
        assert abs(stats[0] - kl_ref[nonempty[rows]].sum()) <= KL_RTOL * abs(kl_ref.sum()) + 1e-5
    else:
        kl_all = _np(out["kl_rows"]).reshape(-1).astype(np.float64)
        assert abs(stats[0] - kl_all[nonempty].sum()) <= 1e-5 * abs(kl_all.sum()) + 1e-5
    _say(f"[gpu] {name}: max err nc {e_nc:.2e} T {e_T:.2e} KL {e_kl:.2e} grad(rel) {e_dz:.2e} "
         f"rows {len(rows)} stats {stats.tolist()}")
    return x, out, rows


# fused=True runs distill_target_fused (window part inside the target kernel) instead of
# window_lse + distill_target; the same oracle values check both.
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("name", ["c1", "c2", "c1_local"])
def test_layer_parity_all_rows(name, fused):
    run_config(name, fused=fused)


# Full sizes, every row against the oracle (the oracle pass is shared by the two paths).
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("name", ["c3", "c4", "c3_local", "c5"])
def test_layer_parity_full_size_every_row(name, fused):
    x, out, rows = run_config(name, fused=fused)
    c = x["cfg"]
    if len(x["kl_zero_rows"]):
        kl = _np(out["kl_rows"]).reshape(-1)[x["kl_zero_rows"]]
        assert np.abs(kl).max() <= 1e-5, f"KL on rows with student = log target: {np.abs(kl).max():.3e}"
    if name == "c3_local":
        # every non-empty row renormalises to 1 although its compressed mass is < 1e-10
        T = _np(out["target"]).reshape(-1, c.K)
        idx = x["idx"].reshape(-1, c.K).numpy()
        ne = ((idx >= 0) & (idx < c.N)).any(-1)
        np.testing.assert_allclose(T[ne].sum(-1), 1.0, atol=1e-4)


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_full_size_every_row_properties(name):
    """Every row at full size, by properties that hold at any size (the sampled test above
    compares chosen rows with the oracle):
      - exact zeros of T and dlogits at invalid slots, T >= 0;
      - sum_k T = 1 on rows with a valid slot (the L1 step; float32-tiny never binds here),
        and empty rows all zero with KL 0;
      - KL >= 0 and sum_k dlogits = g (sum T)(sum softmax - 1) = 0 on every row;
      - the fused kernel's window part and window_lse (separate kernels) give the same
        nc_lse, and both paths the same target and KL, on every row, within twice the
        per-path tolerance against the oracle."""
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs(name)
    c = x["cfg"]
    g = _to(x, dev)
    outs = {}
    for fused in (False, True):
        _say(f"[gpu] {name}: every-row properties, fused={fused}")
        o = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=c.W,
                                 grad_scale=1.0, fused=fused)
        torch.cuda.synchronize()
        outs[fused] = {k: _np(v) for k, v in o.items()}
    idx = x["idx"].reshape(-1, c.K).numpy()
    valid = (idx >= 0) & (idx < c.N)
    nonempty = valid.any(-1)
    for fused, o in outs.items():
        T = o["target"].reshape(-1, c.K)
        dz = o["dlogits"].reshape(-1, c.K)
        kl = o["kl_rows"].reshape(-1)
        assert np.isfinite(o["nc_lse"]).all() and np.isfinite(T).all() and np.isfinite(dz).all()
        assert (T[~valid] == 0).all() and (dz[~valid] == 0).all() and (T >= 0).all()
        rs = T.sum(-1, dtype=np.float64)
        assert np.abs(rs[nonempty] - 1.0).max() <= 1e-5, f"fused={fused}: row sums off by {np.abs(rs[nonempty] - 1).max():.2e}"
        assert (rs[~nonempty] == 0).all() and (kl[~nonempty] == 0).all()
        assert kl.min() >= -1e-5
        assert np.abs(dz.sum(-1, dtype=np.float64)).max() <= 1e-5
    a, b = outs[False], outs[True]
    np.testing.assert_allclose(b["nc_lse"], a["nc_lse"], rtol=2 * NC_RTOL, atol=2 * NC_ATOL)
    np.testing.assert_allclose(b["target"], a["target"], rtol=0, atol=2 * T_ATOL)
    np.testing.assert_allclose(b["kl_rows"], a["kl_rows"], rtol=2 * KL_RTOL, atol=2 * KL_ATOL)
    assert a["stats"][1] == b["stats"][1] == nonempty.sum()


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_shuffled_padding_parity(fused):
    run_config("c2", shuffle_pad=True, fused=fused)


def test_fused_without_nc_out_and_floor_options():
    """distill_target_fused: the target is bitwise the same with and without the optional
    nc_lse output, its nc_lse matches window_lse within the nc tolerance, and the legacy
    1e-10 floor clips local-dominant rows exactly as on the three-call path."""
    sd = _sd()
    dev = _dev()
    for name in ("c2", "c1_local"):
        x = synth.make_inputs(name, shuffle_pad=True)
        c = x["cfg"]
        g = _to(x, dev)
        _say(f"[gpu] {name}: fused options")
        T1, nc1 = sd.distill_target_fused(g["q"], g["kwin"], g["pool"], g["idx"], g["sink"], g["seg"], W=c.W,
                                          want_nc=True)
        T2 = sd.distill_target_fused(g["q"], g["kwin"], g["pool"], g["idx"], g["sink"], g["seg"], W=c.W)
        nc3 = sd.window_lse(g["q"], g["kwin"], g["sink"], g["seg"], W=c.W)
        Tl = sd.distill_target_fused(g["q"], g["kwin"], g["pool"], g["idx"], g["sink"], g["seg"], W=c.W,
                                     l1_floor=1e-10)
        Tl3 = sd.distill_target(g["q"], g["pool"], g["idx"], nc3, l1_floor=1e-10)
        torch.cuda.synchronize()
        assert torch.equal(T1, T2)
        check_nc(_np(nc1).reshape(-1, c.H), _np(nc3).reshape(-1, c.H).astype(np.float64), name + " fused nc")
        idx = x["idx"].reshape(-1, c.K).numpy()
        Tl_ref = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=c.W, scale=c.scale,
                               floor=1e-10)
        check_T(_np(Tl).reshape(-1, c.K), Tl_ref, idx, c.N, name + " fused 1e-10 floor")
        check_T(_np(Tl3).reshape(-1, c.K), Tl_ref, idx, c.N, name + " 3-call 1e-10 floor")


# ------------------------------------------------------------------ isolated kernels
def test_target_isolated_with_given_nc_lse_and_legacy():
    sd = _sd()
    dev = _dev()
    for name in ("c1", "c2"):
        x = synth.make_inputs(name, shuffle_pad=True)
        c = x["cfg"]
        nc_ref = oracle.window_lse(x["q"], x["kwin"], x["sink"], x["seg"], c.W, c.scale)
        nc32 = torch.from_numpy(nc_ref.astype(np.float32)).reshape(c.B, c.S, c.H)
        g = _to(x, dev)
        _say(f"[gpu] {name}: target with oracle nc_lse, and legacy")
        T = sd.distill_target(g["q"], g["pool"], g["idx"], nc32.to(dev))
        Tl = sd.distill_target(g["q"], g["pool"], g["idx"], None, l1_floor=1e-10)
        torch.cuda.synchronize()
        T_ref = oracle.target(x["q"], x["pool"], x["idx"], nc_lse=nc32.reshape(-1, c.H).double().numpy(),
                              scale=c.scale)
        Tl_ref = oracle.target(x["q"], x["pool"], x["idx"], scale=c.scale, floor=1e-10)
        idx = x["idx"].reshape(-1, c.K).numpy()
        check_T(_np(T).reshape(-1, c.K), T_ref, idx, c.N, name + " given nc")
        check_T(_np(Tl).reshape(-1, c.K), Tl_ref, idx, c.N, name + " legacy")


def test_local_dominant_floor_on_gpu():
    """Local-dominant rows: float32-tiny floor renormalises to 1, the legacy floor clips."""
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs("c1_local")
    c = x["cfg"]
    g = _to(x, dev)
    _say("[gpu] c1_local: floors")
    nc = sd.window_lse(g["q"], g["kwin"], g["sink"], g["seg"], W=c.W)
    T = _np(sd.distill_target(g["q"], g["pool"], g["idx"], nc)).reshape(-1, c.K)
    Tl = _np(sd.distill_target(g["q"], g["pool"], g["idx"], nc, l1_floor=1e-10)).reshape(-1, c.K)
    idx = x["idx"].reshape(-1, c.K).numpy()
    ne = ((idx >= 0) & (idx < c.N)).any(-1)
    np.testing.assert_allclose(T[ne].sum(-1), 1.0, atol=1e-5)
    assert (Tl[ne].sum(-1) < 1e-3).all()
    mass_ref = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=c.W,
                             scale=c.scale, floor=1.0).sum(-1)
    np.testing.assert_allclose(Tl[ne].sum(-1), mass_ref[ne] / 1e-10, rtol=1e-3)


def test_kl_isolated_all_configs():
    """KL kernel alone on oracle-independent inputs: T is a normalised random row."""
    sd = _sd()
    dev = _dev()
    for name in ("c1", "c2", "c3", "c5"):
        x = synth.make_inputs(name) if name in ("c1", "c2") else None
        c = synth.CONFIGS[name]
        idx = x["idx"] if x is not None else torch.from_numpy(synth.topk_slots(c, synth.rng_for(c, "idx")))
        rng = np.random.default_rng(c.cid)
        valid = ((idx >= 0) & (idx < c.N)).numpy()
        r = rng.random(idx.shape).astype(np.float32) * valid
        s = r.sum(-1, keepdims=True)
        T = np.where(s > 0, r / np.where(s > 0, s, 1), 0).astype(np.float32)
        z = rng.standard_normal(idx.shape).astype(np.float32)
        z[~valid] = np.nan                                   # never read into the arithmetic
        _say(f"[gpu] {name}: KL isolated")
        kl, dz, st = sd.distill_kl_fwd_bwd(torch.from_numpy(T).to(dev), torch.from_numpy(z).to(dev),
                                           idx.to(dev), c.N, grad_scale=0.5)
        torch.cuda.synchronize()
        kl_ref, dz_ref, st_ref = oracle.kl(T, z, idx, c.N, grad_scale=0.5)
        check_kl(_np(kl).reshape(-1), _np(dz).reshape(-1, c.K), kl_ref, dz_ref, idx.reshape(-1, c.K).numpy(),
                 c.N, name, T.reshape(-1, c.K), grad_scale=0.5)
        stn = _np(st)
        assert stn[1] == st_ref[1]
        assert abs(stn[0] - st_ref[0]) <= KL_RTOL * abs(st_ref[0])
        # forward-only call gives the same forward numbers
        kl2, dz2, st2 = sd.distill_kl_fwd_bwd(torch.from_numpy(T).to(dev), torch.from_numpy(z).to(dev),
                                              idx.to(dev), c.N, want_grad=False)
        assert dz2 is None
        assert torch.equal(kl2, kl) and torch.equal(st2, st)


def test_kl_shared_workspace_across_calls():
    """One workspace serves consecutive calls of different sizes (stale partials from a
    larger call never leak into a smaller one), and stats match the oracle each time."""
    sd = _sd()
    dev = _dev()
    cases = [("c2", None), ("c1", None), ("c2", 7)]
    big = max(sd.distill_kl_workspace_bytes(synth.CONFIGS[n].B, synth.CONFIGS[n].S, synth.CONFIGS[n].K)
              for n, _ in cases)
    ws = torch.full((big,), 0x7F, dtype=torch.uint8, device=dev)  # garbage, not zeros
    for name, seed in cases:
        c = synth.CONFIGS[name]
        x = synth.make_inputs(name)
        idx = x["idx"]
        rng = np.random.default_rng(c.cid if seed is None else seed)
        valid = ((idx >= 0) & (idx < c.N)).numpy()
        r = rng.random(idx.shape).astype(np.float32) * valid
        sm = r.sum(-1, keepdims=True)
        T = np.where(sm > 0, r / np.where(sm > 0, sm, 1), 0).astype(np.float32)
        z = rng.standard_normal(idx.shape).astype(np.float32)
        _say(f"[gpu] {name}: KL with a shared workspace (seed {seed})")
        kl, dz, st = sd.distill_kl_fwd_bwd(torch.from_numpy(T).to(dev), torch.from_numpy(z).to(dev),
                                           idx.to(dev), c.N, grad_scale=1.0, workspace=ws)
        torch.cuda.synchronize()
        _, _, st_ref = oracle.kl(T, z, idx, c.N, grad_scale=1.0)
        stn = _np(st)
        assert stn[1] == st_ref[1]
        assert abs(stn[0] - st_ref[0]) <= KL_RTOL * abs(st_ref[0])


# ------------------------------------------------------------------ edge shapes
EDGE = [
    # (name, B, S, H, D, N, K, W, dtype, segments)
    ("ragged", 2, 37, 5, 64, 9, 13, 6, "bf16", 1),
    ("k1_sparse", 1, 40, 16, 32, 10, 1, 3, "bf16", 1),
    ("w1", 1, 24, 3, 32, 6, 4, 1, "f32", 1),
    ("w_gt_s", 1, 20, 16, 32, 5, 6, 128, "bf16", 1),
    ("h20_d96", 1, 50, 20, 96, 12, 20, 17, "bf16", 2),
    ("h64_k1024", 1, 64, 64, 512, 16, 1024, 128, "bf16", 1),
    ("all_empty", 1, 3, 4, 32, 4, 4, 2, "f32", 1),
    ("f32_h64", 1, 48, 64, 128, 12, 40, 33, "f32", 1),
    ("k_gt_blocks", 2, 44, 8, 32, 11, 300, 20, "bf16", 1),
    # D = 512 bf16 with several tokens per CU: 1, 2 and 4 head tiles, 2 and 3 batch rows
    ("persist_b2_h20", 2, 600, 20, 512, 150, 300, 33, "bf16", 1),
    ("persist_b3_h64", 3, 400, 64, 512, 100, 512, 64, "bf16", 2),
    ("persist_k16_h5", 1, 1024, 5, 512, 256, 16, 40, "bf16", 1),
    # four waves per token (K <= 256) holding all eight window tiles two to a wave; W = 120
    # leaves the last window tile partly masked, across two segments
    ("w128_four_waves", 1, 300, 16, 128, 75, 64, 128, "bf16", 1),
    ("w120_four_waves_seg", 1, 264, 8, 64, 66, 200, 120, "bf16", 2),
    # fp32 inputs on the 16-wave workgroup (K > 512, H > 32) with up to four slot tiles per
    # wave, scored in passes of two, and all eight window tiles
    ("f32_h40_k1024", 1, 4200, 40, 32, 1050, 1024, 128, "f32", 1),
    # 64 < K <= 128: two slot tiles per wave on four waves, bf16 with 64 heads and fp32 with
    # 24 heads (two head tiles, the second one partly filled)
    ("k100_h64_bf16", 1, 600, 64, 512, 150, 100, 128, "bf16", 1),
    ("k128_h64_bf16_seg", 1, 800, 64, 256, 200, 128, 96, "bf16", 2),
    ("k128_h24_f32", 1, 560, 24, 64, 140, 128, 64, "f32", 1),
    ("k100_h24_bf16", 2, 450, 24, 128, 112, 100, 50, "bf16", 1),
]


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("case", EDGE, ids=lambda e: e[0])
def test_edge_shapes(case, fused):
    name, B, S, H, D, N, K, W, dt, segs = case
    cid = 800 + EDGE.index(case)
    if segs > 1:
        S = (S // (4 * segs)) * 4 * segs
        N = S // 4
    cfg = synth.Config(name, cid, B=B, S=S, H=H, D=D, N=N, K=K, W=W, dtype=dt, segments=segs)
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs(cfg, shuffle_pad=True)
    g = _to(x, dev)
    _say(f"[gpu] edge {name}: B={B} S={S} H={H} D={D} N={N} K={K} W={W} {dt} segs={segs} fused={fused}")
    out = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=W,
                               grad_scale=1.0, fused=fused)
    torch.cuda.synchronize()
    nc_ref = oracle.window_lse(x["q"], x["kwin"], x["sink"], x["seg"], W, cfg.scale)
    T_ref = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=W, scale=cfg.scale)
    idx = x["idx"].reshape(-1, K).numpy()
    kl_ref, dz_ref, _ = oracle.kl(T_ref.astype(np.float32), x["z"], x["idx"], N)
    check_nc(_np(out["nc_lse"]).reshape(-1, H), nc_ref, name)
    check_T(_np(out["target"]).reshape(-1, K), T_ref, idx, N, name)
    check_kl(_np(out["kl_rows"]).reshape(-1), _np(out["dlogits"]).reshape(-1, K), kl_ref, dz_ref, idx, N, name,
             T_ref, dT_rows=np.abs(_np(out["target"]).reshape(-1, K) - T_ref).max(-1))


# ------------------------------------------------------------------ poison, isolation, determinism
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_poison_unreferenced_inputs_leave_outputs_bitwise_unchanged(fused):
    sd = _sd()
    dev = _dev()
    cfg = synth.Config("poison", 851, B=1, S=256, H=16, D=128, N=64, K=16, W=20, dtype="bf16", segments=2)
    x = synth.make_inputs(cfg, shuffle_pad=True)
    idx = x["idx"].clone()
    # (a) drop every reference to a set of pool rows, then poison those rows
    dropped = torch.tensor([0, 5, 17, 40, 63])
    idx[torch.isin(idx, dropped)] = -1
    g = _to(x, dev)
    g["idx"] = idx.to(dev)
    _say(f"[gpu] poison: clean run (fused={fused})")
    ref = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=cfg.W,
                               fused=fused)
    pool_p = g["pool"].clone()
    pool_p[:, dropped] = float("nan")
    # (b) keys of segment 0 poisoned: tokens of segment 1 must not see them
    kwin_p = g["kwin"].clone()
    kwin_p[:, : cfg.S // 2] = float("inf")
    # (c) student logits at invalid slots poisoned
    z_p = g["z"].clone()
    z_p[~((g["idx"] >= 0) & (g["idx"] < cfg.N))] = float("nan")
    _say(f"[gpu] poison: poisoned run (fused={fused})")
    out = sd.csa_distill_layer(g["q"], kwin_p, pool_p, g["idx"], z_p, g["sink"], g["seg"], W=cfg.W, fused=fused)
    torch.cuda.synchronize()
    h = cfg.S // 2
    # segment 1 never sees segment 0's keys (the fused kernel loads them and masks them after)
    assert torch.equal(out["nc_lse"][:, h:], ref["nc_lse"][:, h:])
    assert torch.equal(out["target"][:, h:], ref["target"][:, h:])
    assert torch.equal(out["dlogits"][:, h:], ref["dlogits"][:, h:])
    # pool poison only touches unreferenced rows: targets of every token bitwise equal
    if fused:
        T2 = sd.distill_target_fused(g["q"], g["kwin"], pool_p, g["idx"], g["sink"], g["seg"], W=cfg.W)
    else:
        T2 = sd.distill_target(g["q"], pool_p, g["idx"], ref["nc_lse"])
    assert torch.equal(T2, ref["target"])
    # window keys past the token (the fused kernel loads rows past t as row t, then masks them):
    # poisoning keys after the last token of each query's window leaves earlier tokens unchanged
    kwin_f = g["kwin"].clone()
    kwin_f[:, h + 8:] = float("nan")
    o3 = sd.csa_distill_layer(g["q"], kwin_f, g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=cfg.W,
                              fused=fused)
    torch.cuda.synchronize()
    assert torch.equal(o3["nc_lse"][:, : h + 8], ref["nc_lse"][:, : h + 8])
    assert torch.equal(o3["target"][:, : h + 8], ref["target"][:, : h + 8])
    kl2, dz2, st2 = sd.distill_kl_fwd_bwd(ref["target"], z_p, g["idx"], cfg.N)
    assert torch.equal(kl2, ref["kl_rows"]) and torch.equal(dz2, ref["dlogits"]) and torch.equal(st2, ref["stats"])


def test_segment_isolation_perturbation():
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs("c4")
    c = x["cfg"]
    g = _to(x, dev)
    _say("[gpu] c4: segment isolation")
    nc = sd.window_lse(g["q"], g["kwin"], g["sink"], g["seg"], W=c.W)
    k2 = g["kwin"].clone()
    k2[:, : c.S // 2] = torch.randn_like(k2[:, : c.S // 2])
    nc2 = sd.window_lse(g["q"], k2, g["sink"], g["seg"], W=c.W)
    torch.cuda.synchronize()
    assert torch.equal(nc[:, c.S // 2:], nc2[:, c.S // 2:])
    assert not torch.equal(nc[:, : c.S // 2], nc2[:, : c.S // 2])


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_deterministic_bitwise(fused):
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs("c3")
    c = x["cfg"]
    g = _to(x, dev)
    _say(f"[gpu] c3: determinism (fused={fused})")
    a = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=c.W, fused=fused)
    a = {k: v.clone() for k, v in a.items()}
    b = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=c.W, fused=fused)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_graph_capture_replays_match_eager(fused):
    """A layer step captured as a HIP graph replays bit-identically to the eager step, on
    every replay, with other eager work (a different layer into other buffers) between
    the replays.  Every kernel reduction has a fixed order, so equality is exact."""
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs("c2")
    c = x["cfg"]
    g = _to(x, dev)
    B, S, H, K = c.B, c.S, c.H, c.K

    def new_bufs():
        return dict(nc_lse=torch.empty(B, S, H, device=dev), target=torch.empty(B, S, K, device=dev),
                    kl_rows=torch.empty(B, S, device=dev), dlogits=torch.empty(B, S, K, device=dev),
                    stats=torch.empty(2, device=dev),
                    workspace=torch.empty(sd.distill_kl_workspace_bytes(B, S, K), dtype=torch.uint8, device=dev))

    bufs, other = new_bufs(), new_bufs()
    run = lambda bb, z: sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], z, g["sink"], g["seg"],
                                             W=c.W, grad_scale=0.5, fused=fused, bufs=bb)
    _say(f"[gpu] c2: graph capture ({'fused' if fused else '3call'})")
    ref = {k: v.clone() for k, v in run(bufs, g["z"]).items()}
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(bufs, g["z"])
    z2 = g["z"] * 1.5 + 0.25
    for rep in range(3):
        for v in bufs.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(bufs[k], ref[k]), (rep, k)
        run(other, z2)  # eager work between the replays
        torch.cuda.synchronize()


def test_binding_rejects_bad_arguments_on_gpu_tensors():
    sd = _sd()
    dev = _dev()
    q = torch.zeros(1, 8, 4, 48, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 8, 48, dtype=torch.bfloat16, device=dev)
    with pytest.raises(NotImplementedError):
        sd.window_lse(q, k, None, None, W=4)                       # D=48 unsupported
    q = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 8, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        sd.window_lse(q, k, torch.zeros(3, device=dev), None, W=4)  # sink size
    with pytest.raises(ValueError):
        sd.window_lse(q, k, None, None, W=0)
    with pytest.raises(NotImplementedError):
        sd.window_lse(q, k, None, None, W=129)


def test_binding_rejects_bad_output_buffers():
    """Caller-provided outputs and workspaces are written in place, so the binding refuses
    any that is on the host, of the wrong shape or dtype, non-contiguous or too small,
    before anything is launched."""
    sd = _sd()
    dev = _dev()
    B, S, H, D, N, K = 1, 16, 4, 64, 4, 4
    q = torch.zeros(B, S, H, D, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(B, S, D, dtype=torch.bfloat16, device=dev)
    pool = torch.zeros(B, N, D, dtype=torch.bfloat16, device=dev)
    idx = torch.full((B, S, K), -1, dtype=torch.int32, device=dev)
    bad_nc = [torch.empty(B, S, H),                                         # host
              torch.empty(B, S, H + 1, device=dev),                         # shape
              torch.empty(B, S, H, dtype=torch.float64, device=dev),        # dtype
              torch.empty(B, H, S, device=dev).transpose(1, 2)]             # non-contiguous
    for out in bad_nc:
        with pytest.raises(ValueError):
            sd.window_lse(q, k, None, None, W=4, out=out)
        with pytest.raises(ValueError):
            sd.distill_target_fused(q, k, pool, idx, None, None, W=4, nc_out=out)
    for out in (torch.empty(B, S, K), torch.empty(B, S, K + 1, device=dev)):
        with pytest.raises(ValueError):
            sd.distill_target(q, pool, idx, None, out=out)
        with pytest.raises(ValueError):
            sd.distill_target_fused(q, k, pool, idx, None, None, W=4, out=out)
    T = torch.zeros(B, S, K, device=dev)
    z = torch.zeros(B, S, K, device=dev)
    with pytest.raises(ValueError):
        sd.distill_kl_fwd_bwd(T, z, idx, N, stats=torch.empty(3, device=dev))
    with pytest.raises(ValueError):
        sd.distill_kl_fwd_bwd(T, z, idx, N, kl_rows=torch.empty(B, S))
    with pytest.raises(ValueError):
        sd.distill_kl_fwd_bwd(T, z, idx, N, dlogits=torch.empty(B, S, K - 1, device=dev))
    with pytest.raises(ValueError):
        sd.distill_kl_fwd_bwd(T, z, idx, N, workspace=torch.empty(1, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        sd.distill_kl_fwd_bwd(T, z, idx, N, workspace=torch.empty(64, dtype=torch.uint8))
    # valid calls still go through after the rejections
    kl, dz, st = sd.distill_kl_fwd_bwd(T, z, idx, N)
    torch.cuda.synchronize()
    assert st.tolist() == [0.0, 0.0] and (kl == 0).all() and (dz == 0).all()


def test_int64_slots_outside_range_never_wrap_into_valid_rows():
    """An int64 slot such as 2^32 + 1 must stay invalid (it would read as row 1 if it were
    simply cast to int32): target, KL and gradient equal those of the same row with -1."""
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs("c2")
    c = x["cfg"]
    g = _to(x, dev)
    idx64 = g["idx"].to(torch.int64)
    ref_idx = g["idx"].clone()
    t = c.S - 1                                   # a full row: every slot valid
    idx64[0, t, 0] = (1 << 32) + 1
    idx64[0, t, 1] = -(1 << 33)
    ref_idx[0, t, 0] = -1
    ref_idx[0, t, 1] = -1
    _say("[gpu] c2: int64 slots")
    nc = sd.window_lse(g["q"], g["kwin"], g["sink"], g["seg"], W=c.W)
    T64 = sd.distill_target(g["q"], g["pool"], idx64, nc)
    Tref = sd.distill_target(g["q"], g["pool"], ref_idx, nc)
    Tf64 = sd.distill_target_fused(g["q"], g["kwin"], g["pool"], idx64, g["sink"], g["seg"], W=c.W)
    Tfref = sd.distill_target_fused(g["q"], g["kwin"], g["pool"], ref_idx, g["sink"], g["seg"], W=c.W)
    kl64, dz64, st64 = sd.distill_kl_fwd_bwd(Tref, g["z"], idx64, c.N)
    klr, dzr, str_ = sd.distill_kl_fwd_bwd(Tref, g["z"], ref_idx, c.N)
    torch.cuda.synchronize()
    assert torch.equal(T64, Tref) and torch.equal(Tf64, Tfref)
    assert torch.equal(kl64, klr) and torch.equal(dz64, dzr) and torch.equal(st64, str_)
    assert T64[0, t, 0] == 0 and T64[0, t, 1] == 0


# ------------------------------------------------------------------ readings and numerics edges
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_duplicate_slots_parity(name, fused):
    """A block selected twice is two softmax entries (the oracle's reading, pinned on the CPU
    against a pool with the row copied); both slots get the same target value."""
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs(name, shuffle_pad=True)
    c = x["cfg"]
    idx = torch.from_numpy(synth.duplicate_slots(x["idx"].numpy(), c.N, c.cid))
    g = _to(x, dev)
    _say(f"[gpu] {name}: duplicate slots (fused={fused})")
    out = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], idx.to(dev), g["z"], g["sink"], g["seg"], W=c.W,
                               fused=fused)
    torch.cuda.synchronize()
    T_ref = oracle.target(x["q"], x["pool"], idx, x["kwin"], x["sink"], x["seg"], W=c.W, scale=c.scale)
    idx2 = idx.reshape(-1, c.K).numpy()
    check_T(_np(out["target"]).reshape(-1, c.K), T_ref, idx2, c.N, name + " duplicates")
    kl_ref, dz_ref, _ = oracle.kl(T_ref.astype(np.float32), x["z"], idx, c.N)
    check_kl(_np(out["kl_rows"]).reshape(-1), _np(out["dlogits"]).reshape(-1, c.K), kl_ref, dz_ref, idx2, c.N,
             name + " duplicates", T_ref, dT_rows=np.abs(_np(out["target"]).reshape(-1, c.K) - T_ref).max(-1))


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("case", [("c1", 1, 64, 4, 32, 16, 8, 8, "f32"), ("c2", 1, 1024, 16, 128, 256, 64, 64, "bf16"),
                                  ("v4", 1, 700, 64, 512, 175, 512, 128, "bf16")], ids=lambda c: c[0])
def test_row_mass_below_float32_tiny(case, fused):
    """Every head's sink at +100: each head's compressed share is ~e^-94, so a row's mass is
    below float32 tiny (2^-126) and the floor itself binds: T = m / 2^-126 sums to less than 1.
    The kernels form the row total in the log2 domain, so nothing underflows before the floor."""
    name, B, S, H, D, N, K, W, dt = case
    cfg = synth.Config(f"tiny_mass_{name}", 870 + ["c1", "c2", "v4"].index(name), B=B, S=S, H=H, D=D, N=N, K=K, W=W,
                       dtype=dt, sink_hot_heads=H, sink_hot_value=100.0)
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs(cfg)
    g = _to(x, dev)
    _say(f"[gpu] {cfg.name}: row mass below float32 tiny (fused={fused})")
    out = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=W,
                               fused=fused)
    torch.cuda.synchronize()
    T_ref = oracle.target(x["q"], x["pool"], x["idx"], x["kwin"], x["sink"], x["seg"], W=W, scale=cfg.scale)
    idx = x["idx"].reshape(-1, K).numpy()
    ne = ((idx >= 0) & (idx < N)).any(-1)
    rs = T_ref.sum(-1)
    assert (rs[ne] < 0.5).all() and (rs[ne] > 0).all(), "the floor must bind on every non-empty row"
    T = _np(out["target"]).reshape(-1, K)
    check_T(T, T_ref, idx, N, cfg.name)
    # relative agreement of the row sums (the values are far from zero)
    np.testing.assert_allclose(T[ne].sum(-1), rs[ne], rtol=1e-4)


def test_kl_subnormal_target_values():
    """Target values below float32 tiny on valid slots: log T is exact for them, so the row
    KL stays finite and matches the oracle."""
    sd = _sd()
    dev = _dev()
    c = synth.CONFIGS["c2"]
    x = synth.make_inputs("c2")
    idx = x["idx"]
    rng = np.random.default_rng(77)
    valid = ((idx >= 0) & (idx < c.N)).numpy()
    r = rng.random(idx.shape).astype(np.float32) * valid
    sm = r.sum(-1, keepdims=True)
    T = np.where(sm > 0, r / np.where(sm > 0, sm, 1), 0).astype(np.float32)
    sub = valid & (rng.random(idx.shape) < 0.2)
    T[sub] = np.float32(1e-41) * rng.integers(1, 1000, size=sub.sum()).astype(np.float32)   # subnormal
    assert (T[sub] < np.finfo(np.float32).tiny).all() and (T[sub] > 0).all()
    z = rng.standard_normal(idx.shape).astype(np.float32)
    _say("[gpu] c2: KL with subnormal target values")
    kl, dz, st = sd.distill_kl_fwd_bwd(torch.from_numpy(T).to(dev), torch.from_numpy(z).to(dev), idx.to(dev), c.N)
    torch.cuda.synchronize()
    kl_ref, dz_ref, st_ref = oracle.kl(T, z, idx, c.N)
    check_kl(_np(kl).reshape(-1), _np(dz).reshape(-1, c.K), kl_ref, dz_ref, idx.reshape(-1, c.K).numpy(), c.N,
             "subnormal T", T.reshape(-1, c.K))
    assert _np(st)[1] == st_ref[1]


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_explicit_side_stream_matches_default_stream(fused):
    """stream= runs the whole wrapper (temporaries included: a non-contiguous q, int64 slots,
    default outputs and workspace) on the given stream; results equal the default stream's
    bit for bit."""
    sd = _sd()
    dev = _dev()
    x = synth.make_inputs("c2")
    c = x["cfg"]
    g = _to(x, dev)
    ref = sd.csa_distill_layer(g["q"], g["kwin"], g["pool"], g["idx"], g["z"], g["sink"], g["seg"], W=c.W,
                               fused=fused)
    ref = {k: v.clone() for k, v in ref.items()}
    torch.cuda.synchronize()
    q_nc = g["q"].transpose(1, 2).contiguous().transpose(1, 2)     # same values, not contiguous
    assert not q_nc.is_contiguous()
    idx64 = g["idx"].to(torch.int64)
    side = torch.cuda.Stream(device=dev)
    _say(f"[gpu] c2: side stream (fused={fused})")
    for _ in range(3):
        out = sd.csa_distill_layer(q_nc, g["kwin"], g["pool"], idx64, g["z"], g["sink"], g["seg"], W=c.W,
                                   fused=fused, stream=side)
        side.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), k
