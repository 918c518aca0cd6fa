"""Pins for the oracle's indexer selection and its gradient scatter (CPU only).

The selection follows the MaxText PR "Add Indexer Loss [Deepseek v4]": top-k of the
student's block scores under the causal block mask combined with the segment (packing)
mask, unused slots set to -1.  Readings the tests encode (stated in the oracle too):
block n = tokens ratio*n .. ratio*n+ratio-1 is visible to t iff it is complete at t and all
its tokens share t's segment; equal scores prefer the smaller block index; NaN ranks
lowest; kept blocks are written in ascending block order, then -1; a -1 slot's value is
-inf.  The gradient is the adjoint of the gather values = scores[idx].
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def visible_mask(S, N, ratio, seg_b):
    """[S, N] boolean by a vectorised formulation: complete blocks, whole-block segment match."""
    t = np.arange(S)[:, None]
    n = np.arange(N)[None, :]
    vis = ratio * n + ratio - 1 <= t
    if seg_b is not None:
        tok = ratio * np.arange(N)[:, None] + np.arange(ratio)[None, :]        # [N, ratio]
        inb = tok < S
        seg_tok = np.where(inb, seg_b[np.minimum(tok, S - 1)], np.iinfo(np.int64).min)
        same = (seg_tok[None, :, :] == seg_b[:, None, None]).all(-1)          # [S, N]
        vis &= same
    return vis


def numpy_topk(scores, seg, K, ratio):
    """Selection by numpy.lexsort on (NaN flag, -score, index) over the visible blocks."""
    scores = np.asarray(scores, dtype=np.float32)
    B, S, N = scores.shape
    idx = np.full((B, S, K), -1, dtype=np.int32)
    val = np.full((B, S, K), -np.inf, dtype=np.float32)
    for b in range(B):
        vis = visible_mask(S, N, ratio, None if seg is None else np.asarray(seg)[b].astype(np.int64))
        for t in range(S):
            n = np.flatnonzero(vis[t])
            s = scores[b, t, n].astype(np.float64)
            nan = np.isnan(s)
            order = np.lexsort((n, -np.where(nan, 0.0, s), nan))  # last key is primary
            keep = np.sort(n[order[:K]])
            idx[b, t, : len(keep)] = keep
            val[b, t, : len(keep)] = scores[b, t, keep]
    return idx, val


def rand_scores(B, S, N, seed, ties=False):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((B, S, N)).astype(np.float32)
    if ties:
        s = np.floor(s * 2).astype(np.float32)          # few distinct values: many ties
    return s


CASES = [
    # (B, S, N, K, ratio, segments, ties)
    (1, 64, 16, 8, 4, 1, False),
    (2, 72, 18, 5, 4, 1, True),
    (1, 96, 24, 7, 4, 2, True),
    (2, 90, 30, 4, 3, 1, False),       # ratio 3, N beyond S/ratio
    (1, 128, 16, 6, 8, 2, False),      # HCA-like wider blocks
    (1, 40, 10, 10, 4, 1, True),       # K = N
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_topk_matches_numpy_lexsort(case):
    B, S, N, K, ratio, segs, ties = case
    s = rand_scores(B, S, N, seed=sum(case[:5]), ties=ties)
    seg = None
    if segs > 1:
        L = S // segs
        seg = np.repeat(np.arange(segs, dtype=np.int32), L)[None].repeat(B, 0)
        seg = np.pad(seg, ((0, 0), (0, S - seg.shape[1])), mode="edge")
    i, v = oracle.indexer_topk(s, seg, K, ratio)
    ri, rv = numpy_topk(s, seg, K, ratio)
    np.testing.assert_array_equal(i, ri.reshape(i.shape))
    np.testing.assert_array_equal(v, rv.reshape(v.shape))


def test_golden_t4_block_visibility():
    g = json.load(open(os.path.join(GOLDEN, "p3_t4_block_mask.json")))
    r, t = g["compress_ratio"], g["t"]
    S, N, K = 16, 4, 4
    s = np.zeros((1, S, N), dtype=np.float32)
    i, v = oracle.indexer_topk(s, None, K, r)
    row = i.reshape(S, K)[t]
    for n in g["visible_blocks"]:
        assert n in row
    for n in g["masked_blocks"]:
        assert n not in row
    np.testing.assert_array_equal(row, [0, -1, -1, -1])
    assert np.isneginf(v.reshape(S, K)[t, 1:]).all()


def test_ties_prefer_smaller_block_index():
    S, N, K = 64, 16, 5
    s = np.full((1, S, N), 0.5, dtype=np.float32)
    i, _ = oracle.indexer_topk(s, None, K, 4)
    i = i.reshape(S, K)
    np.testing.assert_array_equal(i[63], [0, 1, 2, 3, 4])
    # threshold inside a tie group: blocks 9 and 2 win outright, then ties at 1.0 by index
    s2 = np.zeros((1, S, N), dtype=np.float32)
    s2[0, 63, [9, 2]] = 5.0
    s2[0, 63, [3, 7, 11, 15]] = 1.0
    i2, v2 = oracle.indexer_topk(s2, None, K, 4)
    np.testing.assert_array_equal(i2.reshape(S, K)[63], [2, 3, 7, 9, 11])
    np.testing.assert_array_equal(v2.reshape(S, K)[63], [5.0, 1.0, 1.0, 5.0, 1.0])


def test_nan_ranks_below_every_number():
    S, N, K = 64, 16, 4
    s = np.full((1, S, N), np.nan, dtype=np.float32)
    s[0, 63, 14] = -np.inf
    s[0, 63, 3] = -1e30
    i, v = oracle.indexer_topk(s, None, K, 4)
    row, vals = i.reshape(S, K)[63], v.reshape(S, K)[63]
    # the two numbers first (by value), then NaN blocks by index: 0, 1
    assert set(row.tolist()) == {0, 1, 3, 14}
    np.testing.assert_array_equal(row, [0, 1, 3, 14])
    assert np.isnan(vals[:2]).all() and vals[2] == np.float32(-1e30) and np.isneginf(vals[3])


def test_block_straddling_a_segment_boundary_is_never_visible():
    S, N, K = 32, 8, 8
    seg = np.zeros((1, S), dtype=np.int32)
    seg[0, 10:] = 1                       # boundary inside block 2 (tokens 8..11)
    s = np.random.default_rng(3).standard_normal((1, S, N)).astype(np.float32)
    i, _ = oracle.indexer_topk(s, seg, K, 4)
    i = i.reshape(S, K)
    assert not (i == 2).any()
    for t in range(S):
        sel = set(i[t][i[t] >= 0].tolist())
        if t < 10:
            assert sel == set(range(min(2, (t + 1) // 4)))
        else:
            assert sel == set(range(3, (t + 1) // 4))


def test_selection_invariants_midsize():
    B, S, N, K, r = 2, 512, 128, 40, 4
    s = rand_scores(B, S, N, seed=11)
    i, v = oracle.indexer_topk(s, None, K, r)
    i, v = i.reshape(B, S, K), v.reshape(B, S, K)
    for b in range(B):
        for t in range(S):
            nvis = min(N, (t + 1) // r)
            row = i[b, t]
            kept = row[row >= 0]
            assert len(kept) == min(K, nvis)
            assert (row[len(kept):] == -1).all() and np.isneginf(v[b, t, len(kept):]).all()
            assert (np.diff(kept) > 0).all() and (kept < nvis).all()
            np.testing.assert_array_equal(v[b, t, : len(kept)], s[b, t, kept])
            rest = np.setdiff1d(np.arange(nvis), kept)
            if len(rest):
                assert s[b, t, kept].min() >= s[b, t, rest].max()


def test_selection_visible_set_matches_the_generator_rows_that_take_every_block():
    """The generator's top-k slots take all visible blocks when there are at most K of them:
    on those rows the selection (any scores) keeps exactly that set."""
    for name in ("c1", "c2"):
        x = synth.make_inputs(name)
        c = x["cfg"]
        s = rand_scores(c.B, c.S, c.N, seed=c.cid)
        i, _ = oracle.indexer_topk(s, x["seg"], c.K, 4)
        i = i.reshape(c.B, c.S, c.K)
        g = x["idx"].numpy()
        for t in range(c.S):
            gv = g[0, t][g[0, t] >= 0]
            if len(gv) < c.K:
                np.testing.assert_array_equal(i[0, t][i[0, t] >= 0], np.sort(gv))


def test_scatter_is_the_adjoint_of_the_gather():
    """<scatter(dv), s> = <dv, gather(s)> for random s and dv, including -1 and out-of-range
    slots (which gather nothing) and duplicate slots (whose gradients add)."""
    B, S, N, K = 2, 24, 10, 6
    rng = np.random.default_rng(5)
    idx = rng.integers(-2, N + 2, size=(B, S, K)).astype(np.int32)
    dv = rng.standard_normal((B, S, K)).astype(np.float32)
    sc = rng.standard_normal((B, S, N))
    ds = oracle.indexer_topk_bwd(dv, idx, N).reshape(B, S, N)
    valid = (idx >= 0) & (idx < N)
    gathered = np.where(valid, np.take_along_axis(sc, np.clip(idx, 0, N - 1), axis=2), 0.0)
    np.testing.assert_allclose((ds * sc).sum(), (dv.astype(np.float64) * gathered).sum(), rtol=1e-12)
    # entry by entry against numpy's unbuffered scatter-add
    ref = np.zeros((B, S, N))
    bb, tt, kk = np.nonzero(valid)
    np.add.at(ref, (bb, tt, idx[bb, tt, kk]), dv[bb, tt, kk].astype(np.float64))
    np.testing.assert_array_equal(ds, ref)


def test_scatter_of_a_selection_is_a_plain_copy():
    """Slots of one selection are distinct, so each kept block receives exactly its slot's
    gradient and every other block 0."""
    s = rand_scores(1, 80, 20, seed=9)
    i, _ = oracle.indexer_topk(s, None, 7, 4)
    i = i.reshape(1, 80, 7)
    dv = np.random.default_rng(9).standard_normal((1, 80, 7)).astype(np.float32)
    ds = oracle.indexer_topk_bwd(dv, i, 20).reshape(80, 20)
    for t in range(80):
        for k in range(7):
            if i[0, t, k] >= 0:
                assert ds[t, i[0, t, k]] == dv[0, t, k]
        assert np.count_nonzero(ds[t]) == np.count_nonzero(dv[0, t][i[0, t] >= 0])
