"""Pins for the oracle's compressor pool and its analytic backward (CPU only).

The compressor builds the compressed rows: a softmax over each entry's window of token
positions of (score + ape), per channel, weighting kv (Primus PR "Docker Build for
DeepSeek-v4 (Don't Merge)", commit fusing the compressed-attention small kernels; HCA
windows do not overlap, CSA windows do).  Readings the tests encode: entry n's window is
tokens r*n .. r*n+r-1 (no overlap) or r*(n-1) .. r*n+r-1 (overlap; positions before token 0
absent); ape is [Wc, D]; a position whose token lies in another segment than the entry's
last token is absent; the softmax runs over positions, separately for every channel.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_pool(kv, score, ape, seg, r, overlap):
    """Independent formulation: window index table, masked softmax with torch in float64."""
    kv = torch.as_tensor(kv, dtype=torch.float64)
    score = torch.as_tensor(score, dtype=torch.float64)
    ape = torch.as_tensor(ape, dtype=torch.float64)
    B, S, D = kv.shape
    N, Wc = S // r, r * (2 if overlap else 1)
    j = r * torch.arange(N)[:, None] - (r if overlap else 0) + torch.arange(Wc)[None, :]     # [N, Wc]
    present = (j >= 0).expand(B, N, Wc).clone()
    jc = j.clamp(min=0)
    if seg is not None:
        seg = torch.as_tensor(seg)
        last = seg[:, r * torch.arange(N) + r - 1]                                          # [B, N]
        present &= seg[:, jc] == last[:, :, None]
    logits = score[:, jc, :] + ape[None, None, :, :]                                        # [B, N, Wc, D]
    logits = logits.masked_fill(~present[..., None], -float("inf"))
    w = torch.softmax(logits, dim=2)
    return (w * kv[:, jc, :]).sum(2)


CASES = [
    # (B, S, D, r, overlap, segments)
    (2, 24, 5, 4, True, 1),
    (1, 27, 3, 4, False, 1),      # ragged tail: 3 tokens in no entry
    (2, 32, 4, 4, True, 2),
    (1, 64, 2, 16, False, 1),
    (1, 40, 3, 2, True, 2),
    (1, 256, 2, 128, False, 1),   # HCA-like
]


def _inputs(case, seed=0):
    B, S, D, r, overlap, segs = case
    rng = np.random.default_rng(seed + S + D + r)
    kv = rng.standard_normal((B, S, D)).astype(np.float32)
    score = rng.standard_normal((B, S, D)).astype(np.float32)
    ape = rng.standard_normal((r * (2 if overlap else 1), D)).astype(np.float32)
    seg = None
    if segs > 1:
        L = S // segs + 1                      # segment boundary inside a block
        seg = np.minimum(np.arange(S) // L, segs - 1).astype(np.int32)[None].repeat(B, 0)
    return kv, score, ape, seg


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_pool_matches_torch_formulation(case):
    kv, score, ape, seg = _inputs(case)
    r, overlap = case[3], case[4]
    p = oracle.compressor_pool(kv, score, ape, seg, r, overlap)
    ref = torch_pool(kv, score, ape, seg, r, overlap).numpy()
    np.testing.assert_allclose(p, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_matches_torch_autograd(case):
    kv, score, ape, seg = _inputs(case, seed=1)
    r, overlap = case[3], case[4]
    B, S, D = kv.shape
    dpool = np.random.default_rng(7).standard_normal((B, S // r, D)).astype(np.float32)
    dkv, dsc, dape = oracle.compressor_pool_bwd(kv, score, ape, seg, dpool, r, overlap)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (kv, score, ape)]
    (torch_pool(*t[:3], seg, r, overlap) * torch.as_tensor(dpool, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(dkv, t[0].grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dsc, t[1].grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dape, t[2].grad.numpy(), rtol=0, atol=1e-12)


def test_backward_matches_central_differences():
    case = (1, 16, 2, 4, True, 2)
    kv, score, ape, seg = _inputs(case, seed=3)
    r, overlap = 4, True
    dpool = np.random.default_rng(5).standard_normal((1, 4, 2)).astype(np.float32)
    dkv, dsc, dape = oracle.compressor_pool_bwd(kv, score, ape, seg, dpool, r, overlap)
    loss = lambda a, b, c: (oracle.compressor_pool(a, b, c, seg, r, overlap) * dpool).sum()
    h = np.float32(1e-3)
    for arr, grad, which in ((kv, dkv, 0), (score, dsc, 1), (ape, dape, 2)):
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = [kv, score, ape]
            args_m = [kv, score, ape]
            args_p[which], args_m[which] = ap, am
            fd = (loss(*args_p) - loss(*args_m)) / (float(ap[idx]) - float(am[idx]))
            assert abs(fd - grad[idx]) <= 1e-6 + 1e-5 * abs(grad[idx]), (which, idx, fd, grad[idx])


def test_single_position_window_copies_kv():
    kv, score, ape, _ = _inputs((2, 9, 3, 1, False, 1))
    p = oracle.compressor_pool(kv, score, ape, None, 1, False)
    np.testing.assert_array_equal(p, kv.astype(np.float64))


def test_equal_logits_average_the_present_positions():
    B, S, D, r = 1, 20, 3, 4
    kv = np.random.default_rng(2).standard_normal((B, S, D)).astype(np.float32)
    z = np.zeros((B, S, D), np.float32)
    p = oracle.compressor_pool(kv, z, np.zeros((2 * r, D), np.float32), None, r, True)
    kv64 = kv.astype(np.float64)
    np.testing.assert_allclose(p[0, 0], kv64[0, 0:4].mean(0), rtol=0, atol=1e-15)   # entry 0: own block only
    for n in range(1, S // r):
        np.testing.assert_allclose(p[0, n], kv64[0, r * n - r: r * n + r].mean(0), rtol=0, atol=1e-15)
    ph = oracle.compressor_pool(kv, z, np.zeros((r, D), np.float32), None, r, False)
    for n in range(S // r):
        np.testing.assert_allclose(ph[0, n], kv64[0, r * n: r * n + r].mean(0), rtol=0, atol=1e-15)


def test_softmax_runs_over_positions_per_channel():
    """A constant added to one channel's scores of every token leaves the pool unchanged (the
    softmax is over window positions, channel by channel), while the same constant added to one
    token changes its entries' pools."""
    kv, score, ape, seg = _inputs((1, 32, 4, 4, True, 1))
    score = (np.round(score * 1024) / 1024).astype(np.float32)   # on a grid where +3 is exact in float32
    p = oracle.compressor_pool(kv, score, ape, None, 4, True)
    s2 = score.copy()
    s2[..., 2] += np.float32(3.0)
    np.testing.assert_allclose(oracle.compressor_pool(kv, s2, ape, None, 4, True), p, rtol=0, atol=1e-12)
    s3 = score.copy()
    s3[0, 9] += np.float32(3.0)                 # token 9: block 2, in the windows of entries 2 and 3
    p3 = oracle.compressor_pool(kv, s3, ape, None, 4, True)
    changed = np.flatnonzero(np.abs(p3 - p).max(-1)[0] > 1e-9)
    np.testing.assert_array_equal(changed, [2, 3])


def test_segments_isolate_entries_and_overlap_reaches_one_block_back():
    B, S, D, r = 1, 32, 3, 4
    kv, score, ape, _ = _inputs((B, S, D, r, True, 1))
    seg = np.zeros((B, S), np.int32)
    seg[0, 16:] = 1                              # boundary between blocks 3 and 4
    p = oracle.compressor_pool(kv, score, ape, seg, r, True)
    kv2 = kv.copy()
    kv2[0, :16] = 99.0                           # rewrite the first document
    p2 = oracle.compressor_pool(kv2, score, ape, seg, r, True)
    np.testing.assert_array_equal(p2[0, 4:], p[0, 4:])     # entry 4 no longer reaches block 3
    assert (np.abs(p2[0, :4] - p[0, :4]) > 1e-3).all()
    # without segments entry 4 pools block 3 too
    p_noseg = oracle.compressor_pool(kv2, score, ape, None, r, True)
    assert np.abs(p_noseg[0, 4] - oracle.compressor_pool(kv, score, ape, None, r, True)[0, 4]).max() > 1e-3


def test_backward_tail_tokens_get_zero():
    kv, score, ape, _ = _inputs((1, 27, 3, 4, True, 1))
    dpool = np.ones((1, 6, 3), np.float32)
    dkv, dsc, _ = oracle.compressor_pool_bwd(kv, score, ape, None, dpool, 4, True)
    assert (dkv[0, 24:] == 0).all() and (dsc[0, 24:] == 0).all()
    # each entry's weights sum to one: the kv gradient of all tokens sums to sum(dpool)
    np.testing.assert_allclose(dkv.sum(), dpool.sum(), rtol=1e-12)
