"""Independent dense formulations used to pin the oracle on tiny inputs.

Where the oracle walks each query row and builds an explicit list of logits, these
routines build, per (batch, head), the full dense logit matrices of every query
against every window key and every pool row, mask them with boolean selection, and
take one masked log-sum-exp per query over [all window keys | all pool rows | sink].
The selected pool rows are read back out of the dense probability matrix by column.
Matrix products and log-sum-exp come from numpy/scipy/torch in float64.
"""
from __future__ import annotations

import numpy as np
import torch
from scipy.special import logsumexp

TINY = float(np.finfo(np.float32).tiny)


def _np64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def window_mask(S: int, W: int, seg_b) -> np.ndarray:
    """[S,S] boolean: key j in query t's window."""
    t = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = (j <= t) & (j > t - W)
    if seg_b is not None:
        m &= seg_b[:, None] == seg_b[None, :]
    return m


def selected_mask(idx_b: np.ndarray, N: int) -> np.ndarray:
    """[S,N] boolean: pool row n selected by query t (slots must be distinct)."""
    S, K = idx_b.shape
    m = np.zeros((S, N), dtype=bool)
    for t in range(S):
        for k in range(K):
            if 0 <= idx_b[t, k] < N:
                assert not m[t, idx_b[t, k]], "brute force needs distinct slots"
                m[t, idx_b[t, k]] = True
    return m


def target(q, pool, idx, kwin=None, sink=None, seg=None, W=0, scale=1.0, floor=0.0, extra=None):
    """extra: optional [B,S,H] natural-log logits, one more column of each head's list
    (a given non-compressed log-mass)."""
    q, pool, kwin, sink, extra = _np64(q), _np64(pool), _np64(kwin), _np64(sink), _np64(extra)
    idx = np.asarray(idx)
    B, S, H, D = q.shape
    N = pool.shape[1]
    K = idx.shape[2]
    fl = floor if floor > 0 else TINY
    T = np.zeros((B, S, K))
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        sel = selected_mask(idx[b], N)
        wm = window_mask(S, W, seg_b) if kwin is not None else np.zeros((S, S), bool)
        m = np.zeros((S, N))
        for h in range(H):
            Lp = scale * q[b, :, h, :] @ pool[b].T                      # [S,N]
            cols = [np.where(sel, Lp, -np.inf)]
            if kwin is not None:
                Lw = scale * q[b, :, h, :] @ kwin[b].T                  # [S,S]
                cols.append(np.where(wm, Lw, -np.inf))
            if sink is not None:
                cols.append(np.full((S, 1), sink[h]))
            if extra is not None:
                cols.append(extra[b, :, h][:, None])
            full = logsumexp(np.concatenate(cols, axis=1), axis=1)      # [S]
            with np.errstate(invalid="ignore"):
                P = np.where(sel, np.exp(Lp - full[:, None]), 0.0)
            m += P
        tot = m.sum(axis=1)
        for t in range(S):
            for k in range(K):
                n = idx[b, t, k]
                if 0 <= n < N:
                    T[b, t, k] = m[t, n] / max(tot[t], fl)
    return T


def window_lse(q, kwin, sink, seg, W, scale):
    """[B,S,H] via torch.logsumexp over the dense masked window matrix + sink column."""
    q = torch.as_tensor(_np64(q))
    kwin = torch.as_tensor(_np64(kwin))
    B, S, H, D = q.shape
    out = torch.empty(B, S, H, dtype=torch.float64)
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        wm = torch.as_tensor(window_mask(S, W, seg_b))
        for h in range(H):
            L = scale * q[b, :, h, :] @ kwin[b].T
            L = torch.where(wm, L, torch.tensor(-float("inf"), dtype=torch.float64))
            if sink is not None:
                L = torch.cat([L, torch.full((S, 1), float(_np64(sink)[h]), dtype=torch.float64)], 1)
            out[b, :, h] = torch.logsumexp(L, dim=1)
    return out.numpy()
