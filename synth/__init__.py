"""Seeded synthetic inputs for the CSA indexer-distillation path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it.  Every tensor is drawn on the host from
``numpy.random.Generator(PCG64(seed))`` with ``seed = 1000 * config + tensor_id``
(q=1, pool=2, kwin=3, sink=4, idx=5, logits=6, seg=7, row-pick=8), as N(0,1)
float32 and, for bf16 workloads, rounded to bfloat16 with round-to-nearest-even.

Shapes follow the workloads of the DeepSeek-V4 CSA layer described in the Primus
PR "perf(deepseek-v4): fuse and enable the indexer distillation loss" (V4-Flash
widths: 64 heads, head dim 512, top-k 512, window 128, compress ratio 4).

Top-k slots: a query at segment-local position t sees the completed blocks
n < floor((t+1)/4) of its own segment (block n covers tokens 4n..4n+3; the MaxText
PR "Add Indexer Loss [Deepseek v4]" gives the t=4 example: block 0 visible, block 1
not).  When at most K blocks are visible all of them are taken in random order and
the remaining slots hold -1 (the padding value of that PR's indexer); otherwise K
distinct blocks are drawn uniformly without replacement, in random order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TENSOR_ID = dict(q=1, pool=2, kwin=3, sink=4, idx=5, logits=6, seg=7, rowpick=8, scores=9, kv=10, cscore=11, ape=12,
                 dout=13)
COMPRESS_RATIO = 4


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cid: int            # numeric id used in the seeds
    B: int
    S: int
    H: int
    D: int
    N: int
    K: int
    W: int
    dtype: str = "bf16"          # element type of q / pool / kwin: "bf16" or "f32"
    segments: int = 1            # packed documents per batch row (equal lengths)
    sink_hot_heads: int = 0      # heads h < sink_hot_heads get sink = sink_hot_value
    sink_hot_value: float = 0.0
    window_bias_heads: int = 0   # heads h < window_bias_heads get +window_bias on window logits
    window_bias: float = 0.0
    kl_zero_frac: float = 0.0    # fraction of rows whose student logits are set to log T

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


def _c3(**kw):
    base = dict(B=1, S=4096, H=64, D=512, N=1024, K=512, W=128)
    base.update(kw)
    return base


CONFIGS = {
    # tiny all-fp32 case the oracle finishes in well under a second
    "c1": Config("c1", 1, B=1, S=64, H=4, D=32, N=16, K=8, W=8, dtype="f32"),
    "c2": Config("c2", 2, B=1, S=1024, H=16, D=128, N=256, K=64, W=64),
    # V4-Flash-shaped CSA layer
    "c3": Config("c3", 3, **_c3()),
    # edge-case stress at the V4-Flash shape: two packed segments, sink +30 and
    # window-logit bias +8 on half the heads, 10% of rows with student = log target
    "c4": Config("c4", 4, **_c3(), segments=2, sink_hot_heads=32, sink_hot_value=30.0,
                 window_bias_heads=32, window_bias=8.0, kl_zero_frac=0.1),
    # long-context CSA layer
    "c5": Config("c5", 5, B=2, S=8192, H=64, D=512, N=2048, K=1024, W=128),
    # local-dominant regime (every head sink = +76): the compressed share falls
    # below 1e-10 but stays above float32 tiny
    "c1_local": Config("c1_local", 41, B=1, S=64, H=4, D=32, N=16, K=8, W=8, dtype="f32",
                       sink_hot_heads=4, sink_hot_value=76.0),
    "c3_local": Config("c3_local", 43, **_c3(), sink_hot_heads=64, sink_hot_value=76.0),
}


def rng_for(cfg: Config, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg.cid + TENSOR_ID[tensor]))


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def segment_ids(cfg: Config) -> Optional[np.ndarray]:
    """[B,S] int32 segment ids (equal-length packed documents), or None for one segment."""
    if cfg.segments <= 1:
        return None
    L = cfg.S // cfg.segments
    assert L * cfg.segments == cfg.S and L % COMPRESS_RATIO == 0
    seg = np.repeat(np.arange(cfg.segments, dtype=np.int32), L)
    return np.broadcast_to(seg, (cfg.B, cfg.S)).copy()


def topk_slots(cfg: Config, rng: np.random.Generator, shuffle_pad: bool = False) -> np.ndarray:
    """[B,S,K] int32 top-k slots: causal, same-segment, distinct blocks, -1 padded."""
    B, S, K = cfg.B, cfg.S, cfg.K
    nseg = max(cfg.segments, 1)
    L = S // nseg
    out = np.empty((B, S, K), dtype=np.int32)
    t = np.arange(S)
    t_loc = t % L
    seg_base = (t // L) * (L // COMPRESS_RATIO)          # first pool row of t's segment
    n_vis = (t_loc + 1) // COMPRESS_RATIO                 # completed blocks visible to t
    nmax = int(n_vis.max())
    width = max(nmax, K)
    for b in range(B):
        for lo in range(0, S, 1024):                      # bounded memory per chunk
            hi = min(S, lo + 1024)
            u = rng.random((hi - lo, width))
            u[np.arange(width)[None, :] >= n_vis[lo:hi, None]] = np.inf
            order = np.argsort(u, axis=1, kind="stable")[:, :K]
            sel = order + seg_base[lo:hi, None]
            sel[np.arange(K)[None, :] >= n_vis[lo:hi, None]] = -1
            if shuffle_pad:
                perm = np.argsort(rng.random((hi - lo, K)), axis=1)
                sel = np.take_along_axis(sel, perm, axis=1)
            out[b, lo:hi] = sel
    return out


def duplicate_slots(idx: np.ndarray, N: int, seed: int) -> np.ndarray:
    """Copy of idx [B,S,K] in which, for about 70% of the rows with two or more valid slots,
    one valid slot repeats another valid slot of the same row, and a row with a single valid
    slot holds that block twice (the neighbouring slot is overwritten)."""
    rng = np.random.default_rng(seed)
    d = np.array(idx, copy=True)
    B, S, K = d.shape
    for b in range(B):
        for t in range(S):
            v = np.flatnonzero((d[b, t] >= 0) & (d[b, t] < N))
            if len(v) >= 2 and rng.random() < 0.7:
                src, dst = rng.choice(v, size=2, replace=False)
                d[b, t, dst] = d[b, t, src]
            elif len(v) == 1 and K > 1:
                d[b, t, (v[0] + 1) % K] = d[b, t, v[0]]
    return d


def student_scores(cfg: Config | str, ties: bool = False) -> torch.Tensor:
    """[B,S,N] float32 student block scores, N(0,1); with ties=True floor(2x), so only a
    dozen distinct values occur and top-k thresholds fall inside groups of equal scores."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    s = _normal(rng_for(cfg, "scores"), (cfg.B, cfg.S, cfg.N))
    if ties:
        s = np.floor(2.0 * s).astype(np.float32)
    return torch.from_numpy(s)


def compressor_inputs(cfg: Config | str, ratio: int, overlap: bool, dtype: Optional[str] = None) -> dict:
    """Inputs of the compressor at a workload's shape: kv and score [B,S,D] (N(0,1), rounded to
    bf16 for bf16 workloads), ape [Wc,D] fp32 (N(0,1)/2), the upstream gradient dpool
    [B,S//ratio,D] fp32 (N(0,1)), and the workload's segment ids."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    dt = cfg.dtype if dtype is None else dtype
    B, S, D = cfg.B, cfg.S, cfg.D
    Wc = ratio * (2 if overlap else 1)
    kv = _normal(rng_for(cfg, "kv"), (B, S, D))
    score = _normal(rng_for(cfg, "cscore"), (B, S, D))
    ape = 0.5 * _normal(rng_for(cfg, "ape"), (Wc, D))
    dpool = _normal(rng_for(cfg, "dout"), (B, S // ratio, D))
    seg = segment_ids(cfg)
    return dict(kv=_round(kv, dt), score=_round(score, dt), ape=torch.from_numpy(ape.astype(np.float32)),
                dpool=torch.from_numpy(dpool), seg=None if seg is None else torch.from_numpy(seg))


def make_inputs(cfg: Config | str, shuffle_pad: bool = False) -> dict:
    """Draw every input of one workload.  Returns host tensors:

    q [B,S,H,D], pool [B,N,D], kwin [B,S,D] (bf16 or fp32); sink [H] fp32;
    seg [B,S] int32 or None; idx [B,S,K] int32; z [B,S,K] fp32 student logits;
    kl_zero_rows: sorted flat row ids whose student logits the caller replaces by
    log(target) (empty unless the workload asks for it); plus the config.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B, S, H, D, N, K = cfg.B, cfg.S, cfg.H, cfg.D, cfg.N, cfg.K
    q = _normal(rng_for(cfg, "q"), (B, S, H, D))
    pool = _normal(rng_for(cfg, "pool"), (B, N, D))
    kwin = _normal(rng_for(cfg, "kwin"), (B, S, D))
    sink = _normal(rng_for(cfg, "sink"), (H,))
    if cfg.sink_hot_heads:
        sink[: cfg.sink_hot_heads] = cfg.sink_hot_value
    if cfg.window_bias_heads:
        # Keys are shared by all heads, so a per-head window bias is carried by a
        # reserved dimension: kwin[...,0] = 1, pool[...,0] = 0 and q[..., h, 0] = a
        # with a*scale ~= bias for the biased heads (a = 181 is exact in bf16).
        a = np.float32(round(cfg.window_bias / cfg.scale))
        kwin[..., 0] = 1.0
        pool[..., 0] = 0.0
        q[..., :, 0] = 0.0
        q[..., : cfg.window_bias_heads, 0] = a
    seg = segment_ids(cfg)
    idx = topk_slots(cfg, rng_for(cfg, "idx"), shuffle_pad=shuffle_pad)
    z = _normal(rng_for(cfg, "logits"), (B, S, K))
    rows = np.zeros(0, dtype=np.int64)
    if cfg.kl_zero_frac > 0:
        n = int(round(cfg.kl_zero_frac * B * S))
        rows = np.sort(rng_for(cfg, "rowpick").choice(B * S, size=n, replace=False)).astype(np.int64)
    return dict(
        cfg=cfg,
        q=_round(q, cfg.dtype),
        pool=_round(pool, cfg.dtype),
        kwin=_round(kwin, cfg.dtype),
        sink=torch.from_numpy(sink),
        seg=None if seg is None else torch.from_numpy(seg),
        idx=torch.from_numpy(idx),
        z=torch.from_numpy(z),
        kl_zero_rows=rows,
    )


def sample_rows(cfg: Config | str, n: int, seed_offset: int = 0) -> np.ndarray:
    """Seeded sorted sample of flat row ids (b*S+t) for sampled parity checks.

    Always includes the first and last rows of every batch so the empty-row head of
    the sequence and its fullest tail are both covered, the rows around t = 4K where a
    row's visible blocks first outnumber its K slots (all blocks, padded with -1, give
    way to a random K of them), and the rows around every segment start."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    total = cfg.B * cfg.S
    rng = np.random.Generator(np.random.PCG64(1000 * cfg.cid + TENSOR_ID["rowpick"] + 100 + seed_offset))
    pick = rng.choice(total, size=min(n, total), replace=False)
    edges = []
    L = cfg.S // max(cfg.segments, 1)
    for b in range(cfg.B):
        edges += [b * cfg.S, b * cfg.S + 1, b * cfg.S + 3, b * cfg.S + 4, (b + 1) * cfg.S - 1]
        for s0 in range(0, cfg.S, L):                       # segment starts
            sat = s0 + COMPRESS_RATIO * cfg.K               # n_v = floor((t_loc+1)/4) first exceeds K
            for t in (s0 - 1, s0, s0 + 3, s0 + 4, sat - 2, sat - 1, sat, sat + 1):
                if 0 <= t < cfg.S:
                    edges.append(b * cfg.S + t)
    return np.unique(np.concatenate([pick, np.array(edges)])).astype(np.int64)
