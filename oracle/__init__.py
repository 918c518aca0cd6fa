"""fp64 CPU oracle for the CSA indexer-distillation path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg
may import this package.  It shares no code with the HIP library: the arithmetic
lives in ``oracle.c`` (plain C, double precision, OpenMP over query rows), loaded
here through ctypes.  Each function restates, in its docstring, the definition it
evaluates; the C source cites the pages for each step.

Parity status: every function here is pinned by the CPU tests (brute force over a
dense masked matrix, closed forms, invariants, finite differences, library special
cases, hand-derived fixtures under ``tests/golden``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_window_lse.argtypes = [_fp, _fp, _fp, _ip, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, _lp, ctypes.c_int64, _dp]
        lib.oracle_target.argtypes = [_fp, _fp, _ip, _fp, _fp, _ip, _dp] + [ctypes.c_int] * 7 + \
                                     [ctypes.c_double, ctypes.c_double, _lp, ctypes.c_int64, _dp]
        lib.oracle_kl.argtypes = [_fp, _fp, _ip] + [ctypes.c_int] * 4 + \
                                 [ctypes.c_double, _lp, ctypes.c_int64, _dp, _dp, _dp]
        lib.oracle_indexer_topk.argtypes = [_fp, _ip] + [ctypes.c_int] * 5 + [_lp, ctypes.c_int64, _ip, _fp]
        lib.oracle_indexer_topk_bwd.argtypes = [_fp, _ip] + [ctypes.c_int] * 4 + [_lp, ctypes.c_int64, _dp]
        lib.oracle_compressor_pool.argtypes = [_fp, _fp, _fp, _ip] + [ctypes.c_int] * 5 + [_dp]
        lib.oracle_compressor_pool_bwd.argtypes = [_fp, _fp, _fp, _ip, _fp] + [ctypes.c_int] * 5 + [_dp, _dp, _dp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def _f32(x):
    if x is None:
        return None, None
    if hasattr(x, "detach"):            # torch tensor (any float dtype; bf16 -> f32 is exact)
        x = x.detach().cpu().float().numpy()
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a, a.ctypes.data_as(_fp)


def _i32(x):
    if x is None:
        return None, None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    a = np.ascontiguousarray(x, dtype=np.int32)
    return a, a.ctypes.data_as(_ip)


def _rows(rows, total):
    if rows is None:
        return None, None, total
    a = np.ascontiguousarray(rows, dtype=np.int64)
    assert a.ndim == 1 and (a.size == 0 or (a.min() >= 0 and a.max() < total))
    return a, a.ctypes.data_as(_lp), a.size


def window_lse(q, kwin, sink, seg, W: int, scale: float, rows=None) -> np.ndarray:
    """nc_lse[r, h] = log( sum_{j in win(t)} exp(scale <q[b,t,h], kwin[b,j]>) + exp(sink[h]) )

    win(t) = { j : t-W+1 <= j <= t, j >= 0, seg[b,j] == seg[b,t] }; sink None drops
    its term.  Returns float64 [nrows, H] (nrows = B*S when rows is None)."""
    qa, qp = _f32(q)
    B, S, H, D = qa.shape
    ka, kp = _f32(kwin)
    sa, sp = _f32(sink)
    ga, gp = _i32(seg)
    ra, rp, n = _rows(rows, B * S)
    out = np.empty((n, H), dtype=np.float64)
    _load().oracle_window_lse(qp, kp, sp, gp, B, S, H, D, int(W), float(scale), rp, n,
                              out.ctypes.data_as(_dp))
    return out


def target(q, pool, idx, kwin=None, sink=None, seg=None, nc_lse=None, W: int = 0,
           scale: float = 1.0, floor: float = 0.0, rows=None) -> np.ndarray:
    """KL target T[r, k], the joint softmax written out the long way.

    Per head the logit list is [window logits] ++ [sink] ++ [compressed logits of the
    valid slots] (or [nc_lse[r,h]] ++ [compressed] when nc_lse, shaped [nrows,H], is
    given); T_k = sum_h exp(c_hk - LSE(list)) / max(sum over slots, floor), 0 at
    invalid slots; floor <= 0 means float32 tiny.  With kwin, sink and nc_lse all None
    the list is the compressed part alone (legacy per-branch target).
    Returns float64 [nrows, K]."""
    qa, qp = _f32(q)
    B, S, H, D = qa.shape
    pa, pp = _f32(pool)
    N = pa.shape[1]
    ia, ip = _i32(idx)
    K = ia.shape[2]
    ka, kp = _f32(kwin)
    sa, sp = _f32(sink)
    ga, gp = _i32(seg)
    ra, rp, n = _rows(rows, B * S)
    nca = None
    ncp = None
    if nc_lse is not None:
        nca = np.ascontiguousarray(nc_lse, dtype=np.float64).reshape(n, H)
        ncp = nca.ctypes.data_as(_dp)
    out = np.empty((n, K), dtype=np.float64)
    _load().oracle_target(qp, pp, ip, kp, sp, gp, ncp, B, S, H, D, N, K, int(W),
                          float(scale), float(floor), rp, n, out.ctypes.data_as(_dp))
    return out


def kl(T, z, idx, N: int, grad_scale: float = 1.0, rows=None, want_grad: bool = True):
    """Per-row KL(T || softmax_V(z)) and its gradient; returns (kl [nrows], dz [nrows,K]
    or None, stats [2] = (sum of KL over non-empty selected rows, their count)).

    T and z are read as float32 [B,S,K] (or [nrows_total, K] with B=1)."""
    Ta, Tp = _f32(T)
    za, zp = _f32(z)
    ia, ip = _i32(idx)
    K = ia.shape[-1]
    BS = ia.size // K
    B, S = (ia.shape[0], ia.shape[1]) if ia.ndim == 3 else (1, BS)
    assert Ta.size == ia.size and za.size == ia.size
    ra, rp, n = _rows(rows, BS)
    klo = np.empty(n, dtype=np.float64)
    dz = np.empty((n, K), dtype=np.float64) if want_grad else None
    st = np.zeros(2, dtype=np.float64)
    _load().oracle_kl(Tp, zp, ip, B, S, K, int(N), float(grad_scale), rp, n,
                      klo.ctypes.data_as(_dp), dz.ctypes.data_as(_dp) if want_grad else None,
                      st.ctypes.data_as(_dp))
    return klo, dz, st


def indexer_topk(scores, seg, K: int, ratio: int, rows=None):
    """Masked top-k selection of the indexer.  scores [B,S,N] (read as float32), seg [B,S]
    or None.  Block n is visible to token t iff it is complete at t (ratio*n + ratio - 1
    <= t) and all its tokens share t's segment id.  The K visible blocks with the largest
    scores are kept (equal scores: smaller index first; NaN ranks lowest) and returned in
    ascending block order, then -1.  Returns (idx int32 [nrows,K], values float32 [nrows,K],
    -inf at -1 slots)."""
    sa, sp = _f32(scores)
    B, S, N = sa.shape
    ga, gp = _i32(seg)
    ra, rp, n = _rows(rows, B * S)
    idx = np.empty((n, K), dtype=np.int32)
    val = np.empty((n, K), dtype=np.float32)
    _load().oracle_indexer_topk(sp, gp, B, S, N, int(K), int(ratio), rp, n,
                                idx.ctypes.data_as(_ip), val.ctypes.data_as(_fp))
    return idx, val


def indexer_topk_bwd(dval, idx, N: int, rows=None):
    """Adjoint of the gather values = scores[idx]: dscores[r, n] = sum of dval over the
    valid slots holding n (slot order), 0 elsewhere.  dval, idx [B,S,K].  Returns float64
    [nrows, N]."""
    da, dp = _f32(dval)
    ia, ip = _i32(idx)
    B, S, K = ia.shape
    ra, rp, n = _rows(rows, B * S)
    out = np.empty((n, N), dtype=np.float64)
    _load().oracle_indexer_topk_bwd(dp, ip, B, S, int(N), K, rp, n, out.ctypes.data_as(_dp))
    return out


def compressor_pool(kv, score, ape, seg, ratio: int, overlap: bool):
    """pool[b,n,d] = sum_i softmax_i(score[b,j_i,d] + ape[i,d]) kv[b,j_i,d] over the present
    positions of entry n's window: tokens ratio*n .. ratio*n+ratio-1 (overlap False), or
    ratio*(n-1) .. ratio*n+ratio-1 (overlap True; positions before token 0 absent); a
    position whose token has another segment than the entry's last token is absent.
    kv, score [B,S,D]; ape [Wc,D]; seg [B,S] or None.  Returns float64 [B, S//ratio, D]."""
    ka, kp = _f32(kv)
    B, S, D = ka.shape
    sa, sp = _f32(score)
    aa, ap = _f32(ape)
    ga, gp = _i32(seg)
    Wc = ratio * (2 if overlap else 1)
    assert aa.shape == (Wc, D) and sa.shape == ka.shape
    out = np.empty((B, S // ratio, D), dtype=np.float64)
    _load().oracle_compressor_pool(kp, sp, ap, gp, B, S, D, int(ratio), int(bool(overlap)),
                                   out.ctypes.data_as(_dp))
    return out


def compressor_pool_bwd(kv, score, ape, seg, dpool, ratio: int, overlap: bool):
    """Analytic backward of compressor_pool for dpool [B,N,D]: returns float64 (dkv [B,S,D],
    dscore [B,S,D], dape [Wc,D])."""
    ka, kp = _f32(kv)
    B, S, D = ka.shape
    sa, sp = _f32(score)
    aa, ap = _f32(ape)
    ga, gp = _i32(seg)
    da, dp = _f32(dpool)
    Wc = ratio * (2 if overlap else 1)
    assert da.shape == (B, S // ratio, D)
    dkv = np.empty((B, S, D), dtype=np.float64)
    dsc = np.empty((B, S, D), dtype=np.float64)
    dape = np.empty((Wc, D), dtype=np.float64)
    _load().oracle_compressor_pool_bwd(kp, sp, ap, gp, dp, B, S, D, int(ratio), int(bool(overlap)),
                                       dkv.ctypes.data_as(_dp), dsc.ctypes.data_as(_dp), dape.ctypes.data_as(_dp))
    return dkv, dsc, dape
