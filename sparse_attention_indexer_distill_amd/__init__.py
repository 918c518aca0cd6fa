"""MI355X (gfx950) CSA indexer-distillation path.

A thin ctypes binding over ``libsparse_distill.so`` (C ABI: ``include/sparse_distill.h``).
The functions carry the same names as the C entry points and only marshal arguments:
they check devices, dtypes and shapes, make tensors contiguous, allocate outputs with
torch, and pass raw device pointers plus torch's current HIP stream.  Every step of the
computation runs in the library's kernels; there is no fallback.  If the library is
not built, every call raises.

Semantics (DeepSeek-V4 CSA layer; Primus PR "perf(deepseek-v4): fuse and enable the
indexer distillation loss" and MaxText PR "Add Indexer Loss [Deepseek v4]"):
  window_lse          log-mass of each head's sliding-window keys plus its sink
  distill_target      joint-softmax KL target over each token's top-k pool rows
  distill_kl_fwd_bwd  KL(target || softmax(indexer logits)) and its gradient
"""
from __future__ import annotations

import ctypes
import functools
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["window_lse", "distill_target", "distill_target_fused", "distill_kl_fwd_bwd", "distill_kl_workspace_bytes",
           "distill_kl_fwd_bwd_noalloc", "indexer_topk", "indexer_topk_bwd", "compressor_pool", "compressor_pool_bwd",
           "compressor_pool_bwd_workspace_bytes", "csa_distill_layer", "library_path", "load_library", "SD_BF16", "SD_F32"]

SD_OK, SD_ERR_NULL_ARG, SD_ERR_BAD_SHAPE, SD_ERR_UNSUPPORTED, SD_ERR_DTYPE, SD_ERR_HIP = range(6)
SD_BF16, SD_F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsparse_distill.so")
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsparse_distill.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m sparse_attention_indexer_distill_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.window_lse.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]
    lib.window_lse.restype = _i
    lib.distill_target.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _i, _vp, _vp]
    lib.distill_target.restype = _i
    lib.distill_target_fused.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _f, _i, _vp,
                                         _vp, _vp]
    lib.distill_target_fused.restype = _i
    lib.distill_kl_workspace_bytes.argtypes = [_i, _i, _i]
    lib.distill_kl_workspace_bytes.restype = ctypes.c_size_t
    lib.distill_kl_fwd_bwd.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.distill_kl_fwd_bwd.restype = _i
    lib.distill_kl_fwd_bwd_noalloc.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp]
    lib.distill_kl_fwd_bwd_noalloc.restype = _i
    lib.indexer_topk.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.indexer_topk.restype = _i
    lib.indexer_topk_bwd.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp, _vp]
    lib.indexer_topk_bwd.restype = _i
    lib.compressor_pool.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp]
    lib.compressor_pool.restype = _i
    lib.compressor_pool_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    lib.compressor_pool_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.compressor_pool_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
    lib.compressor_pool_bwd.restype = _i
    lib.sd_status_string.argtypes = [_i]
    lib.sd_status_string.restype = ctypes.c_char_p
    lib.sd_last_error.argtypes = []
    lib.sd_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status == SD_OK:
        return
    lib = load_library()
    msg = f"{what}: {lib.sd_status_string(status).decode()}: {lib.sd_last_error().decode()}"
    if status in (SD_ERR_NULL_ARG, SD_ERR_BAD_SHAPE, SD_ERR_DTYPE):
        raise ValueError(msg)
    if status == SD_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SD_BF16
    if t.dtype == torch.float32:
        return SD_F32
    raise ValueError(f"q/kwin/pool must be bfloat16 or float32, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, device: torch.device) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t if t.is_contiguous() else t.contiguous()


def _out(t: torch.Tensor, name: str, shape, device: torch.device) -> torch.Tensor:
    """A caller-provided output buffer: float32, contiguous, of the given shape, on device
    (the kernels write it in place, so it is never copied)."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor")
    return t


def _workspace(t: Optional[torch.Tensor], need: int, device: torch.device) -> torch.Tensor:
    """Caller-provided scratch (any dtype, contiguous, on device, at least need bytes), or a new one."""
    if t is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous GPU tensor on {device}")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace holds {t.numel() * t.element_size()} bytes, {need} needed")
    return t


def _slots(idx: torch.Tensor, N: int, device: torch.device) -> torch.Tensor:
    """Top-k slots as int32 on device.  Wider integer slots are mapped to -1 outside [0, N)
    before the cast (asynchronously, on the device), so no value can wrap into a valid row."""
    if idx.dtype == torch.int32:
        return _dev(idx, "idx", device)
    if idx.dtype not in (torch.int64, torch.int16, torch.uint8, torch.int8):
        raise ValueError(f"idx must be an integer tensor, got {idx.dtype}")
    idx = _dev(idx, "idx", device)
    return torch.where((idx >= 0) & (idx < N), idx, torch.full_like(idx, -1)).to(torch.int32)


def _stream(device: torch.device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _on_stream(fn):
    """Run a wrapper with ``stream`` (when given) as torch's current stream, so that every
    temporary it makes (contiguous copies, dtype casts, slot remaps, default outputs and
    workspaces) is allocated and written on the stream the kernels run on.  The caching
    allocator then reuses those blocks only in that stream's order, after the kernels that
    read them.  Inputs produced on another stream are the caller's to order, as for any
    torch op run under a stream context."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


@_on_stream
def window_lse(q: torch.Tensor, kwin: torch.Tensor, sink: Optional[torch.Tensor] = None,
               seg: Optional[torch.Tensor] = None, *, W: int, scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """nc_lse [B,S,H] fp32: log-mass of the W window keys ending at t (same segment) plus sink."""
    lib = load_library()
    dev = q.device
    q = _dev(q, "q", dev)
    kwin = _dev(kwin, "kwin", dev)
    B, S, H, D = q.shape
    if kwin.shape != (B, S, D) or kwin.dtype != q.dtype:
        raise ValueError(f"kwin must be [{B},{S},{D}] {q.dtype}, got {tuple(kwin.shape)} {kwin.dtype}")
    if sink is not None:
        sink = _dev(sink.detach().to(torch.float32), "sink", dev)
        if sink.numel() != H:
            raise ValueError(f"sink must hold {H} head values, got {sink.numel()}")
    if seg is not None:
        seg = _dev(seg.to(torch.int32), "seg", dev)
        if seg.shape != (B, S):
            raise ValueError(f"seg must be [{B},{S}]")
    if out is None:
        out = torch.empty((B, S, H), dtype=torch.float32, device=dev)
    else:
        _out(out, "out", (B, S, H), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.window_lse(_ptr(q), _ptr(kwin), _ptr(sink), _ptr(seg), B, S, H, D, int(W), scale,
                        _dtype_code(q), _ptr(out), _stream(dev, stream))
    _check(st, "window_lse")
    return out


@_on_stream
def distill_target(q: torch.Tensor, pool: torch.Tensor, idx: torch.Tensor,
                   nc_lse: Optional[torch.Tensor] = None, *, scale: Optional[float] = None,
                   l1_floor: float = 0.0, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """KL target [B,S,K] fp32 (joint softmax over window+sink mass nc_lse and the selected
    pool rows; nc_lse None = legacy per-branch target).  l1_floor <= 0 means float32 tiny."""
    lib = load_library()
    dev = q.device
    q = _dev(q, "q", dev)
    pool = _dev(pool, "pool", dev)
    B, S, H, D = q.shape
    if pool.dim() != 3 or pool.shape[0] != B or pool.shape[2] != D or pool.dtype != q.dtype:
        raise ValueError(f"pool must be [{B},N,{D}] {q.dtype}, got {tuple(pool.shape)} {pool.dtype}")
    N = pool.shape[1]
    if idx.dim() != 3 or idx.shape[:2] != (B, S):
        raise ValueError(f"idx must be [{B},{S},K]")
    idx = _slots(idx, N, dev)
    K = idx.shape[2]
    if nc_lse is not None:
        nc_lse = _dev(nc_lse.detach().to(torch.float32), "nc_lse", dev)
        if nc_lse.shape != (B, S, H):
            raise ValueError(f"nc_lse must be [{B},{S},{H}]")
    if out is None:
        out = torch.empty((B, S, K), dtype=torch.float32, device=dev)
    else:
        _out(out, "out", (B, S, K), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.distill_target(_ptr(q), _ptr(pool), _ptr(idx), _ptr(nc_lse), B, S, H, D, N, K, scale,
                            float(l1_floor), _dtype_code(q), _ptr(out), _stream(dev, stream))
    _check(st, "distill_target")
    return out


@_on_stream
def distill_target_fused(q: torch.Tensor, kwin: torch.Tensor, pool: torch.Tensor, idx: torch.Tensor,
                         sink: Optional[torch.Tensor] = None, seg: Optional[torch.Tensor] = None, *, W: int,
                         scale: Optional[float] = None, l1_floor: float = 0.0, want_nc: bool = False,
                         out: Optional[torch.Tensor] = None, nc_out: Optional[torch.Tensor] = None,
                         stream=None):
    """KL target [B,S,K] fp32 with the window part computed in the same pass (one read of q).
    Returns target, or (target, nc_lse) when want_nc or nc_out is given."""
    lib = load_library()
    dev = q.device
    q = _dev(q, "q", dev)
    kwin = _dev(kwin, "kwin", dev)
    pool = _dev(pool, "pool", dev)
    B, S, H, D = q.shape
    if kwin.shape != (B, S, D) or kwin.dtype != q.dtype:
        raise ValueError(f"kwin must be [{B},{S},{D}] {q.dtype}, got {tuple(kwin.shape)} {kwin.dtype}")
    if pool.dim() != 3 or pool.shape[0] != B or pool.shape[2] != D or pool.dtype != q.dtype:
        raise ValueError(f"pool must be [{B},N,{D}] {q.dtype}, got {tuple(pool.shape)} {pool.dtype}")
    N = pool.shape[1]
    if idx.dim() != 3 or idx.shape[:2] != (B, S):
        raise ValueError(f"idx must be [{B},{S},K]")
    idx = _slots(idx, N, dev)
    K = idx.shape[2]
    if sink is not None:
        sink = _dev(sink.detach().to(torch.float32), "sink", dev)
        if sink.numel() != H:
            raise ValueError(f"sink must hold {H} head values, got {sink.numel()}")
    if seg is not None:
        seg = _dev(seg.to(torch.int32), "seg", dev)
        if seg.shape != (B, S):
            raise ValueError(f"seg must be [{B},{S}]")
    if out is None:
        out = torch.empty((B, S, K), dtype=torch.float32, device=dev)
    else:
        _out(out, "out", (B, S, K), dev)
    if nc_out is None and want_nc:
        nc_out = torch.empty((B, S, H), dtype=torch.float32, device=dev)
    if nc_out is not None:
        _out(nc_out, "nc_out", (B, S, H), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.distill_target_fused(_ptr(q), _ptr(kwin), _ptr(sink), _ptr(seg), _ptr(pool), _ptr(idx), B, S, H, D, N,
                                  K, int(W), scale, float(l1_floor), _dtype_code(q), _ptr(out), _ptr(nc_out),
                                  _stream(dev, stream))
    _check(st, "distill_target_fused")
    return (out, nc_out) if nc_out is not None else out


def distill_kl_workspace_bytes(B: int, S: int, K: int) -> int:
    return int(load_library().distill_kl_workspace_bytes(B, S, K))


@_on_stream
def distill_kl_fwd_bwd(target: torch.Tensor, logits: torch.Tensor, idx: torch.Tensor, N: int, *,
                       grad_scale: float = 1.0, want_grad: bool = True,
                       kl_rows: Optional[torch.Tensor] = None, dlogits: Optional[torch.Tensor] = None,
                       stats: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """Per-row KL(target || softmax over valid slots of logits), its gradient scaled by
    grad_scale (or None when want_grad is False), and stats = (sum of KL over non-empty
    rows, number of non-empty rows)."""
    lib = load_library()
    dev = target.device
    target = _dev(target, "target", dev)
    logits = _dev(logits, "logits", dev)
    if target.dim() != 3 or logits.shape != target.shape or idx.shape != target.shape:
        raise ValueError("target, logits and idx must share one [B,S,K] shape")
    if target.dtype != torch.float32 or logits.dtype != torch.float32:
        raise ValueError("target and logits must be float32")
    idx = _slots(idx, int(N), dev)
    B, S, K = target.shape
    kl_rows = torch.empty((B, S), dtype=torch.float32, device=dev) if kl_rows is None else \
        _out(kl_rows, "kl_rows", (B, S), dev)
    if not want_grad:
        dlogits = None
    elif dlogits is None:
        dlogits = torch.empty((B, S, K), dtype=torch.float32, device=dev)
    else:
        _out(dlogits, "dlogits", (B, S, K), dev)
    stats = torch.empty(2, dtype=torch.float32, device=dev) if stats is None else _out(stats, "stats", (2,), dev)
    workspace = _workspace(workspace, distill_kl_workspace_bytes(B, S, K), dev)
    st = lib.distill_kl_fwd_bwd(_ptr(target), _ptr(logits), _ptr(idx), B, S, K, int(N), float(grad_scale),
                                _ptr(kl_rows), _ptr(dlogits), _ptr(stats), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(st, "distill_kl_fwd_bwd")
    return kl_rows, dlogits, stats


@_on_stream
def distill_kl_fwd_bwd_noalloc(target: torch.Tensor, logits: torch.Tensor, idx: torch.Tensor, N: int, *,
                               grad_scale: float = 1.0, want_grad: bool = True,
                               kl_rows: Optional[torch.Tensor] = None, dlogits: Optional[torch.Tensor] = None,
                               stats: Optional[torch.Tensor] = None,
                               stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """distill_kl_fwd_bwd without a workspace: the library keeps its partial sums in a fixed
    per-GPU array and the C call allocates nothing (B*S <= 2^21; calls overlapping on one
    GPU race).  Outputs not passed in are allocated here, by torch."""
    lib = load_library()
    dev = target.device
    target = _dev(target, "target", dev)
    logits = _dev(logits, "logits", dev)
    if target.dim() != 3 or logits.shape != target.shape or idx.shape != target.shape:
        raise ValueError("target, logits and idx must share one [B,S,K] shape")
    if target.dtype != torch.float32 or logits.dtype != torch.float32:
        raise ValueError("target and logits must be float32")
    idx = _slots(idx, int(N), dev)
    B, S, K = target.shape
    kl_rows = torch.empty((B, S), dtype=torch.float32, device=dev) if kl_rows is None else \
        _out(kl_rows, "kl_rows", (B, S), dev)
    if not want_grad:
        dlogits = None
    elif dlogits is None:
        dlogits = torch.empty((B, S, K), dtype=torch.float32, device=dev)
    else:
        _out(dlogits, "dlogits", (B, S, K), dev)
    stats = torch.empty(2, dtype=torch.float32, device=dev) if stats is None else _out(stats, "stats", (2,), dev)
    st = lib.distill_kl_fwd_bwd_noalloc(_ptr(target), _ptr(logits), _ptr(idx), B, S, K, int(N), float(grad_scale),
                                        _ptr(kl_rows), _ptr(dlogits), _ptr(stats), _stream(dev, stream))
    _check(st, "distill_kl_fwd_bwd_noalloc")
    return kl_rows, dlogits, stats


@_on_stream
def indexer_topk(scores: torch.Tensor, seg: Optional[torch.Tensor] = None, *, K: int, ratio: int = 4,
                 want_values: bool = True, out_idx: Optional[torch.Tensor] = None,
                 out_values: Optional[torch.Tensor] = None, stream=None):
    """The indexer's masked top-k: idx [B,S,K] int32 (visible blocks with the largest scores,
    ascending block order, -1 after) and values [B,S,K] fp32 (their scores, -inf at -1), or
    (idx, None) when want_values is False.  scores [B,S,N] fp32; seg [B,S] or None."""
    lib = load_library()
    dev = scores.device
    scores = _dev(scores, "scores", dev)
    if scores.dim() != 3 or scores.dtype != torch.float32:
        raise ValueError("scores must be a float32 [B,S,N] tensor")
    B, S, N = scores.shape
    if seg is not None:
        seg = _dev(seg.to(torch.int32), "seg", dev)
        if seg.shape != (B, S):
            raise ValueError(f"seg must be [{B},{S}]")
    if out_idx is None:
        out_idx = torch.empty((B, S, int(K)), dtype=torch.int32, device=dev)
    elif (not out_idx.is_cuda or out_idx.device != dev or tuple(out_idx.shape) != (B, S, int(K))
          or out_idx.dtype != torch.int32 or not out_idx.is_contiguous()):
        raise ValueError(f"out_idx must be a contiguous int32 [{B},{S},{K}] tensor on {dev}")
    if not want_values:
        out_values = None
    elif out_values is None:
        out_values = torch.empty((B, S, int(K)), dtype=torch.float32, device=dev)
    else:
        _out(out_values, "out_values", (B, S, int(K)), dev)
    st = lib.indexer_topk(_ptr(scores), _ptr(seg), B, S, N, int(K), int(ratio), _ptr(out_idx), _ptr(out_values),
                          _stream(dev, stream))
    _check(st, "indexer_topk")
    return out_idx, out_values


@_on_stream
def indexer_topk_bwd(dvalues: torch.Tensor, idx: torch.Tensor, N: int, *, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Gradient of indexer_topk's values w.r.t. the scores: dscores [B,S,N] fp32, each block
    receiving the sum of its slots' dvalues (0 elsewhere)."""
    lib = load_library()
    dev = dvalues.device
    dvalues = _dev(dvalues, "dvalues", dev)
    if dvalues.dim() != 3 or dvalues.dtype != torch.float32 or idx.shape != dvalues.shape:
        raise ValueError("dvalues must be float32 [B,S,K] and idx the same shape")
    idx = _slots(idx, int(N), dev)
    B, S, K = dvalues.shape
    if out is None:
        out = torch.empty((B, S, int(N)), dtype=torch.float32, device=dev)
    else:
        _out(out, "out", (B, S, int(N)), dev)
    st = lib.indexer_topk_bwd(_ptr(dvalues), _ptr(idx), B, S, int(N), K, _ptr(out), _stream(dev, stream))
    _check(st, "indexer_topk_bwd")
    return out


def _compressor_inputs(kv, score, ape, seg, ratio, overlap):
    dev = kv.device
    kv = _dev(kv, "kv", dev)
    score = _dev(score, "score", dev)
    if kv.dim() != 3 or score.shape != kv.shape or score.dtype != kv.dtype:
        raise ValueError("kv and score must share one [B,S,D] shape and dtype")
    B, S, D = kv.shape
    Wc = int(ratio) * (2 if overlap else 1)
    ape = _dev(ape.detach().to(torch.float32), "ape", dev)
    if tuple(ape.shape) != (Wc, D):
        raise ValueError(f"ape must be [{Wc},{D}] (window positions x channels), got {tuple(ape.shape)}")
    if seg is not None:
        seg = _dev(seg.to(torch.int32), "seg", dev)
        if seg.shape != (B, S):
            raise ValueError(f"seg must be [{B},{S}]")
    return dev, kv, score, ape, seg, B, S, D


@_on_stream
def compressor_pool(kv: torch.Tensor, score: torch.Tensor, ape: torch.Tensor, seg: Optional[torch.Tensor] = None, *,
                    ratio: int, overlap: bool, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pool [B, S//ratio, D] fp32: per channel, the softmax over each entry's window of
    score + ape, weighting kv (windows of ratio tokens; with overlap, two blocks)."""
    lib = load_library()
    dev, kv, score, ape, seg, B, S, D = _compressor_inputs(kv, score, ape, seg, ratio, overlap)
    N = S // int(ratio)
    if out is None:
        out = torch.empty((B, N, D), dtype=torch.float32, device=dev)
    else:
        _out(out, "out", (B, N, D), dev)
    st = lib.compressor_pool(_ptr(kv), _ptr(score), _ptr(ape), _ptr(seg), B, S, D, int(ratio), int(bool(overlap)),
                             _dtype_code(kv), _ptr(out), _stream(dev, stream))
    _check(st, "compressor_pool")
    return out


def compressor_pool_bwd_workspace_bytes(B: int, S: int, D: int, ratio: int, overlap: bool) -> int:
    return int(load_library().compressor_pool_bwd_workspace_bytes(B, S, D, int(ratio), int(bool(overlap))))


@_on_stream
def compressor_pool_bwd(kv: torch.Tensor, score: torch.Tensor, ape: torch.Tensor, dpool: torch.Tensor,
                        seg: Optional[torch.Tensor] = None, *, ratio: int, overlap: bool,
                        dkv: Optional[torch.Tensor] = None, dscore: Optional[torch.Tensor] = None,
                        dape: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None):
    """Analytic backward of compressor_pool: (dkv [B,S,D], dscore [B,S,D], dape [Wc,D]), fp32."""
    lib = load_library()
    dev, kv, score, ape, seg, B, S, D = _compressor_inputs(kv, score, ape, seg, ratio, overlap)
    N = S // int(ratio)
    Wc = ape.shape[0]
    dpool = _dev(dpool, "dpool", dev)
    if tuple(dpool.shape) != (B, N, D) or dpool.dtype != torch.float32:
        raise ValueError(f"dpool must be float32 [{B},{N},{D}]")
    dkv = torch.empty((B, S, D), dtype=torch.float32, device=dev) if dkv is None else _out(dkv, "dkv", (B, S, D), dev)
    dscore = torch.empty((B, S, D), dtype=torch.float32, device=dev) if dscore is None else \
        _out(dscore, "dscore", (B, S, D), dev)
    dape = torch.empty((Wc, D), dtype=torch.float32, device=dev) if dape is None else _out(dape, "dape", (Wc, D), dev)
    workspace = _workspace(workspace, compressor_pool_bwd_workspace_bytes(B, S, D, ratio, overlap), dev)
    st = lib.compressor_pool_bwd(_ptr(kv), _ptr(score), _ptr(ape), _ptr(seg), _ptr(dpool), B, S, D, int(ratio),
                                 int(bool(overlap)), _dtype_code(kv), _ptr(dkv), _ptr(dscore), _ptr(dape),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(st, "compressor_pool_bwd")
    return dkv, dscore, dape


@_on_stream
def csa_distill_layer(q, kwin, pool, idx, logits, sink=None, seg=None, *, W: int,
                      scale: Optional[float] = None, grad_scale: float = 1.0, want_grad: bool = True,
                      fused: bool = False, bufs: Optional[dict] = None, stream=None):
    """One CSA layer's distillation step: window_lse -> distill_target -> distill_kl_fwd_bwd, or
    with fused=True distill_target_fused -> distill_kl_fwd_bwd (same outputs, one read of q).
    ``bufs`` may hold preallocated outputs (nc_lse, target, kl_rows, dlogits, stats, workspace).
    Returns a dict with every output."""
    bufs = {} if bufs is None else bufs
    if fused:
        T, nc = distill_target_fused(q, kwin, pool, idx, sink, seg, W=W, scale=scale, want_nc=True,
                                     out=bufs.get("target"), nc_out=bufs.get("nc_lse"), stream=stream)
    else:
        nc = window_lse(q, kwin, sink, seg, W=W, scale=scale, out=bufs.get("nc_lse"), stream=stream)
        T = distill_target(q, pool, idx, nc, scale=scale, out=bufs.get("target"), stream=stream)
    kl, dz, st = distill_kl_fwd_bwd(T, logits, idx, pool.shape[1], grad_scale=grad_scale, want_grad=want_grad,
                                    kl_rows=bufs.get("kl_rows"), dlogits=bufs.get("dlogits"),
                                    stats=bufs.get("stats"), workspace=bufs.get("workspace"), stream=stream)
    return dict(nc_lse=nc, target=T, kl_rows=kl, dlogits=dz, stats=st)
