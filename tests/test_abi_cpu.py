"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host with the documented status codes.

Every call below is invalid on purpose, so the library returns before any HIP call;
no kernel is ever launched from this file (the pointers are placeholders)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_indexer_distill_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_distill.h")
FAKE = ctypes.c_void_p(0x1000)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sd.library_path()):
        from sparse_attention_indexer_distill_amd import build
        build.build()
    return sd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("window_lse", "distill_target", "distill_target_fused", "distill_kl_fwd_bwd",
              "distill_kl_workspace_bytes", "distill_kl_fwd_bwd_noalloc", "indexer_topk", "indexer_topk_bwd",
              "compressor_pool", "compressor_pool_bwd", "compressor_pool_bwd_workspace_bytes",
              "sd_status_string", "sd_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sd.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in exported, f"{n} not exported"
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert lib.sd_status_string(0) == b"SD_OK"
    assert lib.sd_status_string(3) == b"SD_ERR_UNSUPPORTED"
    assert lib.sd_status_string(99) == b"SD_ERR_UNKNOWN"


def _wl(lib, q=FAKE, k=FAKE, out=FAKE, B=1, S=8, H=4, D=32, W=4, scale=0.1, dtype=0):
    return lib.window_lse(q, k, None, None, B, S, H, D, W, scale, dtype, out, None)


def test_window_lse_rejections(lib):
    assert _wl(lib, q=None) == sd.SD_ERR_NULL_ARG
    assert b"required" in lib.sd_last_error()
    assert _wl(lib, out=None) == sd.SD_ERR_NULL_ARG
    assert _wl(lib, B=0) == sd.SD_ERR_BAD_SHAPE
    assert _wl(lib, S=-1) == sd.SD_ERR_BAD_SHAPE
    assert _wl(lib, W=0) == sd.SD_ERR_BAD_SHAPE
    assert _wl(lib, scale=float("inf")) == sd.SD_ERR_BAD_SHAPE
    assert _wl(lib, dtype=7) == sd.SD_ERR_DTYPE
    assert _wl(lib, D=48) == sd.SD_ERR_UNSUPPORTED
    assert _wl(lib, D=544) == sd.SD_ERR_UNSUPPORTED
    assert _wl(lib, H=65) == sd.SD_ERR_UNSUPPORTED
    assert _wl(lib, W=129) == sd.SD_ERR_UNSUPPORTED
    assert b"W=129" in lib.sd_last_error()
    # one batch row of window keys must stay below 2^31 bytes (32-bit buffer offsets)
    assert _wl(lib, S=1 << 21, D=512) == sd.SD_ERR_UNSUPPORTED            # exactly 2^31 bytes of bf16
    assert b"2^31" in lib.sd_last_error()
    assert _wl(lib, S=1 << 20, D=512, dtype=1) == sd.SD_ERR_UNSUPPORTED   # fp32
    # a dispatch counts at most 2^32 - 1 work-items: 512 lanes per two tokens
    assert _wl(lib, S=(1 << 24) - 1, D=32) == sd.SD_ERR_UNSUPPORTED       # kwin row 2^30 bytes: fine
    assert b"2^32 - 1" in lib.sd_last_error()


def _tg(lib, q=FAKE, pool=FAKE, idx=FAKE, out=FAKE, B=1, S=8, H=4, D=32, N=2, K=4, scale=0.1, floor=0.0, dtype=0):
    return lib.distill_target(q, pool, idx, None, B, S, H, D, N, K, scale, floor, dtype, out, None)


def test_distill_target_rejections(lib):
    assert _tg(lib, pool=None) == sd.SD_ERR_NULL_ARG
    assert _tg(lib, idx=None) == sd.SD_ERR_NULL_ARG
    assert _tg(lib, out=None) == sd.SD_ERR_NULL_ARG
    assert _tg(lib, N=0) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, K=0) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, H=0) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, floor=float("nan")) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, scale=0.0) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, scale=-0.1) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, scale=float("nan")) == sd.SD_ERR_BAD_SHAPE
    assert _tg(lib, dtype=-1) == sd.SD_ERR_DTYPE
    assert _tg(lib, K=1025) == sd.SD_ERR_UNSUPPORTED
    assert _tg(lib, D=16) == sd.SD_ERR_UNSUPPORTED
    assert _tg(lib, H=128) == sd.SD_ERR_UNSUPPORTED
    assert _tg(lib, N=1 << 21, D=512) == sd.SD_ERR_UNSUPPORTED           # pool row of 2^31 bytes
    assert b"pool" in lib.sd_last_error()
    # row indices are multiplied in 24 bits: at most 2^24 pool rows, even where the bytes fit
    assert _tg(lib, N=(1 << 24) + 1, D=32) == sd.SD_ERR_UNSUPPORTED
    assert b"2^24 rows" in lib.sd_last_error()
    assert _tf(lib, N=(1 << 24) + 1, D=32) == sd.SD_ERR_UNSUPPORTED
    # up to 1024 lanes per token: B*S must stay below 2^22
    assert _tg(lib, B=1, S=1 << 22, H=1) == sd.SD_ERR_UNSUPPORTED
    assert b"2^22" in lib.sd_last_error()
    assert _tg(lib, B=4, S=1 << 20, H=1) == sd.SD_ERR_UNSUPPORTED


def _tf(lib, q=FAKE, k=FAKE, pool=FAKE, idx=FAKE, out=FAKE, B=1, S=8, H=4, D=32, N=2, K=4, W=4, scale=0.1,
        floor=0.0, dtype=0):
    lib.distill_target_fused.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 7 + [ctypes.c_float] * 2 + \
        [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return lib.distill_target_fused(q, k, None, None, pool, idx, B, S, H, D, N, K, W, scale, floor, dtype, out,
                                    None, None)


def test_distill_target_fused_rejections(lib):
    assert _tf(lib, q=None) == sd.SD_ERR_NULL_ARG
    assert _tf(lib, k=None) == sd.SD_ERR_NULL_ARG
    assert _tf(lib, pool=None) == sd.SD_ERR_NULL_ARG
    assert _tf(lib, idx=None) == sd.SD_ERR_NULL_ARG
    assert _tf(lib, out=None) == sd.SD_ERR_NULL_ARG
    assert _tf(lib, W=0) == sd.SD_ERR_BAD_SHAPE
    assert _tf(lib, N=0) == sd.SD_ERR_BAD_SHAPE
    assert _tf(lib, scale=0.0) == sd.SD_ERR_BAD_SHAPE
    assert _tf(lib, floor=float("nan")) == sd.SD_ERR_BAD_SHAPE
    assert _tf(lib, dtype=7) == sd.SD_ERR_DTYPE
    assert _tf(lib, W=129) == sd.SD_ERR_UNSUPPORTED
    assert _tf(lib, K=1025) == sd.SD_ERR_UNSUPPORTED
    assert _tf(lib, D=48) == sd.SD_ERR_UNSUPPORTED
    assert b"head dim" in lib.sd_last_error()
    assert _tf(lib, N=1 << 21, D=512) == sd.SD_ERR_UNSUPPORTED
    assert b"pool" in lib.sd_last_error()
    assert _tf(lib, S=1 << 21, D=512) == sd.SD_ERR_UNSUPPORTED
    assert b"kwin" in lib.sd_last_error()
    assert _tf(lib, B=2, S=1 << 21, H=1) == sd.SD_ERR_UNSUPPORTED
    assert b"2^22" in lib.sd_last_error()


def _kl(lib, T=FAKE, z=FAKE, idx=FAKE, B=1, S=8, K=4, N=2, g=1.0, rows=FAKE, dz=FAKE, st=FAKE, ws=FAKE,
        wsb=1 << 20):
    return lib.distill_kl_fwd_bwd(T, z, idx, B, S, K, N, g, rows, dz, st, ws, wsb, None)


def test_distill_kl_rejections(lib):
    # 2 floats (sum, count) per 8-row block
    assert lib.distill_kl_workspace_bytes(1, 8, 4) == 1 * 2 * 4
    assert lib.distill_kl_workspace_bytes(1, 12, 4) == 2 * 2 * 4
    assert lib.distill_kl_workspace_bytes(0, 8, 4) == 0
    assert _kl(lib, T=None) == sd.SD_ERR_NULL_ARG
    assert _kl(lib, rows=None) == sd.SD_ERR_NULL_ARG
    assert _kl(lib, st=None) == sd.SD_ERR_NULL_ARG
    assert _kl(lib, ws=None) == sd.SD_ERR_NULL_ARG
    assert _kl(lib, N=0) == sd.SD_ERR_BAD_SHAPE
    assert _kl(lib, g=float("nan")) == sd.SD_ERR_BAD_SHAPE
    assert _kl(lib, wsb=7) == sd.SD_ERR_BAD_SHAPE  # one 8-row block needs 8 bytes
    assert b"workspace" in lib.sd_last_error()
    assert _kl(lib, K=4097) == sd.SD_ERR_UNSUPPORTED
    # stats[1] is a float32 row count, exact up to 2^24: B*S at most 2^24
    assert _kl(lib, B=1, S=(1 << 24) + 1) == sd.SD_ERR_UNSUPPORTED
    assert b"2^24" in lib.sd_last_error()
    assert _kl(lib, B=2, S=(1 << 23) + 1) == sd.SD_ERR_UNSUPPORTED
    assert _kl(lib, B=4, S=1 << 22, wsb=7) == sd.SD_ERR_BAD_SHAPE        # 2^24 rows exactly: admitted
    assert _kl(lib, B=1 << 10, S=1 << 14, wsb=7) == sd.SD_ERR_BAD_SHAPE
    assert _kl(lib, ws=ctypes.c_void_p(0x1004)) == sd.SD_ERR_BAD_SHAPE   # not 16-byte aligned


def test_noalloc_kl_rejections(lib):
    def call(B=1, S=8, K=4, N=2, T=FAKE, st=FAKE, g=1.0):
        return lib.distill_kl_fwd_bwd_noalloc(T, FAKE, FAKE, B, S, K, N, g, FAKE, FAKE, st, None)
    assert call(T=None) == sd.SD_ERR_NULL_ARG
    assert call(st=None) == sd.SD_ERR_NULL_ARG
    assert call(N=0) == sd.SD_ERR_BAD_SHAPE
    assert call(K=4097) == sd.SD_ERR_UNSUPPORTED
    assert call(g=float("inf")) == sd.SD_ERR_BAD_SHAPE
    # its fixed scratch array holds the partials of 2^21 rows
    assert call(B=1, S=(1 << 21) + 1) == sd.SD_ERR_UNSUPPORTED
    assert b"2097152 rows" in lib.sd_last_error()
    assert call(B=2, S=(1 << 20) + 8) == sd.SD_ERR_UNSUPPORTED


def test_indexer_topk_rejections(lib):
    def topk(scores=FAKE, idx=FAKE, B=1, S=8, N=4, K=2, ratio=4):
        return lib.indexer_topk(scores, None, B, S, N, K, ratio, idx, None, None)

    def bwd(dv=FAKE, idx=FAKE, out=FAKE, B=1, S=8, N=4, K=2):
        return lib.indexer_topk_bwd(dv, idx, B, S, N, K, out, None)
    assert topk(scores=None) == sd.SD_ERR_NULL_ARG
    assert topk(idx=None) == sd.SD_ERR_NULL_ARG
    assert topk(N=0) == sd.SD_ERR_BAD_SHAPE
    assert topk(ratio=0) == sd.SD_ERR_BAD_SHAPE
    assert topk(K=-1) == sd.SD_ERR_BAD_SHAPE
    assert topk(N=4097) == sd.SD_ERR_UNSUPPORTED
    assert topk(K=4097) == sd.SD_ERR_UNSUPPORTED
    assert topk(B=1, S=1 << 26) == sd.SD_ERR_UNSUPPORTED           # 256 lanes per 4 rows
    assert b"2^32 - 1" in lib.sd_last_error()
    assert bwd(dv=None) == sd.SD_ERR_NULL_ARG
    assert bwd(out=None) == sd.SD_ERR_NULL_ARG
    assert bwd(S=0) == sd.SD_ERR_BAD_SHAPE
    assert bwd(N=5000) == sd.SD_ERR_UNSUPPORTED


def test_compressor_rejections(lib):
    A = ctypes.c_void_p(0x1000)       # 16-byte aligned placeholder

    def fwd(kv=A, sc=A, ape=A, out=A, B=1, S=16, D=8, r=4, ovl=1, dt=0):
        return lib.compressor_pool(kv, sc, ape, None, B, S, D, r, ovl, dt, out, None)

    def bwd(ws=A, wsb=1 << 20, D=8, r=4, ovl=1, dp=A):
        return lib.compressor_pool_bwd(A, A, A, None, dp, 1, 16, D, r, ovl, 0, A, A, A, ws, wsb, None)
    assert fwd(kv=None) == sd.SD_ERR_NULL_ARG
    assert fwd(out=None) == sd.SD_ERR_NULL_ARG
    assert fwd(dt=3) == sd.SD_ERR_DTYPE
    assert fwd(S=3) == sd.SD_ERR_BAD_SHAPE            # no complete block
    assert fwd(ovl=2) == sd.SD_ERR_BAD_SHAPE
    assert fwd(D=6) == sd.SD_ERR_UNSUPPORTED
    assert fwd(r=3) == sd.SD_ERR_UNSUPPORTED          # not a power of two
    assert fwd(r=32, S=64) == sd.SD_ERR_UNSUPPORTED   # overlap covers ratios up to 16
    assert fwd(r=256, S=512, ovl=0) == sd.SD_ERR_UNSUPPORTED
    assert fwd(kv=ctypes.c_void_p(0x1008)) == sd.SD_ERR_BAD_SHAPE   # not 16-byte aligned
    assert b"aligned" in lib.sd_last_error()
    # workspace: (B * ceil(N / 8)) chunks x Wc x D floats
    assert lib.compressor_pool_bwd_workspace_bytes(1, 16, 8, 4, 1) == 1 * 1 * 8 * 8 * 4
    assert lib.compressor_pool_bwd_workspace_bytes(2, 1000, 8, 4, 0) == 2 * 32 * 4 * 8 * 4
    assert lib.compressor_pool_bwd_workspace_bytes(1, 3, 8, 4, 0) == 0
    assert bwd(ws=None) == sd.SD_ERR_NULL_ARG
    assert bwd(dp=None) == sd.SD_ERR_NULL_ARG
    assert bwd(wsb=8) == sd.SD_ERR_BAD_SHAPE
    assert b"workspace" in lib.sd_last_error()


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 8, 4, 32, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        sd.window_lse(q, k, None, None, W=4)
    with pytest.raises(ValueError, match="GPU tensor"):
        sd.distill_target(q, torch.zeros(1, 2, 32, dtype=torch.bfloat16), torch.zeros(1, 8, 4, dtype=torch.int32))


def test_binding_maps_status_codes_to_exceptions(lib):
    assert _wl(lib, D=48) == sd.SD_ERR_UNSUPPORTED
    with pytest.raises(NotImplementedError, match="SD_ERR_UNSUPPORTED"):
        sd._check(sd.SD_ERR_UNSUPPORTED, "window_lse")
    with pytest.raises(ValueError):
        sd._check(sd.SD_ERR_BAD_SHAPE, "x")
    with pytest.raises(RuntimeError):
        sd._check(sd.SD_ERR_HIP, "x")


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library the binding raises; it has no CPU path to fall back to."""
    monkeypatch.setattr(sd, "_lib", None)
    monkeypatch.setattr(sd, "_LIB_PATH", str(tmp_path / "libsparse_distill.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sd.load_library()
