"""The kernels on the measured paths compile without register spills (CPU only: a device-only
hipcc pass with the library's flags, read from the compiler's resource-usage remarks).

A spill puts scratch-memory loads and stores inside the score loops; it has come from small,
unrelated edits that changed the schedule, so it is checked here rather than found in a timing.
"""
import concurrent.futures as cf
import os
import shutil

import pytest

from sparse_attention_indexer_distill_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which(build.HIPCC) is None,
                                reason="hipcc not available")

# (source, substring of the mangled kernel name, minimum waves per SIMD)
HOT = [
    ("distill_target.hip", "distill_target_kernelILi0ELi4ELi4ELi8ELb1E", 4),    # fused target, K <= 512, 64 heads
    ("distill_target.hip", "distill_target_kernelILi0ELi4ELi4ELi16ELb1E", 4),   # fused target, K <= 1024
    ("distill_target.hip", "distill_target_kernelILi0ELi4ELi4ELi8ELb0E", 4),    # three-call target
    ("window_lse.hip", "window_lse_mfma_kernelILi9E", 1),                       # window LSE, W = 128
    ("distill_kl.hip", "distill_kl_kernelILi4ELi2E", 1),                        # KL, K = 512
    ("distill_kl.hip", "distill_kl_kernelILi4ELi4E", 1),                        # KL, K = 1024
    ("indexer_topk.hip", "indexer_topk_kernelILi16E", 1),                       # top-k, N = 1024
    ("indexer_topk.hip", "indexer_topk_kernelILi32E", 1),                       # top-k, N = 2048
    ("indexer_topk.hip", "indexer_topk_bwd_kernelILi8E", 1),                    # top-k scatter, K = 512
    ("indexer_topk.hip", "indexer_topk_bwd_kernelILi16E", 1),                   # top-k scatter, K = 1024
    ("compressor_pool.hip", "compressor_pool_kernelILi0ELi4ELi1ELi2E", 1),      # CSA compressor, ratio 4
    ("compressor_pool.hip", "compressor_pool_bwd_kernelILi0ELi4ELi1ELi2E", 1),
]


@pytest.fixture(scope="module")
def resources():
    srcs = sorted({s for s, _, _ in HOT})
    with cf.ThreadPoolExecutor(len(srcs)) as ex:
        return dict(zip(srcs, ex.map(build.kernel_resources, srcs)))


@pytest.mark.parametrize("src,pattern,occ", HOT, ids=[p for _, p, _ in HOT])
def test_hot_kernel_has_no_spills(resources, src, pattern, occ):
    found = {k: v for k, v in resources[src].items() if pattern in k}
    assert len(found) == 1, f"{pattern}: {len(found)} kernels match in {src}"
    (name, r), = found.items()
    assert r["scratch"] == 0, f"{name} spills {r['scratch']} bytes per lane ({r})"
    assert r["occupancy"] >= occ, f"{name}: occupancy {r['occupancy']} waves/SIMD < {occ} ({r})"


@pytest.mark.parametrize("src", ["compressor_pool.hip", "indexer_topk.hip", "distill_kl.hip"])
def test_every_instantiation_has_no_spills(resources, src):
    """The next-row kernels and the KL, at every ratio, window and width they are built for."""
    bad = {k: v for k, v in resources[src].items() if v["scratch"] > 0}
    assert not bad, f"{src}: {bad}"
