"""The allocation-free KL entry point, called through the C ABI, against the workspace entry
point (needs an MI355X).  Two calls in a row on one GPU, the second with a smaller input:
each must equal distill_kl_fwd_bwd bit for bit (the same kernels and reduction order; the
fixed scratch array keeps the larger call's partials, which the smaller call must not read),
and the smaller one also matches the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _kl_inputs(name, seed):
    c = synth.CONFIGS[name]
    idx = torch.from_numpy(synth.topk_slots(c, synth.rng_for(c, "idx")))
    rng = np.random.default_rng(seed)
    valid = ((idx >= 0) & (idx < c.N)).numpy()
    r = rng.random(idx.shape).astype(np.float32) * valid
    s = r.sum(-1, keepdims=True)
    T = np.where(s > 0, r / np.where(s > 0, s, 1), 0).astype(np.float32)
    z = rng.standard_normal(idx.shape).astype(np.float32)
    return c, T, z, idx


def test_noalloc_kl_matches_the_workspace_entry_point_on_two_calls():
    import sparse_attention_indexer_distill_amd as sd
    lib = sd.load_library()
    dev = torch.device("cuda:0")
    for name, seed in (("c3", 5), ("c2", 6)):           # the second call is smaller
        c, T, z, idx = _kl_inputs(name, seed)
        Td, zd, idd = torch.from_numpy(T).to(dev), torch.from_numpy(z).to(dev), idx.to(dev)
        print(f"[gpu] noalloc KL: {name} B={c.B} S={c.S} K={c.K}", flush=True)
        kl_ref, dz_ref, st_ref = sd.distill_kl_fwd_bwd(Td, zd, idd, c.N, grad_scale=0.5)
        kl = torch.full((c.B, c.S), float("nan"), device=dev)
        dz = torch.full((c.B, c.S, c.K), float("nan"), device=dev)
        st = torch.full((2,), float("nan"), device=dev)
        status = lib.distill_kl_fwd_bwd_noalloc(Td.data_ptr(), zd.data_ptr(), idd.data_ptr(), c.B, c.S, c.K, c.N,
                                                ctypes.c_float(0.5), kl.data_ptr(), dz.data_ptr(), st.data_ptr(),
                                                ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        assert status == sd.SD_OK, lib.sd_last_error()
        torch.cuda.synchronize(dev)
        assert torch.equal(kl, kl_ref) and torch.equal(dz, dz_ref) and torch.equal(st, st_ref)
        if name == "c2":
            kl_o, dz_o, st_o = oracle.kl(T, z, idx, c.N, grad_scale=0.5)
            kln = kl.cpu().numpy().reshape(-1)
            assert (np.abs(kln - kl_o) <= 1e-4 * np.abs(kl_o) + 2e-6).all()
            assert st.cpu().numpy()[1] == st_o[1]
            assert abs(st.cpu().numpy()[0] - st_o[0]) <= 1e-4 * abs(st_o[0])
    # the binding's wrapper reaches the same entry point
    kl2, dz2, st2 = sd.distill_kl_fwd_bwd_noalloc(Td, zd, idd, c.N, grad_scale=0.5)
    torch.cuda.synchronize(dev)
    assert torch.equal(kl2, kl_ref) and torch.equal(dz2, dz_ref) and torch.equal(st2, st_ref)
