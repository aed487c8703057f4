"""mla_kv_down_noalloc (partial sums in the library's fixed device array)
against mla_kv_down (partial sums in a caller workspace): the same kernels in
the same order, so the outputs must be bit for bit equal.  Two calls in a
row, the second smaller, check that nothing of the first call's scratch
contents leaks into the second; a call too large for the scratch is refused
on the host."""
import numpy as np
import pytest
import torch

from head_latent_attention_12_amd import synthetic as syn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_12_amd import mla
    mla.lib()  # fail loudly if the HIP library is missing


def _dev(a):
    from head_latent_attention_12_amd.step import _dev as dev
    return dev(a, "cuda")


def _both(B, d_model, seed):
    from head_latent_attention_12_amd import mla
    kin = syn.make_kv_down_inputs(B, d_model, seed=seed)
    dims = mla.make_dims(B, 128, 128, 128, kin.r, kin.d_rope, mla.MLA_BF16)
    h, w_dkv, w_kr, g = (_dev(getattr(kin, k)) for k in ("h", "w_dkv", "w_kr", "norm_w"))
    work = torch.empty(mla.mla_kv_down_workspace_size(dims, d_model) // 4, dtype=torch.float32, device="cuda")
    c_ref = torch.empty((B, kin.r), dtype=torch.int16, device="cuda")
    k_ref = torch.empty((B, kin.d_rope), dtype=torch.int16, device="cuda")
    mla.mla_kv_down(dims, d_model, h, w_dkv, w_kr, g, kin.eps, work, c_ref, k_ref)
    c_na = torch.full_like(c_ref, 0x7FC0)
    k_na = torch.full_like(k_ref, 0x7FC0)
    mla.mla_kv_down_noalloc(dims, d_model, h, w_dkv, w_kr, g, kin.eps, c_na, k_na)
    torch.cuda.synchronize()
    return c_ref, k_ref, c_na, k_na


def test_noalloc_matches_workspace_call_twice_second_smaller():
    for B, d_model, seed in ((64, 7168, 41), (16, 2048, 42)):
        print(f"[kv_down_noalloc] B={B} d_model={d_model}", flush=True)
        c_ref, k_ref, c_na, k_na = _both(B, d_model, seed)
        assert torch.equal(c_ref, c_na) and torch.equal(k_ref, k_na)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    from head_latent_attention_12_amd import mla
    dims = mla.make_dims(256, 128, 128, 128, 512, 64, mla.MLA_BF16)
    # 16 chunks x 256 sequences x 576 features x 4 bytes = 9.4 MB > 4 MiB
    t = torch.empty(16, dtype=torch.int16, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_kv_down_noalloc(dims, 8192, t, t, t, t, 1e-6, t, t)
    assert e.value.status == 4
