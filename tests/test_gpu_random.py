"""GPU parity on seeded random configurations of the bf16 DeepSeek-V2 shape:
batch sizes 1..70, cached lengths 0..3000 (an empty sequence now and then),
the planner's split count or an explicit one in 1..64, a packed cache or
pages of 32..256 rows, bf16 or fp8 latents; and of the two fp32 shapes (the
tiny and small workloads' dimensions) with batch sizes 1..20, lengths
0..2000, split counts and page sizes drawn the same way.  Each case runs the step
(absorb_rope, decode_latent, combine_up_v) through the C ABI and compares out
and lse with the fp64 oracle (for fp8, on the dequantised cache) through the
parity gate of the other GPU tests.  The draw is fixed (seeded), so the cases
are the same on every run; the combinations cover what the hand-picked cases
take one axis at a time.
"""
import numpy as np
import pytest
import torch

from head_latent_attention_12_amd import synthetic as syn
from tests._util import gate_failures, oracle_step
from tests.test_gpu_fp8 import fp8_oracle

pytestmark = pytest.mark.gpu

N_CASES = 24


def _cases():
    rng = np.random.default_rng(20261204)
    out = []
    for c in range(N_CASES):
        B = int(rng.integers(1, 71))
        lens = rng.integers(0, min(3000, 60000 // B) + 1, size=B)
        if rng.random() < 0.2:
            lens[rng.integers(0, B)] = 0
        splits = None if rng.random() < 0.4 else int(rng.integers(1, 65))
        page_rows = [None, None, 32, 64, 128, 256][int(rng.integers(0, 6))]
        fp8 = bool(rng.random() < 0.3)
        out.append((c, [int(x) for x in lens], splits, page_rows, fp8))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_12_amd import mla
    mla.lib()  # fail loudly if the HIP library is missing


@pytest.mark.parametrize("case,lens,splits,page_rows,fp8", CASES,
                         ids=[f"c{c}-B{len(l)}-s{s}-p{p}-{'fp8' if f else 'bf16'}" for c, l, s, p, f in CASES])
def test_random_configuration(case, lens, splits, page_rows, fp8):
    from head_latent_attention_12_amd.step import DeviceStep
    inp = syn.make_inputs("dsv2", lens=lens, seed=1000 + case)
    ds = DeviceStep(inp, num_splits=splits, page_rows=page_rows, page_seed=case, fp8=fp8, fp8_seed=7 + case)
    ds.run()
    torch.cuda.synchronize()
    ref = fp8_oracle(inp, ds.fp8)[0] if fp8 else oracle_step(inp)
    out = ds.out.cpu().numpy().astype(np.float64)
    lse = ds.lse.cpu().numpy().astype(np.float64)
    err = np.abs(out - ref["out"])
    print(f"[case {case}] B {inp.B} splits {ds.num_splits} pages {page_rows} fp8 {fp8}: "
          f"max {err.max():.2e} mean {err.mean():.2e}", flush=True)
    assert not gate_failures("bf16", out, ref["out"])
    np.testing.assert_allclose(lse, ref["lse"], rtol=0, atol=2e-2)


def _f32_cases():
    rng = np.random.default_rng(20261205)
    out = []
    for c in range(16):
        name = "tiny" if rng.random() < 0.5 else "small"
        B = int(rng.integers(1, 21))
        lens = rng.integers(0, 2001, size=B)
        if rng.random() < 0.2:
            lens[rng.integers(0, B)] = 0
        splits = None if rng.random() < 0.4 else int(rng.integers(1, 65))
        page_rows = [None, None, 32, 64, 128][int(rng.integers(0, 5))]
        out.append((c, name, [int(x) for x in lens], splits, page_rows))
    return out


F32_CASES = _f32_cases()


@pytest.mark.parametrize("case,name,lens,splits,page_rows", F32_CASES,
                         ids=[f"c{c}-{n}-B{len(l)}-s{s}-p{p}" for c, n, l, s, p in F32_CASES])
def test_random_configuration_f32(case, name, lens, splits, page_rows):
    from head_latent_attention_12_amd.step import DeviceStep
    inp = syn.make_inputs(name, lens=lens, seed=2000 + case)
    ds = DeviceStep(inp, num_splits=splits, page_rows=page_rows, page_seed=case)
    ds.run()
    torch.cuda.synchronize()
    ref = oracle_step(inp)
    out = ds.out.cpu().numpy().astype(np.float64)
    lse = ds.lse.cpu().numpy().astype(np.float64)
    print(f"[f32 case {case}] {name} B {inp.B} splits {ds.num_splits} pages {page_rows}: "
          f"max {np.abs(out - ref['out']).max():.2e}", flush=True)
    assert not gate_failures("f32", out, ref["out"])
    np.testing.assert_allclose(lse, ref["lse"], rtol=0, atol=1e-5 * max(1.0, np.abs(ref["lse"]).max()))
