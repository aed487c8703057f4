"""GPU parity of the fp8 latent cache path: mla_absorb_rope_fp8(_paged),
mla_decode_latent_fp8(_paged) and mla_combine_up_v through the C ABI against
the fp64 oracle run on the dequantised cache (codes times row scales; the
appended row is the oracle's own quantisation of c_kv_new).

Bars: the appended row (codes, scale, RoPE bytes) bit for bit; q_lat as in the
bf16 step; out and lse to the bf16 gates (max 2e-2, mean 5e-3) and to the
tighter bounds relative to the output scale, since the dequantised values are
exact in bf16 and the kernel computes the bf16 decode of them.
"""
import numpy as np
import pytest
import torch

from head_latent_attention_12_amd import synthetic as syn
from oracle import mla_oracle as orc
from tests.test_gpu_parity import check_out

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_12_amd import mla
    mla.lib()  # fail loudly if the HIP library is missing


def _bf16_f64(b: np.ndarray) -> np.ndarray:
    return syn.bf16_bits_to_f64(np.ascontiguousarray(b).view(np.uint16))


def fp8_oracle(inp, fp8: syn.Fp8Cache, batch_ids=None):
    """Oracle step over the dequantised fp8 cache; also the expected (codes,
    scale) of every appended row."""
    r = inp.r
    seqs = []
    for b in range(inp.B):
        o, L = int(inp.row_offsets[b]), int(inp.lens[b])
        seqs.append((orc.fp8_dequantize_rows(fp8.rows[o:o + L, :r], fp8.scale[o:o + L]),
                     _bf16_f64(fp8.rows[o:o + L, r:])))
    quant = [orc.fp8_quantize_row(c) for c in inp.f64("c_kv_new")]
    c_new = np.stack([orc.fp8_dequantize_rows(c[None, :], np.array([s]))[0] for c, s in quant])
    ref = orc.decode_batch(seqs, inp.f64("q_nope"), inp.f64("q_rope"), c_new, inp.f64("k_rope_new"),
                           inp.f64("w_uk"), inp.f64("w_uv"), inp.softmax_scale, inp.rope_base,
                           batch_ids=batch_ids)
    return ref, quant


def _step(inp, num_splits=None, page_rows=None, fp8_seed=3, max_seq_len=None):
    from head_latent_attention_12_amd.step import DeviceStep
    ds = DeviceStep(inp, num_splits=num_splits, page_rows=page_rows, page_seed=7, fp8=True, fp8_seed=fp8_seed,
                    max_seq_len=max_seq_len)
    ds.run()
    torch.cuda.synchronize()
    return ds


def check_fp8_step(inp, ds, ref, quant, tag):
    r = inp.r
    q_lat = ds.q_lat_f64()
    qt_ref = ref["q_lat"][:, :, :r]
    bound = 2.0 ** -8 * np.abs(qt_ref) + 1e-6 * np.abs(qt_ref).max()
    assert np.all(np.abs(q_lat[:, :, :r] - qt_ref) <= bound), tag
    np.testing.assert_array_equal(q_lat[:, :, r:], syn.bf16_bits_to_f64(syn.bf16_bits_from_f64(ref["q_lat"][:, :, r:])))
    # the appended rows: codes and scale exactly the oracle's quantisation,
    # the rotated key as in the bf16 row; every other row untouched
    rows, scale = ds.fp8_raw()
    slots = inp.row_offsets + inp.lens
    np.testing.assert_array_equal(rows[slots, :r], np.stack([c for c, _ in quant]), err_msg=tag)
    np.testing.assert_array_equal(scale[slots].astype(np.float64), np.array([s for _, s in quant]), err_msg=tag)
    np.testing.assert_array_equal(rows[slots, r:].view(np.uint16), syn.bf16_bits_from_f64(ref["new_row"][:, r:]))
    keep = np.ones(inp.total_rows, bool)
    keep[slots] = False
    np.testing.assert_array_equal(rows[keep], ds.fp8.rows[keep])
    np.testing.assert_array_equal(scale[keep], ds.fp8.scale[keep])
    out = ds.out.cpu().numpy().astype(np.float64)
    lse = ds.lse.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(lse, ref["lse"], rtol=0, atol=2e-2)
    check_out(inp, out, ref["out"], tag)


FP8_CASES = [
    ("dsv2", dict(B=2, T=300), None),
    ("dsv2", dict(lens=[0, 1, 30, 31, 32, 33, 63, 64, 65, 200]), None),   # tile edges and one-row splits
    ("dsv2", dict(B=3, T=1000), 1),                                       # one split: a long steady loop
    ("dsv2", dict(B=3, T=1000), 40),                                      # many splits, some empty
    ("dsv2_ragged", dict(B=6, T=(1, 700)), None),
    ("dsv2", {}, None),                                                   # B 16, T 4096 (the bench launch)
    ("dsv2_ragged", {}, None),
]


@pytest.mark.parametrize("name,override,splits", FP8_CASES, ids=[f"{n}-{o}-s{s}" for n, o, s in FP8_CASES])
def test_fp8_step_matches_oracle(name, override, splits):
    inp = syn.make_inputs(name, **override)
    ds = _step(inp, num_splits=splits)
    ref, quant = fp8_oracle(inp, ds.fp8)
    check_fp8_step(inp, ds, ref, quant, f"fp8 {name} {override} splits {ds.num_splits}")


def test_fp8_long_context_sampled():
    """DeepSeek-V2 long context (B 2, T 131072) at its planned split count: the
    appended rows and both sequences' outputs against the oracle."""
    inp = syn.make_inputs("dsv2_long")
    ds = _step(inp)
    ref, quant = fp8_oracle(inp, ds.fp8)
    check_fp8_step(inp, ds, ref, quant, f"fp8 dsv2_long splits {ds.num_splits}")


PAGED_FP8_CASES = [
    ("dsv2", dict(lens=[0, 31, 32, 63, 64, 65, 127, 128]), 64, None),
    ("dsv2", dict(B=2, T=3000), 32, 2),
    ("dsv2_ragged", dict(B=6, T=(1, 700)), 256, None),
    ("dsv2_ragged", {}, 64, None),
]


@pytest.mark.parametrize("name,override,page_rows,splits", PAGED_FP8_CASES,
                         ids=[f"{n}-{o}-p{p}-s{q}" for n, o, p, q in PAGED_FP8_CASES])
def test_fp8_paged_matches_packed_and_oracle(name, override, page_rows, splits):
    """Pages shuffled, unused page rows NaN codes and scales: bit for bit the
    packed fp8 step, and against the oracle."""
    inp = syn.make_inputs(name, **override)
    packed = _step(inp, num_splits=splits)
    ds = _step(inp, num_splits=packed.num_splits, max_seq_len=packed.max_seq_len, page_rows=page_rows)
    assert torch.equal(ds.q_lat, packed.q_lat)
    assert torch.equal(ds.lse_part, packed.lse_part)
    assert torch.equal(ds.out, packed.out) and torch.equal(ds.lse, packed.lse)
    pr, ps = ds.fp8_raw()
    qr, qs = packed.fp8_raw()
    np.testing.assert_array_equal(pr, qr)
    np.testing.assert_array_equal(ps.view(np.uint32), qs.view(np.uint32))
    ref, quant = fp8_oracle(inp, ds.fp8)
    check_fp8_step(inp, ds, ref, quant, f"fp8 paged {name} {override} p{page_rows}")


def test_fp8_score_growth_redo():
    """Row scales raised 2^4 from row 40 on and q_nope scaled by 20 make later
    scores exceed the first tile's reference by far more than 2^64 in weight:
    the work-group rescans and redoes the split.  W_UK is a 0/1 selection so
    that q~ is exact in bf16 (its rounding would otherwise move scores spread
    over hundreds of nats by tenths of a nat, which says nothing about the
    kernel); the output is checked normwise as in the bf16 redo test."""
    import math
    from head_latent_attention_12_amd.step import DeviceStep
    from tests._util import normwise_rel
    inp = syn.make_inputs("dsv2", B=2, T=400)
    w = np.zeros((inp.H, inp.d_head, inp.r))
    w[:, np.arange(inp.d_head), np.arange(inp.d_head)] = 1.0
    inp.w_uk = syn.bf16_bits_from_f64(w)
    inp.q_nope = syn.bf16_bits_from_f64(inp.f64("q_nope") * 20.0)
    ds = DeviceStep(inp, num_splits=1, fp8=True)
    for b in range(inp.B):
        o, L = int(inp.row_offsets[b]), int(inp.lens[b])
        ds.fp8.scale[o + 40:o + L] *= np.float32(16.0)
    ds.kv_scale.copy_(torch.from_numpy(ds.fp8.scale))
    ds.run()
    torch.cuda.synchronize()
    ref, quant = fp8_oracle(inp, ds.fp8)
    assert ref["lse"].max() * math.log2(math.e) > 64   # the scores really do grow past the slack
    rows, scale = ds.fp8_raw()
    slots = inp.row_offsets + inp.lens
    np.testing.assert_array_equal(rows[slots, :inp.r], np.stack([c for c, _ in quant]))
    out = ds.out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out))
    rel = normwise_rel(out, ref["out"])
    print(f"[fp8 redo] normwise rel err {rel:.3e}", flush=True)
    assert rel <= 2e-2


def test_fp8_deterministic_and_graph_replay():
    """Two eager steps give the same bits; a captured graph of the fp8 step
    replays to the same bits (eager work between replays)."""
    inp = syn.make_inputs("dsv2", B=4, T=2000)
    ds = _step(inp)
    out1, lse1 = ds.out.clone(), ds.lse.clone()
    ds.run()
    torch.cuda.synchronize()
    assert torch.equal(ds.out, out1) and torch.equal(ds.lse, lse1)
    g = ds.capture()
    for _ in range(3):
        ds.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ds.out, out1)


def test_fp8_inconsistent_metadata_stays_in_bounds():
    """Device metadata the host cannot check (row offsets before and past the
    cache, lengths past max_seq_len or negative, positions far out, page ids
    out of range, lengths past the block table) is clamped inside the fp8
    append and decode: the calls complete with wrong numbers, never a stray
    access, and a correct fp8 step afterwards still matches the oracle."""
    from head_latent_attention_12_amd.step import DeviceStep
    inp = syn.make_inputs("dsv2", B=3, T=200)
    ds = DeviceStep(inp, num_splits=4, fp8=True)
    ds.row_offsets.copy_(torch.tensor([-(10 ** 9), inp.total_rows + 7, 10 ** 12], dtype=torch.int64))
    ds.seq_lens.copy_(torch.tensor([10 ** 6, -3, int(inp.seq_lens[2])], dtype=torch.int32))
    ds.positions.copy_(torch.tensor([10 ** 6, -9, 2 ** 30], dtype=torch.int32))
    ds.run()
    torch.cuda.synchronize()
    dp = DeviceStep(inp, num_splits=4, page_rows=64, fp8=True)
    bt = dp.block_table.clone()
    bt[:, 0] = -7
    bt[:, -1] = dp.paged.total_pages + 100
    dp.block_table.copy_(bt)
    dp.seq_lens.copy_(torch.tensor([10 ** 6, 1, 64 * dp.paged.bt_stride + 500], dtype=torch.int32))
    dp.run()
    torch.cuda.synchronize()
    clean = _step(inp)
    ref, quant = fp8_oracle(inp, clean.fp8)
    check_fp8_step(inp, clean, ref, quant, "fp8 after bad metadata")


def test_fp8_cache_rows_past_4gib():
    """The fp8 cache with the second sequence's rows 5 GiB in (byte offsets
    past 2^32), the rows between NaN codes and NaN scales: both sequences
    match the oracle, the appended rows land in their slots, nothing else
    changes."""
    import dataclasses
    from head_latent_attention_12_amd.step import DeviceStep
    inp = syn.make_inputs("dsv2", lens=[300, 700])
    ds = DeviceStep(inp, fp8=True, fp8_seed=3)
    ref, quant = fp8_oracle(inp, ds.fp8)
    r = inp.r
    o1, n1 = int(inp.row_offsets[1]), int(inp.seq_lens[1])
    row_b = ds.kv_cache.shape[1]
    gap = -(-5 * (1 << 30) // row_b)
    small, small_s = ds.kv_cache, ds.kv_scale
    big = torch.full((gap + n1, row_b), 0x7F, dtype=small.dtype, device=small.device)
    big_s = torch.full((gap + n1,), float("nan"), dtype=torch.float32, device=small.device)
    big[:o1], big[gap:] = small[:o1], small[o1:]
    big_s[:o1], big_s[gap:] = small_s[:o1], small_s[o1:]
    ds.kv_cache, ds.kv_scale = big, big_s
    ds.row_offsets.copy_(torch.tensor([0, gap], dtype=torch.int64))
    ds.inp = dataclasses.replace(inp, row_offsets=np.array([0, gap], np.int64), total_rows=gap + n1)
    slots = [int(inp.lens[0]), gap + int(inp.lens[1])]
    assert slots[1] * row_b >= 4 * (1 << 30)
    ds.run()
    torch.cuda.synchronize()
    tag = "fp8 cache past 4 GiB"
    q_lat = ds.q_lat_f64()
    qt_ref = ref["q_lat"][:, :, :r]
    assert np.all(np.abs(q_lat[:, :, :r] - qt_ref) <= 2.0 ** -8 * np.abs(qt_ref) + 1e-6 * np.abs(qt_ref).max())
    np.testing.assert_allclose(ds.lse.cpu().numpy().astype(np.float64), ref["lse"], rtol=0, atol=2e-2)
    check_out(inp, ds.out.cpu().numpy().astype(np.float64), ref["out"], tag)
    # the appended rows: codes, scale and rotated key bytes
    rope_bits = syn.bf16_bits_from_f64(ref["new_row"][:, r:])
    for b in range(2):
        row = big[slots[b]].cpu().numpy()
        np.testing.assert_array_equal(row[:r], quant[b][0], err_msg=tag)
        np.testing.assert_array_equal(row[r:].view(np.uint16), rope_bits[b], err_msg=tag)
        assert float(big_s[slots[b]]) == quant[b][1], tag
    # the other rows: the live regions as before, the rows between still NaN
    for first, end, src in ((0, o1, 0), (gap, gap + n1, o1)):
        keep = torch.ones(end - first, dtype=torch.bool, device=big.device)
        for b in range(2):
            if first <= slots[b] < end:
                keep[slots[b] - first] = False
        assert torch.equal(big[first:end][keep], small[src:src + end - first][keep]), tag
        assert torch.equal(big_s[first:end][keep].view(torch.int32), small_s[src:src + end - first][keep].view(torch.int32)), tag
    assert bool((big[o1:gap] == 0x7F).all()) and bool(torch.isnan(big_s[o1:gap]).all()), tag
