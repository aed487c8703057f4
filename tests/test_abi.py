"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/mla.h, and rejects bad arguments on the host before any
HIP call (so no compute call is made here)."""
import ctypes
import os
import re

import pytest

from head_latent_attention_12_amd import mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH), reason="libmla.so not built")

P16 = 0x1000  # an aligned, never-dereferenced stand-in address (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("mla_absorb_q", "mla_rope_append", "mla_decode_latent", "mla_combine", "mla_up_v"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(mla.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(mla.EXPORTS) == set(declared_functions())


def dsv2():
    return mla.make_dims(16, 128, 128, 128, 512, 64, mla.MLA_BF16)


def test_status_strings():
    L = mla.lib()
    for code, name in mla.STATUS.items():
        assert L.mla_status_string(code).decode() == name


@pytest.mark.parametrize("dims,code", [
    (mla.make_dims(16, 128, 128, 128, 512, 64, mla.MLA_BF16), 0),
    (mla.make_dims(1, 8, 32, 32, 64, 16, mla.MLA_F32), 0),
    (mla.make_dims(8, 16, 64, 64, 64, 32, mla.MLA_F32), 0),
    (mla.make_dims(0, 128, 128, 128, 512, 64, mla.MLA_BF16), 1),      # batch 0
    (mla.make_dims(16, 128, 128, 128, 512, 63, mla.MLA_BF16), 1),     # odd d_rope
    (mla.make_dims(16, 128, 128, 128, 512, 64, 7), 1),                # unknown dtype
    (mla.make_dims(16, 128, -1, 128, 512, 64, mla.MLA_BF16), 1),      # negative width
    (mla.make_dims(16, 64, 128, 128, 512, 64, mla.MLA_BF16), 2),      # no instantiation
    (mla.make_dims(16, 128, 128, 128, 512, 64, mla.MLA_F32), 2),      # fp32 at this shape
    (mla.make_dims(16, 128, 96, 128, 512, 64, mla.MLA_BF16), 2),      # d_head 96
    (mla.make_dims(16, 128, 128, 100, 512, 64, mla.MLA_BF16), 2),     # d_v not a multiple of 32
])
def test_check_dims(dims, code):
    assert mla.mla_check_dims(dims) == code


def test_null_dims():
    L = mla.lib()
    assert L.mla_check_dims(None) == 1
    assert L.mla_absorb_q(None, P16, P16, P16, None) == 1


def _expect(code, fn, *args):
    with pytest.raises(mla.MlaError) as e:
        fn(*args)
    assert e.value.status == code
    assert mla.lib().mla_last_error().decode() != ""


def test_entry_points_reject_null_and_misaligned_pointers():
    d = dsv2()
    _expect(1, mla.mla_absorb_q, d, 0, P16, P16, 0)
    _expect(3, mla.mla_absorb_q, d, P16 + 2, P16, P16, 0)
    _expect(1, mla.mla_rope_append, d, P16, P16, P16, 0, P16, 10, P16, P16, 0)
    _expect(3, mla.mla_rope_append, d, P16, P16, P16, P16, P16, 10, P16, P16 + 8, 0)
    _expect(1, mla.mla_rope_append, d, P16, P16, P16, P16, P16, 0, P16, P16, 0)       # total_rows 0
    _expect(1, mla.mla_decode_latent, d, P16, P16, P16, P16, 10, 5, 1, 0, P16, 0)     # o_part NULL
    _expect(3, mla.mla_decode_latent, d, P16, P16 + 4, P16, P16, 10, 5, 1, P16, P16, 0)
    _expect(1, mla.mla_combine, d, P16, P16, 1, 0, None, 0)
    _expect(1, mla.mla_up_v, d, P16, 0, P16, 0)
    _expect(3, mla.mla_up_v, d, P16, P16, P16 + 12, 0)
    _expect(1, mla.mla_absorb_rope, d, P16, P16, P16, P16, P16, P16, P16, 0, P16, P16, 0)   # total_rows 0
    _expect(1, mla.mla_absorb_rope, d, P16, P16, P16, P16, P16, 0, P16, 10, P16, P16, 0)    # positions NULL
    _expect(1, mla.mla_absorb_rope, d, 0, P16, P16, P16, P16, P16, P16, 10, P16, P16, 0)    # q_nope NULL
    _expect(3, mla.mla_absorb_rope, d, P16, P16 + 2, P16, P16, P16, P16, P16, 10, P16, P16, 0)
    _expect(1, mla.mla_combine_up_v, d, P16, P16, 1, 0, P16, None, 0)               # w_uv NULL
    _expect(1, mla.mla_combine_up_v, d, P16, 0, 1, P16, P16, None, 0)               # lse_part NULL
    _expect(3, mla.mla_combine_up_v, d, P16, P16, 1, P16, P16 + 4, None, 0)


def test_split_count_limits():
    d = dsv2()
    _expect(1, mla.mla_decode_latent, d, P16, P16, P16, P16, 10, 5, 0, P16, P16, 0)
    _expect(4, mla.mla_decode_latent, d, P16, P16, P16, P16, 10, 5, 4097, P16, P16, 0)
    _expect(1, mla.mla_decode_latent, d, P16, P16, P16, P16, 10, 0, 1, P16, P16, 0)   # max_seq_len 0
    _expect(1, mla.mla_combine, d, P16, P16, 0, P16, None, 0)
    _expect(4, mla.mla_combine, d, P16, P16, 5000, P16, None, 0)
    _expect(1, mla.mla_combine_up_v, d, P16, P16, 0, P16, P16, None, 0)
    _expect(4, mla.mla_combine_up_v, d, P16, P16, 4097, P16, P16, None, 0)
    _expect(4, mla.mla_partials_size, d, 4097)


def test_partials_size():
    # partials are stored in the cache dtype: bf16 here, fp32 for MLA_F32
    d = dsv2()
    o, l = mla.mla_partials_size(d, 7)
    assert o == 16 * 7 * 128 * 512 * 2 and l == 16 * 7 * 128 * 4
    f = mla.make_dims(8, 16, 64, 64, 64, 32, mla.MLA_F32)
    o, l = mla.mla_partials_size(f, 3)
    assert o == 8 * 3 * 16 * 64 * 4 and l == 8 * 3 * 16 * 4


@pytest.mark.parametrize("B,T,total,cus,expect_max_wgs", [
    (16, 4097, 16 * 4097, 256, 256),
    (2, 131073, 2 * 131073, 256, 256),
    (64, 8193, 278592, 256, 300),
    (1, 129, 129, 256, 256),
])
def test_plan_splits(B, T, total, cus, expect_max_wgs):
    d = mla.make_dims(B, 128, 128, 128, 512, 64, mla.MLA_BF16)
    s = mla.mla_plan_splits(d, T, total, cus)
    assert 1 <= s <= 4096
    chunk = -(-T // s)
    chunk = -(-chunk // 32) * 32
    assert chunk % 32 == 0 and s * chunk >= T
    # uniform lengths: every split of every sequence holds rows
    if total == B * T:
        assert B * s <= expect_max_wgs


def test_plan_splits_rejects_bad_args():
    d = dsv2()
    with pytest.raises(mla.MlaError):
        mla.mla_plan_splits(d, 0, 10, 256)


@pytest.mark.parametrize("seed", range(6))
def test_plan_splits_ragged_one_round(seed):
    """Ragged batches (64 sequences, 512..8192 cached tokens): the planned split
    count gives at most one work-group per CU (the non-empty splits fit the
    256 CUs), and never fewer than a quarter of the CUs' worth of work items."""
    import numpy as np
    lens = np.random.default_rng(100 + seed).integers(512, 8192, size=64, endpoint=True) + 1
    T, total = int(lens.max()), int(lens.sum())
    d = mla.make_dims(64, 128, 128, 128, 512, 64, mla.MLA_BF16)
    s = mla.mla_plan_splits(d, T, total, 256)
    chunk = -(-T // s)
    chunk = -(-chunk // 32) * 32
    items = int(sum(min(s, -(-int(l) // chunk)) for l in lens))
    assert 64 <= items <= 256, (s, chunk, items)


def test_plan_splits_prefers_one_round_over_finer_splits():
    """A uniform batch whose finer split would need two rounds of work-groups
    stays at a coarser split (B = 16, T = 4097: at most 256 work items)."""
    d = mla.make_dims(16, 128, 128, 128, 512, 64, mla.MLA_BF16)
    s = mla.mla_plan_splits(d, 4097, 16 * 4097, 256)
    chunk = -(-(-(-4097 // s)) // 32) * 32
    assert 16 * -(-4097 // chunk) <= 256
    assert s >= 8


@pytest.mark.parametrize("seed", range(6))
def test_plan_splits_for_lengths_ragged(seed):
    """With the lengths known, ragged batches of 64 sequences (512..8192
    cached tokens) get a chunk whose non-empty splits fill the 256 CUs in one
    round (at most 32 per XCD) with splits no longer than the length-blind
    plan's; the returned max_seq_len is at least every length and yields that
    chunk."""
    import numpy as np
    lens = np.random.default_rng(100 + seed).integers(512, 8192, size=64, endpoint=True) + 1
    d = mla.make_dims(64, 128, 128, 128, 512, 64, mla.MLA_BF16)
    s, mls = mla.mla_plan_splits_for_lengths(d, lens, 256)
    assert mls >= lens.max() and 1 <= s <= 4096
    chunk = -(-(-(-mls // s)) // 32) * 32
    items = int(sum(-(-int(l) // chunk) for l in lens))
    assert max(-(-int(l) // chunk) for l in lens) <= s
    assert -(-items // 8) <= 32, (s, chunk, items)
    s0 = mla.mla_plan_splits(d, int(lens.max()), int(lens.sum()), 256)
    chunk0 = -(-(-(-int(lens.max()) // s0)) // 32) * 32
    assert chunk <= chunk0


def test_plan_splits_for_lengths_seeded_ragged_workload():
    """The seeded ragged workload: 37-tile splits, 253 work items (the
    length-blind plan takes 42-tile splits)."""
    from head_latent_attention_12_amd import synthetic as syn
    inp = syn.make_inputs("dsv2_ragged")
    d = mla.make_dims(inp.B, 128, 128, 128, 512, 64, mla.MLA_BF16)
    s, mls = mla.mla_plan_splits_for_lengths(d, inp.seq_lens, 256)
    chunk = -(-(-(-mls // s)) // 32) * 32
    assert chunk == 37 * 32
    assert int(sum(-(-int(l) // chunk) for l in inp.seq_lens)) == 253


@pytest.mark.parametrize("B,L,expect", [(16, 4097, 13), (2, 131073, 125)])
def test_plan_splits_for_lengths_uniform(B, L, expect):
    d = mla.make_dims(B, 128, 128, 128, 512, 64, mla.MLA_BF16)
    s, mls = mla.mla_plan_splits_for_lengths(d, [L] * B, 256)
    assert s == expect == mla.mla_plan_splits(d, L, B * L, 256)
    assert mls >= L


def test_plan_splits_for_lengths_rejects_bad_args():
    d = mla.make_dims(3, 128, 128, 128, 512, 64, mla.MLA_BF16)
    with pytest.raises(mla.MlaError):
        mla.mla_plan_splits_for_lengths(d, [5, 0, 7], 256)


def test_paged_argument_checks():
    """Host-side checks of the paged calls: page size a power of two from 32
    to 65536, a block table, at least one page and one entry per sequence."""
    d = dsv2()
    ok = dict(bt=P16, stride=4, page=64, pages=10)

    def dec(bt=ok["bt"], stride=ok["stride"], page=ok["page"], pages=ok["pages"]):
        mla.mla_decode_latent_paged(d, P16, P16, bt, stride, page, pages, P16, 100, 2, P16, P16, 0)

    def rope(bt=ok["bt"], stride=ok["stride"], page=ok["page"], pages=ok["pages"]):
        mla.mla_rope_append_paged(d, P16, P16, P16, P16, bt, stride, page, pages, P16, P16, 0)

    def absorb(bt=ok["bt"], stride=ok["stride"], page=ok["page"], pages=ok["pages"]):
        mla.mla_absorb_rope_paged(d, P16, P16, P16, P16, P16, P16, bt, stride, page, pages, P16, P16, 0)

    for fn in (dec, rope, absorb):
        for bad in (dict(bt=0), dict(stride=0), dict(page=16), dict(page=96), dict(page=1 << 17), dict(pages=0)):
            _expect(1, lambda: fn(**bad))
    _expect(1, mla.mla_decode_latent_paged, d, P16, P16, P16, 4, 64, 10, 0, 100, 2, P16, P16, 0)   # seq_lens NULL
    _expect(4, mla.mla_decode_latent_paged, d, P16, P16, P16, 4, 64, 10, P16, 100, 4097, P16, P16, 0)
    _expect(3, mla.mla_decode_latent_paged, d, P16, P16 + 8, P16, 4, 64, 10, P16, 100, 2, P16, P16, 0)


def test_fp8_argument_checks():
    """Host-side checks of the fp8 cache calls (no kernel runs): only the bf16
    (128, 512, 64) instance, a non-NULL 16-byte-aligned scale array, and the
    checks of the bf16 counterparts (row offsets, pages, splits, alignment)."""
    d = dsv2()
    small = mla.make_dims(8, 16, 64, 64, 64, 32, mla.MLA_F32)

    def dec(dims=d, scale=P16, off=P16, rows=100, splits=2, cache=P16):
        mla.mla_decode_latent_fp8(dims, P16, cache, scale, off, P16, rows, 100, splits, P16, P16, 0)

    def dec_paged(dims=d, scale=P16, page=64):
        mla.mla_decode_latent_fp8_paged(dims, P16, P16, scale, P16, 4, page, 10, P16, 100, 2, P16, P16, 0)

    def absorb(dims=d, scale=P16, off=P16, rows=100):
        mla.mla_absorb_rope_fp8(dims, P16, P16, P16, P16, P16, P16, off, rows, P16, P16, scale, 0)

    def absorb_paged(dims=d, scale=P16, page=64):
        mla.mla_absorb_rope_fp8_paged(dims, P16, P16, P16, P16, P16, P16, P16, 4, page, 10, P16, P16, scale, 0)

    for fn in (dec, dec_paged, absorb, absorb_paged):
        _expect(2, lambda: fn(dims=small))        # no fp8 form of the fp32 instances
        _expect(1, lambda: fn(scale=0))           # kv_scale NULL
        _expect(3, lambda: fn(scale=P16 + 4))     # kv_scale misaligned
    for fn in (dec, absorb):
        _expect(1, lambda: fn(off=0))             # row_offsets NULL
        _expect(1, lambda: fn(rows=0))            # no cache rows
    for fn in (dec_paged, absorb_paged):
        _expect(1, lambda: fn(page=48))           # page size not a power of two
    _expect(4, lambda: dec(splits=4097))
    _expect(3, lambda: dec(cache=P16 + 8))


def test_paginate_layout():
    """The paged layout helper: every sequence's rows land on distinct pages of
    its own, the gather through the block table gives the packed rows back,
    and the rest of the paged cache is NaN."""
    import numpy as np
    from head_latent_attention_12_amd import synthetic as syn
    inp = syn.make_inputs("small", lens=[0, 31, 32, 100, 64])
    pc = syn.paginate(inp, 32, seed=3)
    used = set()
    for b in range(inp.B):
        n = int(inp.lens[b]) + 1
        pages = set(int(p) for p in pc.block_table[b, :(n + 31) // 32])
        assert not (pages & used)
        used |= pages
        o = int(inp.row_offsets[b])
        rows = pc.cache[pc.rows_of(b, n)]
        same = (rows == inp.kv_cache[o:o + n]) | (np.isnan(rows) & np.isnan(inp.kv_cache[o:o + n]))
        assert same.all()
    mask = np.ones(pc.cache.shape[0], bool)
    for b in range(inp.B):
        mask[pc.rows_of(b, int(inp.lens[b]) + 1)] = False
    assert np.isnan(pc.cache[mask]).all()
    assert pc.block_table.min() >= 0 and pc.block_table.max() < pc.total_pages


def test_kv_down_argument_checks():
    """mla_kv_down: bf16 only, d_model a multiple of 512, eps >= 0, no NULLs;
    the workspace holds one fp32 partial per (512-input chunk, sequence,
    output feature)."""
    d = dsv2()
    assert mla.mla_kv_down_workspace_size(d, 5120) == 10 * 16 * 576 * 4
    _expect(2, mla.mla_kv_down_workspace_size, d, 1000)
    _expect(2, mla.mla_kv_down, d, 768, P16, P16, P16, P16, 1e-6, P16, P16, P16, 0)
    _expect(1, mla.mla_kv_down, d, 512, 0, P16, P16, P16, 1e-6, P16, P16, P16, 0)
    _expect(1, mla.mla_kv_down, d, 512, P16, P16, P16, P16, 1e-6, 0, P16, P16, 0)
    _expect(1, mla.mla_kv_down, d, 512, P16, P16, P16, P16, -1.0, P16, P16, P16, 0)
    f = mla.make_dims(8, 16, 64, 64, 64, 32, mla.MLA_F32)
    _expect(2, mla.mla_kv_down, f, 512, P16, P16, P16, P16, 1e-6, P16, P16, P16, 0)


def test_fold_argument_checks():
    """Folded projections: bf16 only, d_c_q a multiple of 256, d_model a
    multiple of 64, no NULL or misaligned pointers; the output product's
    workspace holds one fp32 partial per (k group, sequence, output) of a
    batch slice of up to 64 sequences.  k groups at H 128, r 512 (K 65536),
    from the plan with the fewest estimated bytes per compute unit: B 16,
    d_model 5120 -> 160-row blocks, 32 of them, 8 groups of 8192 (one
    work-group per compute unit); B 100, d_model 256 -> slices of 64 and 36
    sequences, 128-row blocks, 64 groups of 1024 (the 16-tile minimum)."""
    d = dsv2()
    assert mla.mla_out_folded_workspace_size(d, 5120) == 8 * 16 * 5120 * 4
    assert mla.mla_out_folded_workspace_size(mla.make_dims(100, 128, 128, 128, 512, 64, mla.MLA_BF16), 256) \
        == 64 * 64 * 256 * 4
    _expect(2, mla.mla_out_folded_workspace_size, d, 100)
    _expect(1, mla.mla_out_folded_workspace_size, d, 0)
    _expect(2, mla.mla_fold_query, d, 1000, P16, P16, P16, 0)           # d_c_q not a multiple of 256
    _expect(1, mla.mla_fold_query, d, 0, P16, P16, P16, 0)
    _expect(1, mla.mla_fold_query, d, 1536, 0, P16, P16, 0)
    _expect(3, mla.mla_fold_query, d, 1536, P16, P16 + 2, P16, 0)
    _expect(2, mla.mla_fold_output, d, 5000, P16, P16, P16, 0)          # d_model not a multiple of 64
    _expect(1, mla.mla_fold_output, d, 5120, P16, 0, P16, 0)
    _expect(3, mla.mla_fold_output, d, 5120, P16, P16, P16 + 8, 0)
    _expect(1, mla.mla_absorb_q_folded, d, 1536, P16, P16, 0, 0)
    _expect(2, mla.mla_absorb_q_folded, d, 96, P16, P16, P16, 0)
    _expect(1, mla.mla_out_folded, d, 5120, P16, P16, 0, P16, 0)        # workspace NULL
    _expect(3, mla.mla_out_folded, d, 5120, P16, P16, P16, P16 + 4, 0)
    f = mla.make_dims(8, 16, 64, 64, 64, 32, mla.MLA_F32)
    _expect(2, mla.mla_fold_query, f, 256, P16, P16, P16, 0)
    _expect(2, mla.mla_out_folded, f, 512, P16, P16, P16, P16, 0)


def test_kv_down_noalloc_argument_checks():
    """mla_kv_down_noalloc: the checks of mla_kv_down, and partial sums
    beyond its 4 MiB scratch refused on the host (MLA_ERR_WORKSPACE)."""
    d = dsv2()
    _expect(2, mla.mla_kv_down_noalloc, d, 768, P16, P16, P16, P16, 1e-6, P16, P16, 0)
    _expect(1, mla.mla_kv_down_noalloc, d, 512, 0, P16, P16, P16, 1e-6, P16, P16, 0)
    _expect(3, mla.mla_kv_down_noalloc, d, 512, P16, P16, P16, P16 + 2, 1e-6, P16, P16, 0)
    _expect(1, mla.mla_kv_down_noalloc, d, 512, P16, P16, P16, P16, -1.0, P16, P16, 0)
    big = mla.make_dims(256, 128, 128, 128, 512, 64, mla.MLA_BF16)
    assert mla.mla_kv_down_workspace_size(big, 8192) > 4 << 20
    _expect(4, mla.mla_kv_down_noalloc, big, 8192, P16, P16, P16, P16, 1e-6, P16, P16, 0)
    f = mla.make_dims(8, 16, 64, 64, 64, 32, mla.MLA_F32)
    _expect(2, mla.mla_kv_down_noalloc, f, 512, P16, P16, P16, P16, 1e-6, P16, P16, 0)
