"""Pins for the CPU oracle (no GPU).

Every check here ties the oracle to something other than itself: numbers the
pages print (fixtures under tests/golden/), an exact identity, a textbook or
library routine, a closed form, or brute force on tiny inputs.  Several
checks plant a mistake in the oracle and require the same comparison to
catch it, so that a loose tolerance cannot make a pin vacuous.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from head_latent_attention_12_amd import synthetic as syn
from oracle import mla_oracle as orc
from tests._util import normwise_rel, oracle_args, oracle_step

IDENTITY_TOL = 1e-12


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _rand_case(rng, H, dh, dv, r, dr, L):
    return dict(
        q_nope=rng.standard_normal((H, dh)), q_rope=rng.standard_normal((H, dr)),
        c_cached=rng.standard_normal((L, r)), krot_cached=rng.standard_normal((L, dr)),
        c_new=rng.standard_normal(r), k_rope_new=rng.standard_normal(dr),
        w_uk=rng.standard_normal((H, dh, r)) / math.sqrt(r),
        w_uv=rng.standard_normal((H, dv, r)) / math.sqrt(r),
        scale=1.0 / math.sqrt(dh + dr), base=10000.0)


# ---------------------------------------------------------------------------
# Cache-size formulas against the pages' printed values
# ---------------------------------------------------------------------------


def test_cache_table_by_heads(golden_dir):
    g = _load(golden_dir, "cache_table_by_heads.json")
    for row in g["rows"]:
        d_head = row["mha"] // (2 * row["n_heads"])
        assert d_head == 64
        assert orc.cache_values_mha(row["n_heads"], 64) == row["mha"]
        assert orc.cache_values_gqa(row["kv_heads"], 64) == row["gqa"]
        assert row["n_heads"] == 4 * row["kv_heads"]
        # the MLA column does not move with the head count
        assert orc.cache_values_mla(64, 16) == row["mla"]


def test_cache_training_table(golden_dir):
    g = _load(golden_dir, "cache_training_table.json")
    d_head = g["hidden"] // g["n_heads"]
    assert orc.cache_values_mha(g["n_heads"], d_head) == g["cache_per_token"]["mha"]
    assert orc.cache_values_gqa(g["gqa_kv_heads"], d_head) == g["cache_per_token"]["gqa"]
    assert g["cache_per_token"]["mha"] / g["cache_per_token"]["mla"] == pytest.approx(g["mha_over_mla"])


def test_deepseek_v2_cache(golden_dir):
    g = _load(golden_dir, "deepseek_v2_cache.json")
    mla = orc.cache_values_mla(g["r_kv"], g["d_rope"])
    mha = orc.cache_values_mha(g["n_heads"], g["d_head"])
    assert mla == g["mla_values"] == 576
    assert mha == g["mha_values"]
    assert round(mha / mla) == g["saving_rounded"]
    assert mha / g["r_kv"] == g["latent_only_ratio"]
    assert round(100.0 * (1.0 - mla / mha), 1) == g["reduction_percent_1dp"]


def test_gqa2_vs_mla_width256(golden_dir):
    g = _load(golden_dir, "gqa2_vs_mla_width256.json")
    d_head = g["width"] // g["n_heads"]
    assert d_head == g["d_head"]
    gqa2 = orc.cache_values_gqa(g["gqa_kv_heads"], d_head)
    mla = orc.cache_values_mla(g["mla_rank"], g["mla_rope"])
    assert gqa2 == g["gqa2_values"] and mla == g["mla_values"]
    assert gqa2 / mla == pytest.approx(g["ratio"])
    crossover = next(r for r in range(1, 1024) if orc.cache_values_mla(r, g["mla_rope"]) >= gqa2)
    assert crossover == g["crossover_rank"]
    assert orc.cache_values_mha(1, g["wide_model"]["width"]) == g["wide_model"]["mha_values"]


def test_workload_shapes_match_pages(golden_dir):
    g = _load(golden_dir, "hyperparameters.json")
    s, d = g["small"], g["deepseek_v2"]
    w = syn.WORKLOADS["small"]
    assert (w["H"], w["d_head"], w["r"], w["d_rope"]) == (s["n_heads"], s["d_head"], s["d_c_kv"], s["d_head_rope"])
    assert s["n_heads"] * s["d_head"] == s["d_kv_full"]
    for name in ("dsv2", "dsv2_ragged", "dsv2_long"):
        w = syn.WORKLOADS[name]
        assert (w["H"], w["d_head"], w["d_v"], w["r"], w["d_rope"]) == (
            d["n_heads"], d["d_head"], d["d_head"], d["d_c_kv"], d["d_head_rope"])
        assert orc.cache_values_mla(w["r"], w["d_rope"]) == 576


def test_append_grows_cache_by_one_row(golden_dir):
    g = _load(golden_dir, "shape_trace.json")
    rng = np.random.default_rng(5)
    B, L, r, dr = g["B"], g["prefill_len"], g["d_c"], 8
    caches = [(rng.standard_normal((L, r)), rng.standard_normal((L, dr))) for _ in range(B)]
    shape = [B] + list(caches[0][0].shape)
    assert shape == g["cache_after_prefill"]
    grown = [orc.append(c, k, rng.standard_normal(r), rng.standard_normal(dr), 10000.0) for c, k in caches]
    assert [B] + list(grown[0][0].shape) == g["cache_after_one_decode_step"]
    for (c0, k0), (c1, k1) in zip(caches, grown):
        np.testing.assert_array_equal(c1[:L], c0)      # old rows untouched
        np.testing.assert_array_equal(k1[:L], k0)
        assert k1.shape == (L + 1, dr)


def test_appended_row_layout():
    rng = np.random.default_rng(6)
    c, k = rng.standard_normal(8), rng.standard_normal(4)
    row = orc.appended_row(c, k, 0, 10000.0)          # position 0: no rotation
    np.testing.assert_array_equal(row, np.concatenate([c, k]))


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(7).standard_normal((3, 16))
    np.testing.assert_array_equal(orc.rope(x, 0, 10000.0), x)


def test_rope_worked_values():
    # pair 0 always has frequency 1: position 1 turns it by exactly 1 radian
    x0, x1 = 0.3, -1.7
    got = orc.rope(np.array([x0, x1]), 1, 10000.0)
    assert got[0] == pytest.approx(x0 * math.cos(1.0) - x1 * math.sin(1.0), abs=1e-15)
    assert got[1] == pytest.approx(x0 * math.sin(1.0) + x1 * math.cos(1.0), abs=1e-15)
    # d=4, base 10000: pair 1 has frequency 10000**(-1/2) = 0.01, so position
    # 100 turns dims (2, 3) by 1 radian and dims (0, 1) by 100 radians
    e = np.eye(4)
    r2 = orc.rope(e[2], 100, 10000.0)
    np.testing.assert_allclose(r2, [0, 0, math.cos(1.0), math.sin(1.0)], atol=1e-13)
    r0 = orc.rope(e[0], 100, 10000.0)
    np.testing.assert_allclose(r0, [math.cos(100.0), math.sin(100.0), 0, 0], atol=1e-13)
    # adjacent pairing: dim 0 never leaks into the upper half (it would if the
    # halves (i, i + d/2) were paired instead)
    r = orc.rope(np.eye(8)[0], 3, 10000.0)
    assert np.all(r[2:] == 0) and r[1] != 0


def test_rope_is_a_rotation():
    rng = np.random.default_rng(8)
    for d in (2, 16, 64):
        x = rng.standard_normal(d)
        for pos in (1, 17, 4096, 131072):
            y = orc.rope(x, pos, 10000.0)
            assert np.linalg.norm(y) == pytest.approx(np.linalg.norm(x), rel=1e-13)
        # as a matrix: orthogonal with determinant 1
        R = np.stack([orc.rope(e, 37, 10000.0) for e in np.eye(d)], axis=1)
        np.testing.assert_allclose(R.T @ R, np.eye(d), atol=1e-13)
        assert np.linalg.det(R) == pytest.approx(1.0, abs=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    for m, n in ((5, 2), (100, 99), (4096, 17), (3, 3)):
        lhs = orc.rope(q, m, 10000.0) @ orc.rope(k, n, 10000.0)
        rhs = orc.rope(q, m - n, 10000.0) @ k
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-11)


def test_rope_does_not_commute_with_projection():
    """Counterexample: RoPE on the rebuilt content key defeats absorption."""
    rng = np.random.default_rng(10)
    dh, r, L = 8, 6, 5
    w_uk = rng.standard_normal((dh, r))
    q = rng.standard_normal(dh)
    c = rng.standard_normal((L, r))
    true, folded = orc.rope_through_projection_scores(q, w_uk, c, q_pos=L, k_pos=np.arange(L), base=10000.0)
    assert np.max(np.abs(true - folded)) > 1e-2
    # without any rotation the same fold is exact
    true0, folded0 = orc.rope_through_projection_scores(q, w_uk, c, q_pos=0, k_pos=np.zeros(L), base=10000.0)
    np.testing.assert_allclose(true0, folded0, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Softmax
# ---------------------------------------------------------------------------


def test_softmax_brute_force():
    rng = np.random.default_rng(11)
    for n in (1, 2, 7, 50):
        s = rng.uniform(-29, 29, n)
        e = [math.exp(v) for v in s]
        tot = math.fsum(e)
        np.testing.assert_allclose(orc.softmax(s), [v / tot for v in e], rtol=1e-13, atol=0)
        assert math.fsum(orc.softmax(s)) == pytest.approx(1.0, abs=1e-14)
        np.testing.assert_allclose(orc.softmax(s + 123.0), orc.softmax(s), rtol=1e-12)
        assert orc.logsumexp(s) == pytest.approx(math.log(tot), rel=1e-14)


def test_softmax_large_logits_no_overflow():
    p = orc.softmax(np.array([1000.0, 1000.0, 999.0]))
    assert np.all(np.isfinite(p)) and p[0] == pytest.approx(p[1])


# ---------------------------------------------------------------------------
# The absorption identity (naive == absorbed) and its sensitivity
# ---------------------------------------------------------------------------


def _both(case):
    naive = orc.naive_decode_seq(**case)
    absorbed = orc.absorbed_decode_seq(**case)["out"]
    return naive, absorbed


def test_identity_tiny_shapes():
    rng = np.random.default_rng(12)
    for H, r, dr, L, dh, dv in itertools.product((1, 2, 3), (4, 8), (2, 4), (0, 1, 5), (3, 4), (2, 5)):
        naive, absorbed = _both(_rand_case(rng, H, dh, dv, r, dr, L))
        assert normwise_rel(absorbed, naive) <= IDENTITY_TOL, (H, r, dr, L, dh, dv)


@pytest.mark.parametrize("name,override", [
    ("tiny", {}),
    ("small", {}),
    ("dsv2", dict(lens=[257])),          # one DeepSeek-V2-shaped sequence
])
def test_identity_on_workloads(name, override):
    step = syn.make_inputs(name, **override)
    ids = [0, step.B - 1] if step.B > 1 else [0]
    naive = oracle_step(step, form="naive", batch_ids=ids)
    absorbed = oracle_step(step, batch_ids=ids)["out"]
    assert normwise_rel(absorbed, naive) <= IDENTITY_TOL


def test_identity_detects_planted_mistakes(monkeypatch):
    """The same comparison must flag a genuine difference (several kinds)."""
    rng = np.random.default_rng(13)
    case = _rand_case(rng, 3, 8, 8, 16, 4, 9)
    naive = orc.naive_decode_seq(**case)
    # a slightly wrong W_UK entry in the absorbed path only
    bad = dict(case, w_uk=case["w_uk"].copy())
    bad["w_uk"][1, 2, 3] += 1e-3
    assert normwise_rel(orc.absorbed_decode_seq(**bad)["out"], naive) > 1e3 * IDENTITY_TOL
    # a slightly wrong W_UV entry
    bad = dict(case, w_uv=case["w_uv"].copy())
    bad["w_uv"][0, 1, 2] += 1e-3
    assert normwise_rel(orc.absorbed_decode_seq(**bad)["out"], naive) > 1e3 * IDENTITY_TOL
    # the RoPE term dropped from the score
    bad = dict(case, q_rope=np.zeros_like(case["q_rope"]))
    assert normwise_rel(orc.absorbed_decode_seq(**bad)["out"], naive) > 1e3 * IDENTITY_TOL
    # the query rotated to the wrong position (off by one)
    real_rope = orc.rope
    monkeypatch.setattr(orc, "rope", lambda x, pos, base, dtype=np.float64: real_rope(x, pos + 1, base, dtype))
    shifted = orc.absorbed_decode_seq(**case)["out"]
    monkeypatch.setattr(orc, "rope", real_rope)
    assert normwise_rel(shifted, naive) > 1e3 * IDENTITY_TOL


def test_naive_matches_library_attention():
    """Per head, the naive form is plain scaled-dot-product attention."""
    rng = np.random.default_rng(14)
    H, dh, dv, r, dr, L = 4, 8, 6, 12, 4, 10
    case = _rand_case(rng, H, dh, dv, r, dr, L)
    out = orc.naive_decode_seq(**case)
    C = np.vstack([case["c_cached"], case["c_new"]])
    KR = np.vstack([case["krot_cached"], orc.rope(case["k_rope_new"], L, 10000.0)])
    for h in range(H):
        K = np.hstack([C @ case["w_uk"][h].T, KR])
        V = C @ case["w_uv"][h].T
        q = np.concatenate([case["q_nope"][h], orc.rope(case["q_rope"][h], L, 10000.0)])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None, :], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], scale=case["scale"])
        np.testing.assert_allclose(out[h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------


def test_single_row_gives_projected_new_latent():
    rng = np.random.default_rng(15)
    case = _rand_case(rng, 3, 5, 4, 8, 4, 0)             # empty cache: only the new row
    res = orc.absorbed_decode_seq(**case)
    for h in range(3):
        np.testing.assert_allclose(res["out"][h], case["w_uv"][h] @ case["c_new"], rtol=1e-13)
    np.testing.assert_allclose(orc.naive_decode_seq(**case), res["out"], rtol=1e-13)


def test_zero_query_gives_mean_latent():
    rng = np.random.default_rng(16)
    case = _rand_case(rng, 2, 6, 5, 8, 4, 7)
    case.update(q_nope=np.zeros((2, 6)), q_rope=np.zeros((2, 4)))
    res = orc.absorbed_decode_seq(**case)
    mean_c = np.vstack([case["c_cached"], case["c_new"]]).mean(axis=0)
    np.testing.assert_allclose(res["o_lat"], np.tile(mean_c, (2, 1)), rtol=1e-13)
    np.testing.assert_allclose(res["lse"], math.log(8.0), rtol=1e-14)
    for h in range(2):
        np.testing.assert_allclose(res["out"][h], case["w_uv"][h] @ mean_c, rtol=1e-12)


def test_identical_latents_ignore_weights():
    rng = np.random.default_rng(17)
    case = _rand_case(rng, 2, 6, 5, 8, 4, 6)
    case["c_cached"] = np.tile(case["c_new"], (6, 1))     # every latent equal, RoPE keys differ
    res = orc.absorbed_decode_seq(**case)
    for h in range(2):
        np.testing.assert_allclose(res["out"][h], case["w_uv"][h] @ case["c_new"], rtol=1e-12)


def test_zero_w_uk_is_position_only_attention():
    rng = np.random.default_rng(18)
    case = _rand_case(rng, 2, 6, 5, 8, 4, 6)
    case["w_uk"] = np.zeros_like(case["w_uk"])
    a = orc.absorbed_decode_seq(**case)["out"]
    b = orc.absorbed_decode_seq(**dict(case, q_nope=rng.standard_normal((2, 6))))["out"]
    np.testing.assert_allclose(a, b, rtol=1e-14)
    # and with equal RoPE keys on top, attention is uniform
    case["krot_cached"] = np.tile(orc.rope(case["k_rope_new"], 6, 10000.0), (6, 1))
    res = orc.absorbed_decode_seq(**case)
    mean_c = np.vstack([case["c_cached"], case["c_new"]]).mean(axis=0)
    np.testing.assert_allclose(res["o_lat"], np.tile(mean_c, (2, 1)), rtol=1e-12)


def test_shift_by_one_row_changes_result():
    """Dropping the appended row (attending T instead of T+1 rows) is visible."""
    step = syn.make_inputs("tiny")
    seqs, qn, qr, cn, kn, wuk, wuv = oracle_args(step)
    full = orc.absorbed_decode_seq(qn[0], qr[0], seqs[0][0], seqs[0][1], cn[0], kn[0],
                                   wuk, wuv, step.softmax_scale, step.rope_base)
    # attend over the cached rows only, query still at position L
    L = seqs[0][0].shape[0]
    q_t = np.stack([wuk[h].T @ qn[0, h] for h in range(step.H)])
    q_r = np.stack([orc.rope(qr[0, h], L, step.rope_base) for h in range(step.H)])
    p = orc.softmax(step.softmax_scale * (q_t @ seqs[0][0].T + q_r @ seqs[0][1].T))
    o = p @ seqs[0][0]
    assert normwise_rel(o, full["o_lat"]) > 1e-2


# ---------------------------------------------------------------------------
# The seeded generator (input side only)
# ---------------------------------------------------------------------------


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(19)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40]])
    bits = syn.bf16_bits_from_f64(x)
    y = syn.bf16_bits_to_f64(bits)
    up = syn.bf16_bits_to_f64(bits + 1)
    dn = syn.bf16_bits_to_f64(bits - 1)
    nz = x != 0
    err = np.abs(y - x)
    assert np.all(err[nz] <= np.abs(up - x)[nz]) and np.all(err[nz] <= np.abs(dn - x)[nz])
    assert y[-4] == 1.0
    assert y[-3] == 1.0                       # 1 + half an ulp: tie -> even (down)
    assert y[-2] == 1.0 + 2.0 ** -6           # 1 + 1.5 ulp: tie -> even (up)
    assert y[-1] == 1.0 + 2.0 ** -7           # just above the tie rounds up


def test_generator_layout_and_determinism():
    a = syn.make_inputs("dsv2_ragged", B=5, T=(3, 9))
    b = syn.make_inputs("dsv2_ragged", B=5, T=(3, 9))
    np.testing.assert_array_equal(a.kv_cache, b.kv_cache)
    assert np.all(a.lens >= 3) and np.all(a.lens <= 9)
    ends = a.row_offsets + a.lens + 1
    assert a.row_offsets[0] == 0 and np.all(a.row_offsets[1:] == ends[:-1]) and ends[-1] == a.total_rows
    for bi in range(a.B):
        slot = a.kv_cache[a.row_offsets[bi] + a.lens[bi]]
        assert np.all(slot == 0x7FC0)         # append slot holds NaN
        rows = a.cached_rows_f64(bi)[:, :a.r]
        np.testing.assert_allclose(np.sqrt(np.mean(rows ** 2, axis=1)), 1.0, atol=1e-2)


# ---------------------------------------------------------------------------
# latent KV production from the hidden state (W_DKV, RMSNorm, W_KR)
# ---------------------------------------------------------------------------

def test_kv_down_worked_by_hand():
    """h = (1, 2); W_DKV rows (1, 0), (0, 1), (1, 1) give x = (1, 2, 3), whose
    mean square is 14/3, so with unit gain and eps 0 the latent is
    x / sqrt(14/3) (sqrt(14/3) = 2.1602468994692865...); W_KR = (1, -1) gives
    the key -1."""
    h = np.array([[1.0, 2.0]])
    w_dkv = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    w_kr = np.array([[1.0, -1.0]])
    c, k = orc.kv_down(h, w_dkv, w_kr, np.ones(3), 0.0)
    np.testing.assert_allclose(c, [[0.46291004988627573, 0.92582009977255146, 1.38873014965882720]], rtol=1e-15)
    np.testing.assert_allclose(k, [[-1.0]], rtol=0)


def test_kv_down_invariants():
    """With eps 0 the latent does not change when h is scaled (RMSNorm is
    scale invariant) while the key scales with it (linear); with unit gain the
    latent has unit mean square; with a gain g and eps > 0, (c/g) has mean
    square ms / (ms + eps) for the row's mean square ms."""
    rng = np.random.default_rng(5)
    h = rng.standard_normal((3, 40))
    w_dkv = rng.standard_normal((16, 40))
    w_kr = rng.standard_normal((4, 40))
    g = 1.0 + 0.2 * rng.standard_normal(16)
    c1, k1 = orc.kv_down(h, w_dkv, w_kr, g, 0.0)
    c3, k3 = orc.kv_down(3.0 * h, w_dkv, w_kr, g, 0.0)
    np.testing.assert_allclose(c3, c1, rtol=1e-13)
    np.testing.assert_allclose(k3, 3.0 * k1, rtol=1e-13)
    cu, _ = orc.kv_down(h, w_dkv, w_kr, np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(cu * cu, axis=-1), 1.0, rtol=1e-13)
    eps = 0.7
    ce, _ = orc.kv_down(h, w_dkv, w_kr, g, eps)
    x = h @ w_dkv.T
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean((ce / g) ** 2, axis=-1), ms / (ms + eps), rtol=1e-13)


# ---------------------------------------------------------------------------
# FP8 latent cache: the E4M3FN format and the row quantisation
# ---------------------------------------------------------------------------

def test_e4m3_values_from_the_format_definition():
    # exponent bias 7, 3 mantissa bits: a few values fixed by the definition
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, v in known.items():
        assert orc.e4m3_value(code) == v, hex(code)
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))
    assert orc.e4m3_value(0x80) == 0.0 and math.copysign(1.0, orc.e4m3_value(0x80)) == -1.0
    pos = np.array([orc.e4m3_value(c) for c in range(0x7F)])
    assert np.all(np.diff(pos) > 0)                       # 127 distinct, increasing
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)          # subnormals and the first normal evenly spaced
    neg = np.array([orc.e4m3_value(c | 0x80) for c in range(0x7F)])
    np.testing.assert_array_equal(neg, -pos)


def test_e4m3_encode_round_trip_ties_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)
    # ties go to the even code
    cases = {1.0625: 0x38, 1.1875: 0x3A, 1.5 * 2.0 ** -9: 0x02, 0.5 * 2.0 ** -9: 0x00, 2.5 * 2.0 ** -9: 0x02,
             -1.0625: 0xB8, 464.0: 0x7E, 500.0: 0x7E, 1e30: 0x7E, -1e30: 0xFE, 0.25 * 2.0 ** -9: 0x00}
    for y, code in cases.items():
        assert int(orc.e4m3_encode(np.array([y]))[0]) == code, y


def test_e4m3_encode_is_the_nearest_code():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.5, 4000),
                        rng.uniform(-448, 448, 1000)])
    got = orc.e4m3_decode(orc.e4m3_encode(y))
    finite = np.array([orc.e4m3_value(c) for c in range(256) if c not in (0x7F, 0xFF)])
    best = np.min(np.abs(y[:, None] - finite[None, :]), axis=1)  # brute force over every code
    np.testing.assert_array_equal(np.abs(got - y), best)
    assert np.all(np.sign(got) * np.sign(y) >= 0)


def test_fp8_row_exponent_and_quantised_row():
    assert orc.fp8_row_exponent(448.0) == 0
    assert orc.fp8_row_exponent(np.nextafter(448.0, 1e9)) == 1
    assert orc.fp8_row_exponent(224.0) == -1
    assert orc.fp8_row_exponent(1.0) == -8                  # 448 / 256 = 1.75 >= 1 > 448 / 512
    assert orc.fp8_row_exponent(0.0) == orc.FP8_MIN_EXP
    assert orc.fp8_row_exponent(1e300) == orc.FP8_MAX_EXP
    rng = np.random.default_rng(6)
    for amax in 10.0 ** rng.uniform(-30, 20, 200):
        e = orc.fp8_row_exponent(amax)
        assert amax <= 448.0 * 2.0 ** e and (e == orc.FP8_MIN_EXP or amax > 448.0 * 2.0 ** (e - 1))
    c = rng.standard_normal(512)
    codes, s = orc.fp8_quantize_row(c)
    deq = orc.fp8_dequantize_rows(codes[None, :], np.array([s]))[0]
    assert np.max(np.abs(deq)) <= 448.0 * s and np.max(np.abs(c)) > 224.0 * s   # the scale is tight
    # every element is its nearest code times s; normal-range errors are within half a step (2^-4 relative)
    np.testing.assert_array_equal(deq, orc.e4m3_decode(orc.e4m3_encode(c / s)) * s)
    normal = np.abs(c) >= 2.0 ** -6 * s
    assert np.all(np.abs(deq - c)[normal] <= 2.0 ** -4 * np.abs(c)[normal])


# ---------------------------------------------------------------------------
# Folded projections ("MLA from scratch", absorbing projections: W_O absorbs
# W_UV, the query side absorbs the key up-projection; octlm "What we didn't
# build, and why": the part most likely to hide a silent bug)
# ---------------------------------------------------------------------------


def _fold_case(rng, H, dh, dv, r, dr, L, dcq, dmodel):
    case = _rand_case(rng, H, dh, dv, r, dr, L)
    c_q = rng.standard_normal(dcq)
    w_uq = rng.standard_normal((H * dh, dcq)) / math.sqrt(dcq)
    w_o = rng.standard_normal((dmodel, H * dv)) / math.sqrt(H * dv)
    return case, c_q, w_uq, w_o


def _unfolded_y(case, c_q, w_uq, w_o):
    """The page's forward pass: q = W_UQ c_q per head, naive attention, W_O."""
    q_nope = orc.query_projection(c_q, w_uq, case["w_uk"].shape[0])
    out = orc.naive_decode_seq(**dict(case, q_nope=q_nope))
    return orc.output_projection(out, w_o)


def _folded(case, c_q, w_qk, w_ov):
    return orc.folded_decode_seq(c_q, case["q_rope"], case["c_cached"], case["krot_cached"], case["c_new"],
                                 case["k_rope_new"], w_qk, w_ov, case["scale"], case["base"])


def test_fold_identity_tiny_shapes():
    rng = np.random.default_rng(31)
    for H, dh, r, dr, L, dcq, dmodel in itertools.product((1, 3), (4, 8), (4, 8), (2, 4), (0, 1, 5), (6, 16), (5, 12)):
        case, c_q, w_uq, w_o = _fold_case(rng, H, dh, dh + 2, r, dr, L, dcq, dmodel)
        got = _folded(case, c_q, orc.fold_query(w_uq, case["w_uk"]), orc.fold_output(w_o, case["w_uv"]))
        assert normwise_rel(got["y"], _unfolded_y(case, c_q, w_uq, w_o)) <= IDENTITY_TOL
        q_nope = orc.query_projection(c_q, w_uq, H)
        q_ref = np.stack([case["w_uk"][h].T @ q_nope[h] for h in range(H)])
        assert normwise_rel(got["q_tilde"], q_ref) <= IDENTITY_TOL


def test_fold_identity_deepseek_v2_heads(golden_dir):
    """The DeepSeek-V2 head dims of the page's hyperparameter block (H 128,
    d_head 128, r 512, d_rope 64, d_c' 1536); d_model is cut to 256 here
    (5120 would make a 2.7 GB fp64 folded output matrix in a CPU test)."""
    hp = _load(golden_dir, "hyperparameters.json")["deepseek_v2"]
    rng = np.random.default_rng(32)
    H, dh, r, dr, dcq = hp["n_heads"], hp["d_head"], hp["d_c_kv"], hp["d_head_rope"], hp["d_c_q"]
    case, c_q, w_uq, w_o = _fold_case(rng, H, dh, dh, r, dr, 16, dcq, 256)
    w_qk, w_ov = orc.fold_query(w_uq, case["w_uk"]), orc.fold_output(w_o, case["w_uv"])
    assert w_qk.shape == (H, r, dcq) and w_ov.shape == (256, H * r)
    got = _folded(case, c_q, w_qk, w_ov)
    assert normwise_rel(got["y"], _unfolded_y(case, c_q, w_uq, w_o)) <= IDENTITY_TOL


def test_fold_entries_brute_force():
    """Every folded entry is the sum its definition states, added up with
    math.fsum over the shared index (no matrix product)."""
    rng = np.random.default_rng(33)
    H, dh, dv, r, dcq, dmodel = 2, 3, 4, 5, 6, 7
    w_uk = rng.standard_normal((H, dh, r))
    w_uv = rng.standard_normal((H, dv, r))
    w_uq = rng.standard_normal((H * dh, dcq))
    w_o = rng.standard_normal((dmodel, H * dv))
    w_qk, w_ov = orc.fold_query(w_uq, w_uk), orc.fold_output(w_o, w_uv)
    for h in range(H):
        for j in range(r):
            for i in range(dcq):
                ref = math.fsum(w_uk[h, d, j] * w_uq[h * dh + d, i] for d in range(dh))
                assert w_qk[h, j, i] == pytest.approx(ref, rel=1e-13, abs=1e-13)
            for m in range(dmodel):
                ref = math.fsum(w_o[m, h * dv + d] * w_uv[h, d, j] for d in range(dv))
                assert w_ov[m, h * r + j] == pytest.approx(ref, rel=1e-13, abs=1e-13)


def test_fold_closed_forms():
    """W_O = identity turns the folded output into the heads' outputs
    concatenated; W_UQ made of identity blocks turns the folded query into
    W_UK^T applied to c_q in every head (the absorbed form's q~)."""
    rng = np.random.default_rng(34)
    H, dh, dv, r, dr, L = 3, 8, 8, 8, 4, 6
    case, c_q, _, _ = _fold_case(rng, H, dh, dv, r, dr, L, dh, H * dv)
    w_uq = np.vstack([np.eye(dh)] * H)
    w_o = np.eye(H * dv)
    got = _folded(case, c_q, orc.fold_query(w_uq, case["w_uk"]), orc.fold_output(w_o, case["w_uv"]))
    ref = orc.absorbed_decode_seq(**dict(case, q_nope=np.stack([c_q] * H)))
    assert normwise_rel(got["y"], ref["out"].reshape(-1)) <= IDENTITY_TOL
    assert normwise_rel(got["q_tilde"], ref["q_lat"][:, :r]) <= IDENTITY_TOL


def test_fold_detects_planted_mistakes():
    """The identity comparison must flag a wrong fold: a perturbed weight in
    the folded path only, head blocks taken from the wrong rows or columns,
    and the page's literal shape (the heads summed before the fold)."""
    rng = np.random.default_rng(35)
    H, dh, dv, r, dr, L, dcq, dmodel = 3, 8, 8, 8, 4, 9, 8, 10
    case, c_q, w_uq, w_o = _fold_case(rng, H, dh, dv, r, dr, L, dcq, dmodel)
    ref = _unfolded_y(case, c_q, w_uq, w_o)
    w_qk, w_ov = orc.fold_query(w_uq, case["w_uk"]), orc.fold_output(w_o, case["w_uv"])
    assert normwise_rel(_folded(case, c_q, w_qk, w_ov)["y"], ref) <= IDENTITY_TOL

    def flagged(qk, ov):
        return normwise_rel(_folded(case, c_q, qk, ov)["y"], ref) > 1e3 * IDENTITY_TOL

    bad = w_uq.copy()
    bad[1 * dh + 2, 3] += 1e-3
    assert flagged(orc.fold_query(bad, case["w_uk"]), w_ov)
    bad = w_o.copy()
    bad[4, 2 * dv + 1] += 1e-3
    assert flagged(w_qk, orc.fold_output(bad, case["w_uv"]))
    bad = case["w_uv"].copy()
    bad[0, 1, 2] += 1e-3
    assert flagged(w_qk, orc.fold_output(w_o, bad))
    # head h's query rows taken as rows h, h+H, ... (interleaved, not blocks)
    inter = np.vstack([w_uq[h::H] for h in range(H)])
    assert flagged(orc.fold_query(inter, case["w_uk"]), w_ov)
    # head h's W_O columns taken interleaved
    inter = np.hstack([w_o[:, h::H] for h in range(H)])
    assert flagged(w_qk, orc.fold_output(inter, case["w_uv"]))
    # one (d_model, r) matrix for all heads applied to the summed latents
    summed = sum(w_o[:, h * dv:(h + 1) * dv] @ case["w_uv"][h] for h in range(H))
    o_lat = _folded(case, c_q, w_qk, w_ov)["o_lat"]
    assert normwise_rel(summed @ o_lat.sum(axis=0), ref) > 1e3 * IDENTITY_TOL


def test_identity_error_order_in_float32(golden_dir):
    """'DeepSeek MLA, Built From the Paper' section 3 prints max|naive -
    absorbed| = 2.38e-07 without shapes or dtype; 2^-22 is a float32-sized
    gap.  Both forms evaluated in float32 at the page's lab shape (8 heads of
    32, rank 64 plus a 16-wide RoPE key, the tiny workload's inputs) differ by
    that order, and in float64 by none of it."""
    g = _load(golden_dir, "identity_error.json")
    step = syn.make_inputs("tiny")
    seqs, qn, qr, cn, kn, wuk, wuv = oracle_args(step)
    args = (qn[0], qr[0], seqs[0][0], seqs[0][1], cn[0], kn[0], wuk, wuv, step.softmax_scale, step.rope_base)
    f32 = np.abs(orc.naive_decode_seq(*args, dtype=np.float32)
                 - orc.absorbed_decode_seq(*args, dtype=np.float32)["out"]).max()
    f64 = np.abs(orc.naive_decode_seq(*args) - orc.absorbed_decode_seq(*args)["out"]).max()
    page = g["max_abs_naive_minus_absorbed"]
    assert page / 30 <= f32 <= page * 30, f32
    assert f64 <= 1e-13
