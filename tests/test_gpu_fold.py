"""GPU parity of the folded projections ("MLA from scratch", absorbing
projections; octlm "What we didn't build, and why") against the fp64 oracle.

The folded weights are checked entry by entry against the oracle's fp64 fold:
one bf16 rounding of an fp32 sum over d_head (or d_v) terms, so
|gpu - fold| <= 2^-8 |fold| + 2^-16 fold_abs, with fold_abs the same fold of
the weights' absolute values (a bound on the fp32 accumulation error that
holds however much the terms cancel).

The folded step (mla_absorb_q_folded, mla_rope_append, mla_decode_latent,
mla_combine, mla_out_folded) is checked against the page's unfolded forward
pass in fp64: q = W_UQ c_q per head, attention (the absorbed form, pinned to
the naive one; the naive form itself at a reduced size), W_O over the
concatenated heads.  q~ = W_QK c_q carries the rounding of the folded weight
on top of its own: |gpu - q~| <= 2^-8 |q~| + 2^-8 (W_QK_abs |c_q|).  The
output y gets the bf16 gates and the tighter bounds of the step tests.
"""
import numpy as np
import pytest
import torch

from head_latent_attention_12_amd import synthetic as syn
from oracle import mla_oracle as orc
from tests._util import oracle_args

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 5e-3
TIGHT_MAX_REL, TIGHT_MEAN_REL = 1e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_12_amd import mla
    mla.lib()  # fail loudly if the HIP library is missing


def _dev(a):
    from head_latent_attention_12_amd.step import _dev as dev
    return dev(a, "cuda")


def _bits(t):
    return syn.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))


def folded_step(inp, fin, num_splits=None):
    """The folded step on the GPU: fold both weights, then absorb_q_folded,
    rope_append, decode_latent, combine, out_folded.  Returns (DeviceStep,
    w_qk, w_ov, y)."""
    from head_latent_attention_12_amd import mla
    from head_latent_attention_12_amd.step import DeviceStep
    ds = DeviceStep(inp, num_splits=num_splits)
    H, r, dcq, dm = inp.H, inp.r, fin.d_c_q, fin.d_model
    w_uq, w_o, c_q = _dev(fin.w_uq), _dev(fin.w_o), _dev(fin.c_q)
    w_qk = torch.empty((H, r, dcq), dtype=torch.int16, device="cuda")
    w_ov = torch.empty((dm, H * r), dtype=torch.int16, device="cuda")
    mla.mla_fold_query(ds.dims, dcq, w_uq, ds.w_uk, w_qk)
    mla.mla_fold_output(ds.dims, dm, w_o, ds.w_uv, w_ov)
    mla.mla_absorb_q_folded(ds.dims, dcq, c_q, w_qk, ds.q_lat)
    ds.rope_append()
    ds.decode_latent()
    ds.combine()
    ws = torch.empty(mla.mla_out_folded_workspace_size(ds.dims, dm) // 4, dtype=torch.float32, device="cuda")
    y = torch.empty((inp.B, dm), dtype=torch.float32, device="cuda")
    mla.mla_out_folded(ds.dims, dm, ds.o_lat, w_ov, ws, y)
    torch.cuda.synchronize()
    return ds, w_qk, w_ov, y


def unfolded_reference(inp, fin, form="absorbed"):
    """The page's forward pass in fp64: q_nope = W_UQ c_q, attention, W_O.
    Returns (q~ [B, H, r], y [B, d_model])."""
    seqs, _, qr, cn, kn, wuk, wuv = oracle_args(inp)
    c_q, w_uq, w_o = fin.f64("c_q"), fin.f64("w_uq"), fin.f64("w_o")
    q_t, ys = [], []
    for b in range(inp.B):
        q_nope = orc.query_projection(c_q[b], w_uq, inp.H)
        q_t.append(np.stack([wuk[h].T @ q_nope[h] for h in range(inp.H)]))
        args = (q_nope, qr[b], seqs[b][0], seqs[b][1], cn[b], kn[b], wuk, wuv, inp.softmax_scale, inp.rope_base)
        out = orc.naive_decode_seq(*args) if form == "naive" else orc.absorbed_decode_seq(*args)["out"]
        ys.append(orc.output_projection(out, w_o))
    return np.stack(q_t), np.stack(ys)


def check_fold(got, ref, ref_abs, tag):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * ref_abs
    print(f"[{tag}] max abs err {err.max():.3e}, worst err/bound {np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound), tag


def check_q(inp, fin, ds, q_ref, w_qk_abs, tag):
    got = ds.q_lat_f64()[:, :, :inp.r]
    cq_abs = np.abs(fin.f64("c_q"))
    H, r, dcq = w_qk_abs.shape
    env = (w_qk_abs.reshape(H * r, dcq) @ cq_abs.T).T.reshape(-1, H, r)
    bound = 2.0 ** -8 * np.abs(q_ref) + 2.0 ** -8 * env
    err = np.abs(got - q_ref)
    print(f"[{tag}] q~ max abs err {err.max():.3e}, worst err/bound {np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound), tag


def check_y(got, ref, tag):
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    print(f"[{tag}] y max abs {err.max():.3e} mean abs {err.mean():.3e} (max|y| {scale:.3e})", flush=True)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, tag
    assert err.max() <= TIGHT_MAX_REL * scale and err.mean() <= TIGHT_MEAN_REL * scale, tag


@pytest.fixture(scope="module")
def dsv2_fold():
    """DeepSeek-V2 batch of 16 with the page's d_c' 1536 and d_model 5120
    (cached length cut to 300 rows: the fold does not touch the cache)."""
    inp = syn.make_inputs("dsv2", T=300)
    fin = syn.make_fold_inputs(inp)
    return inp, fin, folded_step(inp, fin)


def test_fold_query_full_size(dsv2_fold):
    inp, fin, (ds, w_qk, _, _) = dsv2_fold
    w_uq, w_uk = fin.f64("w_uq"), inp.f64("w_uk")
    ref = orc.fold_query(w_uq, w_uk)
    ref_abs = orc.fold_query(np.abs(w_uq), np.abs(w_uk))
    check_fold(_bits(w_qk), ref, ref_abs, "fold_query H128 r512 d_c_q1536")


def test_fold_output_sampled_rows(dsv2_fold):
    """All heads, 256 of the 5120 output rows (seeded sample incl. the first
    and last): the oracle's fold of those rows of W_O."""
    inp, fin, (ds, _, w_ov, _) = dsv2_fold
    rows = np.unique(np.concatenate([[0, fin.d_model - 1],
                                     np.random.default_rng(5).choice(fin.d_model, 254, replace=False)]))
    w_o, w_uv = fin.f64("w_o")[rows], inp.f64("w_uv")
    ref = orc.fold_output(w_o, w_uv)
    ref_abs = orc.fold_output(np.abs(w_o), np.abs(w_uv))
    got = _bits(w_ov[torch.as_tensor(rows, device="cuda")])
    check_fold(got, ref, ref_abs, "fold_output d_model5120 (sampled rows)")


def test_folded_step_full_size(dsv2_fold):
    inp, fin, (ds, w_qk, _, y) = dsv2_fold
    q_ref, y_ref = unfolded_reference(inp, fin)
    w_qk_abs = orc.fold_query(np.abs(fin.f64("w_uq")), np.abs(inp.f64("w_uk")))
    check_q(inp, fin, ds, q_ref, w_qk_abs, "folded dsv2 B16")
    check_y(y.cpu().numpy().astype(np.float64), y_ref, "folded dsv2 B16")


def test_folded_step_matches_naive_form():
    """The fold against the page's naive forward pass (K and V rebuilt per
    head) at the DeepSeek-V2 head dims, two short sequences, d_c' and d_model
    cut to 256."""
    inp = syn.make_inputs("dsv2", B=2, T=45)
    fin = syn.make_fold_inputs(inp, d_c_q=256, d_model=256, seed=22)
    _, _, _, y = folded_step(inp, fin)
    _, y_ref = unfolded_reference(inp, fin, form="naive")
    check_y(y.cpu().numpy().astype(np.float64), y_ref, "folded vs naive B2")


def test_folded_step_batch_slices_and_ragged():
    """65 ragged sequences: the folded products run in slices of 64
    sequences (the second slice has one)."""
    inp = syn.make_inputs("dsv2_ragged", B=65, T=(3, 90), seed=7)
    fin = syn.make_fold_inputs(inp, d_c_q=512, d_model=384, seed=23)
    ds, _, _, y = folded_step(inp, fin)
    q_ref, y_ref = unfolded_reference(inp, fin)
    w_qk_abs = orc.fold_query(np.abs(fin.f64("w_uq")), np.abs(inp.f64("w_uk")))
    check_q(inp, fin, ds, q_ref, w_qk_abs, "folded ragged B65")
    check_y(y.cpu().numpy().astype(np.float64), y_ref, "folded ragged B65")


def test_out_folded_is_deterministic(dsv2_fold):
    from head_latent_attention_12_amd import mla
    inp, fin, (ds, _, w_ov, y) = dsv2_fold
    ws = torch.empty(mla.mla_out_folded_workspace_size(ds.dims, fin.d_model) // 4, dtype=torch.float32,
                     device="cuda")
    y2 = torch.empty_like(y)
    mla.mla_out_folded(ds.dims, fin.d_model, ds.o_lat, w_ov, ws, y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_folded_step_ragged_full_size():
    """The folded step on the full ragged DeepSeek-V2 batch (64 sequences,
    lengths U[512, 8192], the planned splits) with the page's d_c' 1536 and
    d_model 5120, against the unfolded fp64 forward pass."""
    inp = syn.make_inputs("dsv2_ragged")
    fin = syn.make_fold_inputs(inp, seed=24)
    ds, w_qk, _, y = folded_step(inp, fin)
    q_ref, y_ref = unfolded_reference(inp, fin)
    w_qk_abs = orc.fold_query(np.abs(fin.f64("w_uq")), np.abs(inp.f64("w_uk")))
    check_q(inp, fin, ds, q_ref, w_qk_abs, "folded dsv2_ragged B64")
    check_y(y.cpu().numpy().astype(np.float64), y_ref, "folded dsv2_ragged B64")


@pytest.mark.parametrize("B", [5, 24, 40])
def test_folded_products_small_shapes(B):
    """mla_absorb_q_folded and mla_out_folded alone at the DeepSeek-V2 head
    dims with d_c' 256 and d_model 320 (not a multiple of 128: the output
    product's 64-row work-groups) and a batch whose X tiles hold 16, 32 and 64
    rows (one or two 32-column blocks).  q~ against the oracle's fold of
    W_UQ and W_UK applied to c_q (the bound of check_q); y against the fp64
    product of the kernel's own folded weight with o_lat: the only error left
    is fp32 o_lat entering the bf16 MFMA as a high and a low part (a residual
    below 2^-17 of each value) and fp32 accumulation, well inside 2^-12 of
    |W_OV| |o_lat|."""
    from head_latent_attention_12_amd import mla
    inp = syn.make_inputs("dsv2", B=B, T=4, seed=31)
    H, r, dh, dcq, dm = inp.H, inp.r, inp.d_head, 256, 320
    fin = syn.make_fold_inputs(inp, d_c_q=dcq, d_model=dm, seed=32)
    dims = mla.make_dims(B, H, dh, dh, r, inp.d_rope, mla.MLA_BF16, inp.softmax_scale, inp.rope_base)
    w_uq, w_uk, w_o, w_uv, c_q = (_dev(fin.w_uq), _dev(inp.w_uk), _dev(fin.w_o), _dev(inp.w_uv), _dev(fin.c_q))
    w_qk = torch.empty((H, r, dcq), dtype=torch.int16, device="cuda")
    w_ov = torch.empty((dm, H * r), dtype=torch.int16, device="cuda")
    mla.mla_fold_query(dims, dcq, w_uq, w_uk, w_qk)
    mla.mla_fold_output(dims, dm, w_o, w_uv, w_ov)
    q_lat = torch.zeros((B, H, r + inp.d_rope), dtype=torch.int16, device="cuda")
    mla.mla_absorb_q_folded(dims, dcq, c_q, w_qk, q_lat)
    o_lat = torch.as_tensor(np.random.default_rng(33).standard_normal((B, H, r)), dtype=torch.float32).cuda()
    ws = torch.empty(mla.mla_out_folded_workspace_size(dims, dm) // 4, dtype=torch.float32, device="cuda")
    y = torch.empty((B, dm), dtype=torch.float32, device="cuda")
    mla.mla_out_folded(dims, dm, o_lat, w_ov, ws, y)
    torch.cuda.synchronize()

    cq, wuq, wuk = fin.f64("c_q"), fin.f64("w_uq"), inp.f64("w_uk")
    q_ref = np.stack([np.stack([wuk[h].T @ qn[h] for h in range(H)])
                      for qn in (orc.query_projection(cq[b], wuq, H) for b in range(B))])
    w_qk_abs = orc.fold_query(np.abs(wuq), np.abs(wuk))
    env = (w_qk_abs.reshape(H * r, dcq) @ np.abs(cq).T).T.reshape(B, H, r)
    got_q = _bits(q_lat)[:, :, :r]
    err_q = np.abs(got_q - q_ref)
    assert np.all(err_q <= 2.0 ** -8 * np.abs(q_ref) + 2.0 ** -8 * env), f"q~ B{B}"
    assert np.all(_bits(q_lat)[:, :, r:] == 0), "the RoPE columns are not the folded product's"

    w = _bits(w_ov)
    x = o_lat.cpu().numpy().astype(np.float64).reshape(B, H * r)
    y_ref = x @ w.T
    env_y = np.abs(x) @ np.abs(w).T
    err_y = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    print(f"[small folded B{B}] q~ worst err/bound "
          f"{np.max(err_q / (2.0 ** -8 * np.abs(q_ref) + 2.0 ** -8 * env)):.3f}, "
          f"y max err / envelope {np.max(err_y / env_y):.2e}", flush=True)
    assert np.all(err_y <= 2.0 ** -12 * env_y), f"y B{B}"


def test_folded_products_graph_replay():
    """mla_absorb_q_folded and mla_out_folded (its split-k partial sums in the
    caller's workspace, then the fixed-order reduction) recorded as one HIP
    graph: every replay, with eager work on the outputs and the workspace and
    synchronisation between replays, reproduces the eager bits."""
    from head_latent_attention_12_amd import mla
    B, dcq, dm = 24, 512, 320
    inp = syn.make_inputs("dsv2", B=B, T=4, seed=34)
    fin = syn.make_fold_inputs(inp, d_c_q=dcq, d_model=dm, seed=35)
    H, r = inp.H, inp.r
    dims = mla.make_dims(B, H, inp.d_head, inp.d_v, r, inp.d_rope, mla.MLA_BF16, inp.softmax_scale, inp.rope_base)
    w_uq, w_uk, w_o, w_uv, c_q = (_dev(fin.w_uq), _dev(inp.w_uk), _dev(fin.w_o), _dev(inp.w_uv), _dev(fin.c_q))
    w_qk = torch.empty((H, r, dcq), dtype=torch.int16, device="cuda")
    w_ov = torch.empty((dm, H * r), dtype=torch.int16, device="cuda")
    mla.mla_fold_query(dims, dcq, w_uq, w_uk, w_qk)
    mla.mla_fold_output(dims, dm, w_o, w_uv, w_ov)
    q_lat = torch.zeros((B, H, r + inp.d_rope), dtype=torch.int16, device="cuda")
    o_lat = torch.as_tensor(np.random.default_rng(36).standard_normal((B, H, r)), dtype=torch.float32).cuda()
    ws = torch.empty(mla.mla_out_folded_workspace_size(dims, dm) // 4, dtype=torch.float32, device="cuda")
    y = torch.empty((B, dm), dtype=torch.float32, device="cuda")

    def products():
        mla.mla_absorb_q_folded(dims, dcq, c_q, w_qk, q_lat)
        mla.mla_out_folded(dims, dm, o_lat, w_ov, ws, y)

    products()
    torch.cuda.synchronize()
    eager_q, eager_y = q_lat.clone(), y.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        products()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        products()
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        ws.fill_(float("nan"))
        q_lat.fill_(-1)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(y, eager_y), f"replay {rep}: y differs from the eager run"
        assert torch.equal(q_lat[:, :, :r], eager_q[:, :, :r]), f"replay {rep}: q~ differs from the eager run"
