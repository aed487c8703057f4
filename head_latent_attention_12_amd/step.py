"""One decode step on the GPU: upload seeded inputs, run the C-ABI calls.

Marshalling only: buffers are torch tensors (device memory), every step of
the computation runs in libmla.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import mla
from .synthetic import BF16, Fp8Cache, PagedCache, StepInputs, make_fp8_cache, paginate


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits_to_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor in storage form -> fp64 numpy."""
    a = t.detach().cpu().numpy()
    if dtype == BF16:
        return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class DeviceStep:
    """Device buffers of one step and the calls that compute it: absorb_q,
    rope_append, decode_latent, combine and up_v.  ``run`` issues them as
    absorb_rope, decode_latent and combine_up_v (the fused entry points); the
    separate calls stay available."""

    def __init__(self, inp: StepInputs, num_splits: int | None = None, device: str = "cuda:0",
                 weights: "DeviceStep | None" = None, scratch: "DeviceStep | None" = None,
                 page_rows: int | None = None, page_seed: int = 0, fp8: bool = False, fp8_seed: int = 3,
                 max_seq_len: int | None = None):
        """``weights``: share W_UK/W_UV with another step (same layer).
        ``scratch``: share the per-step temporaries (q_lat, split partials,
        o_lat, lse, out) with another step of the same shape, as successive
        layers of one decode step would.  ``page_rows``: keep the cache in
        pages of that many rows behind a block table (the paged calls).
        ``fp8``: keep the cache in the fp8 row layout (codes drawn with
        ``fp8_seed``, the fp8 calls).  ``num_splits`` None: the planner's split
        count and max_seq_len; given: that count with ``max_seq_len`` (default
        the longest length), which together fix the splits' rows."""
        self.inp = inp
        self.device = device
        self.dims = mla.make_dims(inp.B, inp.H, inp.d_head, inp.d_v, inp.r, inp.d_rope,
                                  mla.MLA_BF16 if inp.dtype == BF16 else mla.MLA_F32,
                                  inp.softmax_scale, inp.rope_base)
        st = torch.int16 if inp.dtype == BF16 else torch.float32
        if weights is None:
            self.w_uk = _dev(inp.w_uk, device)
            self.w_uv = _dev(inp.w_uv, device)
        else:  # share weights with another step (e.g. several caches, one layer)
            self.w_uk, self.w_uv = weights.w_uk, weights.w_uv
        self.q_nope = _dev(inp.q_nope, device)
        self.q_rope = _dev(inp.q_rope, device)
        self.paged: PagedCache | None = None
        self.fp8: Fp8Cache | None = make_fp8_cache(inp, fp8_seed) if fp8 else None
        if page_rows is None:
            self.kv_cache = _dev(self.fp8.rows if fp8 else inp.kv_cache, device)
            if fp8:
                self.kv_scale = _dev(self.fp8.scale, device)
        else:
            self.paged = paginate(inp, page_rows, seed=page_seed, fp8=self.fp8)
            self.kv_cache = _dev(self.paged.cache, device)
            self.block_table = _dev(self.paged.block_table, device)
            if fp8:
                self.kv_scale = _dev(self.paged.scale, device)
        self.c_kv_new = _dev(inp.c_kv_new, device)
        self.k_rope_new = _dev(inp.k_rope_new, device)
        self.positions = _dev(inp.positions.astype(np.int32), device)
        self.row_offsets = _dev(inp.row_offsets.astype(np.int64), device)
        self.seq_lens = _dev(inp.seq_lens.astype(np.int32), device)
        if scratch is not None:
            self.q_lat, self.o_lat, self.lse, self.out = scratch.q_lat, scratch.o_lat, scratch.lse, scratch.out
            self.num_splits, self.o_part, self.lse_part = scratch.num_splits, scratch.o_part, scratch.lse_part
            self.max_seq_len = scratch.max_seq_len
            return
        self.q_lat = torch.zeros((inp.B, inp.H, inp.W), dtype=st, device=device)
        self.set_splits(num_splits, max_seq_len)
        self.o_lat = torch.empty((inp.B, inp.H, inp.r), dtype=torch.float32, device=device)
        self.lse = torch.empty((inp.B, inp.H), dtype=torch.float32, device=device)
        self.out = torch.empty((inp.B, inp.H, inp.d_v), dtype=torch.float32, device=device)

    def set_splits(self, num_splits: int | None, max_seq_len: int | None = None) -> None:
        inp = self.inp
        # the max_seq_len passed to the decode calls: with a planned split count
        # the planner's value (at least every length), which sets the chunk
        self.max_seq_len = inp.max_seq_len if max_seq_len is None else int(max_seq_len)
        if num_splits is None:  # the lengths are known on the host here
            num_splits, self.max_seq_len = mla.mla_plan_splits_for_lengths(self.dims, inp.seq_lens)
        self.num_splits = int(num_splits)
        o_bytes, _ = mla.mla_partials_size(self.dims, self.num_splits)
        self.o_part = torch.empty((o_bytes // 4,), dtype=torch.int32, device=self.device)  # raw partials buffer
        self.lse_part = torch.empty((inp.B, self.num_splits, inp.H), dtype=torch.float32, device=self.device)

    # the calls ----------------------------------------------------------------
    def absorb_q(self, stream=None):
        self._no_fp8("absorb_q")
        mla.mla_absorb_q(self.dims, self.q_nope, self.w_uk, self.q_lat, stream)

    def _pages(self):
        pc = self.paged
        return self.block_table, pc.bt_stride, pc.page_rows, pc.total_pages

    def _no_fp8(self, call):
        if self.fp8 is not None:
            raise RuntimeError(f"{call}: the fp8 cache is written by absorb_rope (mla_absorb_rope_fp8*)")

    def rope_append(self, stream=None):
        self._no_fp8("rope_append")
        if self.paged is not None:
            mla.mla_rope_append_paged(self.dims, self.q_rope, self.c_kv_new, self.k_rope_new, self.positions,
                                      *self._pages(), self.q_lat, self.kv_cache, stream)
            return
        mla.mla_rope_append(self.dims, self.q_rope, self.c_kv_new, self.k_rope_new, self.positions,
                            self.row_offsets, self.inp.total_rows, self.q_lat, self.kv_cache, stream)

    def absorb_rope(self, stream=None):
        if self.fp8 is not None:
            if self.paged is not None:
                mla.mla_absorb_rope_fp8_paged(self.dims, self.q_nope, self.w_uk, self.q_rope, self.c_kv_new,
                                              self.k_rope_new, self.positions, *self._pages(), self.q_lat,
                                              self.kv_cache, self.kv_scale, stream)
            else:
                mla.mla_absorb_rope_fp8(self.dims, self.q_nope, self.w_uk, self.q_rope, self.c_kv_new,
                                        self.k_rope_new, self.positions, self.row_offsets, self.inp.total_rows,
                                        self.q_lat, self.kv_cache, self.kv_scale, stream)
            return
        if self.paged is not None:
            mla.mla_absorb_rope_paged(self.dims, self.q_nope, self.w_uk, self.q_rope, self.c_kv_new,
                                      self.k_rope_new, self.positions, *self._pages(), self.q_lat, self.kv_cache,
                                      stream)
            return
        mla.mla_absorb_rope(self.dims, self.q_nope, self.w_uk, self.q_rope, self.c_kv_new, self.k_rope_new,
                            self.positions, self.row_offsets, self.inp.total_rows, self.q_lat, self.kv_cache, stream)

    def decode_latent(self, stream=None):
        if self.fp8 is not None:
            if self.paged is not None:
                mla.mla_decode_latent_fp8_paged(self.dims, self.q_lat, self.kv_cache, self.kv_scale, *self._pages(),
                                                self.seq_lens, self.max_seq_len, self.num_splits, self.o_part,
                                                self.lse_part, stream)
            else:
                mla.mla_decode_latent_fp8(self.dims, self.q_lat, self.kv_cache, self.kv_scale, self.row_offsets,
                                          self.seq_lens, self.inp.total_rows, self.max_seq_len,
                                          self.num_splits, self.o_part, self.lse_part, stream)
            return
        if self.paged is not None:
            mla.mla_decode_latent_paged(self.dims, self.q_lat, self.kv_cache, *self._pages(), self.seq_lens,
                                        self.max_seq_len, self.num_splits, self.o_part, self.lse_part, stream)
            return
        mla.mla_decode_latent(self.dims, self.q_lat, self.kv_cache, self.row_offsets, self.seq_lens,
                              self.inp.total_rows, self.max_seq_len, self.num_splits, self.o_part,
                              self.lse_part, stream)

    def combine(self, stream=None):
        mla.mla_combine(self.dims, self.o_part, self.lse_part, self.num_splits, self.o_lat, self.lse, stream)

    def up_v(self, stream=None):
        mla.mla_up_v(self.dims, self.o_lat, self.w_uv, self.out, stream)

    def combine_up_v(self, stream=None):
        mla.mla_combine_up_v(self.dims, self.o_part, self.lse_part, self.num_splits, self.w_uv, self.out,
                             self.lse, stream)

    def run(self, stream=None):
        """One step: out and lse (o_lat is only written by ``combine``)."""
        self.absorb_rope(stream)
        self.decode_latent(stream)
        self.combine_up_v(stream)

    def capture(self) -> "torch.cuda.CUDAGraph":
        """The calls of ``run`` recorded once as a HIP graph (the library launches
        kernels only: no allocation, copy or memset), replayed with
        ``graph.replay()`` on the current stream."""
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()  # one eager pass on the capture stream before recording
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            self.run()
        return graph

    # results ----------------------------------------------------------------
    def q_lat_f64(self) -> np.ndarray:
        return bits_to_f64(self.q_lat, self.inp.dtype)

    def cache_f64(self) -> np.ndarray:
        return bits_to_f64(self.kv_cache, self.inp.dtype)

    def fp8_raw(self):
        """(row bytes, scales) of an fp8 cache in the packed order."""
        rows, scale = self.kv_cache.cpu().numpy(), self.kv_scale.cpu().numpy()
        if self.paged is None:
            return rows, scale
        out_r, out_s = self.fp8.rows.copy(), self.fp8.scale.copy()
        for b in range(self.inp.B):
            n = int(self.inp.lens[b]) + 1
            o = int(self.inp.row_offsets[b])
            idx = self.paged.rows_of(b, n)
            out_r[o:o + n], out_s[o:o + n] = rows[idx], scale[idx]
        return out_r, out_s

    def cache_raw(self) -> np.ndarray:
        """The cache in storage form, in the packed order (a paged cache is
        gathered back through its block table)."""
        a = self.kv_cache.cpu().numpy()
        a = a.view(np.uint16) if self.inp.dtype == BF16 else a
        if self.paged is None:
            return a
        out = self.inp.kv_cache.copy()
        for b in range(self.inp.B):
            n = int(self.inp.lens[b]) + 1
            o = int(self.inp.row_offsets[b])
            out[o:o + n] = a[self.paged.rows_of(b, n)]
        return out
