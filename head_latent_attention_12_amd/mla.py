"""Python binding of libmla.so (ctypes).  Argument marshalling only.

Each function takes torch tensors (device memory) and passes their data
pointers and the stream to the C entry point of the same name declared in
include/mla.h.  All arithmetic of the decode step runs in the HIP kernels of
libmla.so; if the library is missing the binding raises instead of computing
anything itself.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree library; MLA_LIBRARY names another build of it (the host-sanitized
# build that the argument-check tests also run against)
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(_PKG, "libmla.so")

MLA_F32 = 0
MLA_BF16 = 1

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_ALIGNMENT",
          4: "MLA_ERR_WORKSPACE", 5: "MLA_ERR_HIP"}

EXPORTS = ("mla_absorb_q", "mla_rope_append", "mla_decode_latent", "mla_combine", "mla_up_v",
           "mla_combine_up_v", "mla_absorb_rope", "mla_decode_latent_paged", "mla_rope_append_paged",
           "mla_absorb_rope_paged", "mla_decode_latent_fp8", "mla_decode_latent_fp8_paged",
           "mla_absorb_rope_fp8", "mla_absorb_rope_fp8_paged", "mla_kv_down", "mla_kv_down_workspace_size",
           "mla_kv_down_noalloc",
           "mla_fold_query", "mla_fold_output", "mla_absorb_q_folded", "mla_out_folded",
           "mla_out_folded_workspace_size", "mla_partials_size", "mla_plan_splits", "mla_plan_splits_for_lengths",
           "mla_check_dims",
           "mla_status_string", "mla_last_error")


class MlaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("rank", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float)]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m head_latent_attention_12_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(MlaDims)
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        sig = {
            "mla_absorb_q": (i32, [D, P, P, P, P]),
            "mla_rope_append": (i32, [D, P, P, P, P, P, i64, P, P, P]),
            "mla_decode_latent": (i32, [D, P, P, P, P, i64, i32, i32, P, P, P]),
            "mla_combine": (i32, [D, P, P, i32, P, P, P]),
            "mla_up_v": (i32, [D, P, P, P, P]),
            "mla_combine_up_v": (i32, [D, P, P, i32, P, P, P, P]),
            "mla_absorb_rope": (i32, [D, P, P, P, P, P, P, P, i64, P, P, P]),
            "mla_decode_latent_paged": (i32, [D, P, P, P, i32, i32, i64, P, i32, i32, P, P, P]),
            "mla_rope_append_paged": (i32, [D, P, P, P, P, P, i32, i32, i64, P, P, P]),
            "mla_absorb_rope_paged": (i32, [D, P, P, P, P, P, P, P, i32, i32, i64, P, P, P]),
            "mla_decode_latent_fp8": (i32, [D, P, P, P, P, P, i64, i32, i32, P, P, P]),
            "mla_decode_latent_fp8_paged": (i32, [D, P, P, P, P, i32, i32, i64, P, i32, i32, P, P, P]),
            "mla_absorb_rope_fp8": (i32, [D, P, P, P, P, P, P, P, i64, P, P, P, P]),
            "mla_absorb_rope_fp8_paged": (i32, [D, P, P, P, P, P, P, P, i32, i32, i64, P, P, P, P]),
            "mla_kv_down": (i32, [D, i32, P, P, P, P, ctypes.c_float, P, P, P, P]),
            "mla_kv_down_workspace_size": (i32, [D, i32, ctypes.POINTER(ctypes.c_size_t)]),
            "mla_kv_down_noalloc": (i32, [D, i32, P, P, P, P, ctypes.c_float, P, P, P]),
            "mla_fold_query": (i32, [D, i32, P, P, P, P]),
            "mla_fold_output": (i32, [D, i32, P, P, P, P]),
            "mla_absorb_q_folded": (i32, [D, i32, P, P, P, P]),
            "mla_out_folded": (i32, [D, i32, P, P, P, P, P]),
            "mla_out_folded_workspace_size": (i32, [D, i32, ctypes.POINTER(ctypes.c_size_t)]),
            "mla_partials_size": (i32, [D, i32, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
            "mla_plan_splits": (i32, [D, i32, i64, i32]),
            "mla_plan_splits_for_lengths": (i32, [D, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]),
            "mla_check_dims": (i32, [D]),
            "mla_status_string": (ctypes.c_char_p, [i32]),
            "mla_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def make_dims(batch, heads, d_head, d_v, rank, d_rope, dtype, softmax_scale=0.0, rope_base=0.0) -> MlaDims:
    return MlaDims(int(batch), int(heads), int(d_head), int(d_v), int(rank), int(d_rope), int(dtype),
                   float(softmax_scale), float(rope_base))


def _p(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise MlaError(fn, st, lib().mla_last_error().decode())


def mla_absorb_q(dims, q_nope, w_uk, q_lat, stream=None):
    _check("mla_absorb_q", lib().mla_absorb_q(ctypes.byref(dims), _p(q_nope), _p(w_uk), _p(q_lat), _s(stream)))


def mla_rope_append(dims, q_rope, c_kv_new, k_rope_new, positions, row_offsets, total_rows, q_lat, kv_cache,
                    stream=None):
    _check("mla_rope_append", lib().mla_rope_append(
        ctypes.byref(dims), _p(q_rope), _p(c_kv_new), _p(k_rope_new), _p(positions), _p(row_offsets),
        int(total_rows), _p(q_lat), _p(kv_cache), _s(stream)))


def mla_absorb_rope(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, row_offsets, total_rows, q_lat,
                    kv_cache, stream=None):
    _check("mla_absorb_rope", lib().mla_absorb_rope(
        ctypes.byref(dims), _p(q_nope), _p(w_uk), _p(q_rope), _p(c_kv_new), _p(k_rope_new), _p(positions),
        _p(row_offsets), int(total_rows), _p(q_lat), _p(kv_cache), _s(stream)))


def mla_decode_latent(dims, q_lat, kv_cache, row_offsets, seq_lens, total_rows, max_seq_len, num_splits, o_part,
                      lse_part, stream=None):
    _check("mla_decode_latent", lib().mla_decode_latent(
        ctypes.byref(dims), _p(q_lat), _p(kv_cache), _p(row_offsets), _p(seq_lens), int(total_rows),
        int(max_seq_len), int(num_splits), _p(o_part), _p(lse_part), _s(stream)))


def mla_decode_latent_paged(dims, q_lat, kv_cache, block_table, bt_stride, page_rows, total_pages, seq_lens,
                            max_seq_len, num_splits, o_part, lse_part, stream=None):
    _check("mla_decode_latent_paged", lib().mla_decode_latent_paged(
        ctypes.byref(dims), _p(q_lat), _p(kv_cache), _p(block_table), int(bt_stride), int(page_rows),
        int(total_pages), _p(seq_lens), int(max_seq_len), int(num_splits), _p(o_part), _p(lse_part), _s(stream)))


def mla_rope_append_paged(dims, q_rope, c_kv_new, k_rope_new, positions, block_table, bt_stride, page_rows,
                          total_pages, q_lat, kv_cache, stream=None):
    _check("mla_rope_append_paged", lib().mla_rope_append_paged(
        ctypes.byref(dims), _p(q_rope), _p(c_kv_new), _p(k_rope_new), _p(positions), _p(block_table),
        int(bt_stride), int(page_rows), int(total_pages), _p(q_lat), _p(kv_cache), _s(stream)))


def mla_absorb_rope_paged(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, block_table, bt_stride,
                          page_rows, total_pages, q_lat, kv_cache, stream=None):
    _check("mla_absorb_rope_paged", lib().mla_absorb_rope_paged(
        ctypes.byref(dims), _p(q_nope), _p(w_uk), _p(q_rope), _p(c_kv_new), _p(k_rope_new), _p(positions),
        _p(block_table), int(bt_stride), int(page_rows), int(total_pages), _p(q_lat), _p(kv_cache), _s(stream)))


def mla_decode_latent_fp8(dims, q_lat, kv_cache, kv_scale, row_offsets, seq_lens, total_rows, max_seq_len,
                          num_splits, o_part, lse_part, stream=None):
    _check("mla_decode_latent_fp8", lib().mla_decode_latent_fp8(
        ctypes.byref(dims), _p(q_lat), _p(kv_cache), _p(kv_scale), _p(row_offsets), _p(seq_lens), int(total_rows),
        int(max_seq_len), int(num_splits), _p(o_part), _p(lse_part), _s(stream)))


def mla_decode_latent_fp8_paged(dims, q_lat, kv_cache, kv_scale, block_table, bt_stride, page_rows, total_pages,
                                seq_lens, max_seq_len, num_splits, o_part, lse_part, stream=None):
    _check("mla_decode_latent_fp8_paged", lib().mla_decode_latent_fp8_paged(
        ctypes.byref(dims), _p(q_lat), _p(kv_cache), _p(kv_scale), _p(block_table), int(bt_stride),
        int(page_rows), int(total_pages), _p(seq_lens), int(max_seq_len), int(num_splits), _p(o_part),
        _p(lse_part), _s(stream)))


def mla_absorb_rope_fp8(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, row_offsets, total_rows,
                        q_lat, kv_cache, kv_scale, stream=None):
    _check("mla_absorb_rope_fp8", lib().mla_absorb_rope_fp8(
        ctypes.byref(dims), _p(q_nope), _p(w_uk), _p(q_rope), _p(c_kv_new), _p(k_rope_new), _p(positions),
        _p(row_offsets), int(total_rows), _p(q_lat), _p(kv_cache), _p(kv_scale), _s(stream)))


def mla_absorb_rope_fp8_paged(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, block_table, bt_stride,
                              page_rows, total_pages, q_lat, kv_cache, kv_scale, stream=None):
    _check("mla_absorb_rope_fp8_paged", lib().mla_absorb_rope_fp8_paged(
        ctypes.byref(dims), _p(q_nope), _p(w_uk), _p(q_rope), _p(c_kv_new), _p(k_rope_new), _p(positions),
        _p(block_table), int(bt_stride), int(page_rows), int(total_pages), _p(q_lat), _p(kv_cache), _p(kv_scale),
        _s(stream)))


def mla_combine(dims, o_part, lse_part, num_splits, o_lat, lse=None, stream=None):
    _check("mla_combine", lib().mla_combine(ctypes.byref(dims), _p(o_part), _p(lse_part), int(num_splits),
                                            _p(o_lat), _p(lse), _s(stream)))


def mla_up_v(dims, o_lat, w_uv, out, stream=None):
    _check("mla_up_v", lib().mla_up_v(ctypes.byref(dims), _p(o_lat), _p(w_uv), _p(out), _s(stream)))


def mla_combine_up_v(dims, o_part, lse_part, num_splits, w_uv, out, lse=None, stream=None):
    _check("mla_combine_up_v", lib().mla_combine_up_v(ctypes.byref(dims), _p(o_part), _p(lse_part),
                                                      int(num_splits), _p(w_uv), _p(out), _p(lse), _s(stream)))


def mla_kv_down_workspace_size(dims, d_model) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_kv_down_workspace_size", lib().mla_kv_down_workspace_size(ctypes.byref(dims), int(d_model),
                                                                          ctypes.byref(n)))
    return n.value


def mla_kv_down(dims, d_model, h, w_dkv, w_kr, norm_w, eps, workspace, c_kv_new, k_rope_new, stream=None):
    _check("mla_kv_down", lib().mla_kv_down(ctypes.byref(dims), int(d_model), _p(h), _p(w_dkv), _p(w_kr), _p(norm_w),
                                            float(eps), _p(workspace), _p(c_kv_new), _p(k_rope_new), _s(stream)))


def mla_kv_down_noalloc(dims, d_model, h, w_dkv, w_kr, norm_w, eps, c_kv_new, k_rope_new, stream=None):
    _check("mla_kv_down_noalloc", lib().mla_kv_down_noalloc(ctypes.byref(dims), int(d_model), _p(h), _p(w_dkv),
                                                            _p(w_kr), _p(norm_w), float(eps), _p(c_kv_new),
                                                            _p(k_rope_new), _s(stream)))


def mla_fold_query(dims, d_c_q, w_uq, w_uk, w_qk, stream=None):
    _check("mla_fold_query", lib().mla_fold_query(ctypes.byref(dims), int(d_c_q), _p(w_uq), _p(w_uk), _p(w_qk),
                                                  _s(stream)))


def mla_fold_output(dims, d_model, w_o, w_uv, w_ov, stream=None):
    _check("mla_fold_output", lib().mla_fold_output(ctypes.byref(dims), int(d_model), _p(w_o), _p(w_uv), _p(w_ov),
                                                    _s(stream)))


def mla_absorb_q_folded(dims, d_c_q, c_q, w_qk, q_lat, stream=None):
    _check("mla_absorb_q_folded", lib().mla_absorb_q_folded(ctypes.byref(dims), int(d_c_q), _p(c_q), _p(w_qk),
                                                            _p(q_lat), _s(stream)))


def mla_out_folded_workspace_size(dims, d_model) -> int:
    n = ctypes.c_size_t(0)
    _check("mla_out_folded_workspace_size", lib().mla_out_folded_workspace_size(ctypes.byref(dims), int(d_model),
                                                                                ctypes.byref(n)))
    return n.value


def mla_out_folded(dims, d_model, o_lat, w_ov, workspace, y, stream=None):
    _check("mla_out_folded", lib().mla_out_folded(ctypes.byref(dims), int(d_model), _p(o_lat), _p(w_ov),
                                                  _p(workspace), _p(y), _s(stream)))


def mla_partials_size(dims, num_splits):
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_partials_size", lib().mla_partials_size(ctypes.byref(dims), int(num_splits), ctypes.byref(a),
                                                        ctypes.byref(b)))
    return a.value, b.value


def mla_plan_splits(dims, max_seq_len, total_rows, num_cus=0) -> int:
    n = lib().mla_plan_splits(ctypes.byref(dims), int(max_seq_len), int(total_rows), int(num_cus))
    if n < 1:
        raise MlaError("mla_plan_splits", 1, lib().mla_last_error().decode())
    return n


def mla_plan_splits_for_lengths(dims, seq_lens, num_cus=0) -> tuple[int, int]:
    """seq_lens: host sequence of dims.batch ints (rows attended per sequence).
    Returns (num_splits, max_seq_len to pass with it)."""
    arr = (ctypes.c_int32 * int(dims.batch))(*[int(x) for x in seq_lens])
    mls = ctypes.c_int32(0)
    n = lib().mla_plan_splits_for_lengths(ctypes.byref(dims), arr, int(num_cus), ctypes.byref(mls))
    if n < 1:
        raise MlaError("mla_plan_splits_for_lengths", 1, lib().mla_last_error().decode())
    return n, mls.value


def mla_check_dims(dims) -> int:
    return lib().mla_check_dims(ctypes.byref(dims))
