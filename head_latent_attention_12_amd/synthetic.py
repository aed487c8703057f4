"""Seeded synthetic inputs for one absorbed-MLA decode step.

This module draws random numbers and stores them in the storage dtype. It
holds none of the decode arithmetic (no rotation, no absorption, no softmax):
both the GPU path and the CPU oracle take their inputs from here, and nothing
else is shared between them.

Workloads (the shapes of the DeepSeek-V2 MLA attention layer as the pages
describe it, plus two small fp32 cases):

  tiny          fp32  B=1   H=8   d_head=d_v=32  r=64  d_rope=16  T=128
  small         fp32  B=8   H=16  d_head=d_v=64  r=64  d_rope=32  T=1024
  dsv2          bf16  B=16  H=128 d_head=d_v=128 r=512 d_rope=64  T=4096
  dsv2_ragged   bf16  B=64  same dims, L_b ~ U{512..8192} (inclusive)
  dsv2_long     bf16  B=2   same dims, T=131072

Recipe (fixed draw order from ``numpy.random.default_rng(seed)``, all fp64,
then rounded to nearest-even into the storage dtype):

  1. (ragged only) L_b, integers in [lo, hi] inclusive
  2. W_UK [H, d_head, r] ~ N(0, 1/r)
  3. W_UV [H, d_v, r]    ~ N(0, 1/r)
  4. q_nope [B, H, d_head] ~ N(0, 1)
  5. q_rope [B, H, d_rope] ~ N(0, 1)      (not yet rotated)
  6. cached c_kv [sum L_b, r] ~ N(0, 1); rows scaled to unit RMS for the
     bf16 DeepSeek-V2-shaped workloads
  7. cached k_rope [sum L_b, d_rope] ~ N(0, 1).  The cache holds keys that
     were already rotated by their own positions; a rotation maps an
     isotropic Gaussian pair to an isotropic Gaussian pair, so drawing the
     stored (rotated) keys directly from N(0, 1) gives exactly that
     distribution without doing any rotation here.
  8. c_kv_new [B, r]       (same treatment as 6)
  9. k_rope_new [B, d_rope] ~ N(0, 1)     (raw, rotated by the step itself)

Cache layout: sequence b owns rows [row_offsets[b], row_offsets[b] + L_b + 1);
its first L_b rows hold the cached tokens and the last one is the slot the
step appends into.  Append slots are filled with NaN so that a step which
fails to write them poisons its own output.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"

# name -> (B, H, d_head, d_v, r, d_rope, T or (lo, hi), dtype, unit-RMS c_kv rows, seed)
WORKLOADS = {
    "tiny": dict(B=1, H=8, d_head=32, d_v=32, r=64, d_rope=16, T=128, dtype=F32, rms_rows=False, seed=0),
    "small": dict(B=8, H=16, d_head=64, d_v=64, r=64, d_rope=32, T=1024, dtype=F32, rms_rows=False, seed=1),
    "dsv2": dict(B=16, H=128, d_head=128, d_v=128, r=512, d_rope=64, T=4096, dtype=BF16, rms_rows=True, seed=2),
    "dsv2_ragged": dict(B=64, H=128, d_head=128, d_v=128, r=512, d_rope=64, T=(512, 8192), dtype=BF16,
                        rms_rows=True, seed=3),
    "dsv2_long": dict(B=2, H=128, d_head=128, d_v=128, r=512, d_rope=64, T=131072, dtype=BF16,
                      rms_rows=True, seed=4),
}

ROPE_BASE = 10000.0


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even); return uint16 bits.

    fp64 -> fp32 is done with round-to-odd (truncate, then set the last bit
    when inexact), which keeps the second rounding fp32 -> bf16 correct.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    t = x.astype(np.float32)                       # nearest-even
    t64 = t.astype(np.float64)
    # step back toward zero where nearest-even rounded away from zero
    away = np.abs(t64) > np.abs(x)
    tb = t.view(np.uint32).copy()
    tb[away] -= 1                                  # same sign: one ulp toward zero
    inexact = t64 != x
    tb[inexact] |= 1                               # sticky bit (round to odd)
    nan = np.isnan(x)
    lsb = (tb >> 16) & 1
    out = ((tb + 0x7FFF + lsb) >> 16).astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class StepInputs:
    """One decode step's inputs, in storage form (float32 or bf16 bits)."""

    name: str
    seed: int
    B: int
    H: int
    d_head: int
    d_v: int
    r: int
    d_rope: int
    dtype: str
    softmax_scale: float
    rope_base: float
    lens: np.ndarray          # [B] int32   L_b, tokens cached before the step
    row_offsets: np.ndarray   # [B] int64   first cache row of sequence b
    total_rows: int           # rows in the packed cache
    w_uk: np.ndarray          # [H, d_head, r]
    w_uv: np.ndarray          # [H, d_v, r]
    q_nope: np.ndarray        # [B, H, d_head]
    q_rope: np.ndarray        # [B, H, d_rope]
    kv_cache: np.ndarray      # [total_rows, r + d_rope]; append slots hold NaN
    c_kv_new: np.ndarray      # [B, r]
    k_rope_new: np.ndarray    # [B, d_rope]

    @property
    def W(self) -> int:
        return self.r + self.d_rope

    @property
    def positions(self) -> np.ndarray:
        """Position of the new token = its row index inside its sequence."""
        return self.lens.astype(np.int32)

    @property
    def seq_lens(self) -> np.ndarray:
        """Rows attended per sequence after the append."""
        return (self.lens + 1).astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    def f64(self, field: str) -> np.ndarray:
        """Stored values of ``field`` upcast exactly to fp64."""
        a = getattr(self, field)
        if self.dtype == BF16:
            return bf16_bits_to_f64(a)
        return a.astype(np.float64)

    def cached_rows_f64(self, b: int) -> np.ndarray:
        """fp64 view of the L_b cached rows of sequence b (append slot excluded)."""
        o = int(self.row_offsets[b])
        L = int(self.lens[b])
        a = self.kv_cache[o:o + L]
        if self.dtype == BF16:
            return bf16_bits_to_f64(a)
        return a.astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_from_f64(x)
    return np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)


def _unit_rms_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def make_inputs(name: str, seed: int | None = None, **override) -> StepInputs:
    """Draw the inputs of workload ``name``.

    ``override`` may replace B, T (an int or an inclusive (lo, hi) pair) or
    ``lens`` (an explicit list of per-sequence cached lengths, no draw) to get
    smaller cases of the same shape family for tests.
    """
    spec = dict(WORKLOADS[name])
    lens_explicit = override.pop("lens", None)
    spec.update(override)
    if seed is None:
        seed = spec["seed"]
    rng = np.random.default_rng(seed)
    B, H, dh, dv, r, dr = (spec[k] for k in ("B", "H", "d_head", "d_v", "r", "d_rope"))
    dtype = spec["dtype"]
    T = spec["T"]
    if lens_explicit is not None:
        lens = np.asarray(lens_explicit, dtype=np.int64)
        B = len(lens)
    elif isinstance(T, tuple):
        lens = rng.integers(T[0], T[1], size=B, endpoint=True).astype(np.int64)
    else:
        lens = np.full(B, T, dtype=np.int64)
    rows_per_seq = lens + 1
    row_offsets = np.zeros(B, dtype=np.int64)
    row_offsets[1:] = np.cumsum(rows_per_seq)[:-1]
    total_rows = int(rows_per_seq.sum())
    n_cached = int(lens.sum())

    w_uk = rng.standard_normal((H, dh, r)) / math.sqrt(r)
    w_uv = rng.standard_normal((H, dv, r)) / math.sqrt(r)
    q_nope = rng.standard_normal((B, H, dh))
    q_rope = rng.standard_normal((B, H, dr))
    c_cached = rng.standard_normal((n_cached, r))
    if spec["rms_rows"]:
        c_cached = _unit_rms_rows(c_cached)
    k_cached = rng.standard_normal((n_cached, dr))
    c_new = rng.standard_normal((B, r))
    if spec["rms_rows"]:
        c_new = _unit_rms_rows(c_new)
    k_new = rng.standard_normal((B, dr))

    W = r + dr
    if dtype == BF16:
        cache = np.full((total_rows, W), 0x7FC0, dtype=np.uint16)
    else:
        cache = np.full((total_rows, W), np.nan, dtype=np.float32)
    c_st = _store(c_cached, dtype)
    k_st = _store(k_cached, dtype)
    del c_cached, k_cached
    src = 0
    for b in range(B):
        o, L = int(row_offsets[b]), int(lens[b])
        cache[o:o + L, :r] = c_st[src:src + L]
        cache[o:o + L, r:] = k_st[src:src + L]
        src += L
    del c_st, k_st

    return StepInputs(
        name=name, seed=int(seed), B=B, H=H, d_head=dh, d_v=dv, r=r, d_rope=dr, dtype=dtype,
        softmax_scale=1.0 / math.sqrt(dh + dr), rope_base=ROPE_BASE,
        lens=lens.astype(np.int32), row_offsets=row_offsets, total_rows=total_rows,
        w_uk=_store(w_uk, dtype), w_uv=_store(w_uv, dtype),
        q_nope=_store(q_nope, dtype), q_rope=_store(q_rope, dtype),
        kv_cache=cache, c_kv_new=_store(c_new, dtype), k_rope_new=_store(k_new, dtype),
    )


@dataclasses.dataclass
class PagedCache:
    """The same cache rows laid out in pages: row t of sequence b is row
    t % page_rows of page block_table[b, t // page_rows]."""

    page_rows: int
    block_table: np.ndarray   # [B, bt_stride] int32 physical page ids
    cache: np.ndarray         # [total_pages * page_rows, r + d_rope], storage form (fp8: row bytes)
    scale: np.ndarray | None = None  # fp8 cache: [total_pages * page_rows] row scales

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def total_pages(self) -> int:
        return self.cache.shape[0] // self.page_rows

    def rows_of(self, b: int, n: int) -> np.ndarray:
        """Physical cache rows of the first n in-sequence rows of sequence b."""
        t = np.arange(n)
        return self.block_table[b, t // self.page_rows].astype(np.int64) * self.page_rows + t % self.page_rows


def paginate(step: StepInputs, page_rows: int, seed: int = 0, spare_pages: int = 3,
             fp8: "Fp8Cache | None" = None) -> PagedCache:
    """Scatter the packed cache of ``step`` (or its fp8 form ``fp8``) into
    pages of ``page_rows`` rows, page ids shuffled with a seeded permutation
    (so the pages of different sequences interleave), each sequence given the
    pages for its L_b + 1 rows (the appended row included).  Unused page rows
    and the ``spare_pages`` never referenced hold NaN (fp8: NaN codes and
    scales), so that a read through a wrong page cannot pass."""
    rng = np.random.default_rng(seed)
    need = [(int(L) + 1 + page_rows - 1) // page_rows for L in step.lens]
    bt_stride = max(need) + 1
    total_pages = sum(need) + spare_pages
    perm = rng.permutation(total_pages).astype(np.int32)
    n_phys = total_pages * page_rows
    if fp8 is None:
        nan = np.uint16(0x7FC0) if step.dtype == BF16 else np.float32(np.nan)
        src_rows, src_scale = step.kv_cache, None
        cache = np.full((n_phys, step.W), nan, dtype=step.kv_cache.dtype)
        scale = None
    else:
        src_rows, src_scale = fp8.rows, fp8.scale
        cache = np.full((n_phys, fp8.rows.shape[1]), 0x7F, dtype=np.uint8)
        scale = np.full(n_phys, np.nan, dtype=np.float32)
    block_table = np.full((step.B, bt_stride), -1, dtype=np.int32)
    k = 0
    for b in range(step.B):
        block_table[b, :need[b]] = perm[k:k + need[b]]
        k += need[b]
    paged = PagedCache(page_rows, block_table, cache, scale)
    for b in range(step.B):
        n = int(step.lens[b]) + 1
        src = int(step.row_offsets[b])
        dst = paged.rows_of(b, n)
        cache[dst] = src_rows[src:src + n]
        if scale is not None:
            scale[dst] = src_scale[src:src + n]
    # unused entries point at a spare page (in range, never read for valid rows)
    block_table[block_table < 0] = perm[-1]
    return paged


@dataclasses.dataclass
class Fp8Cache:
    """A latent cache in the fp8 row layout: per row, r E4M3 codes then the
    d_rope bf16 RoPE values as little-endian bytes, plus one fp32 scale."""

    rows: np.ndarray    # [total_rows, r + 2 * d_rope] uint8
    scale: np.ndarray   # [total_rows] float32


def make_fp8_cache(step: StepInputs, seed: int = 3) -> Fp8Cache:
    """Cached rows of ``step`` in the fp8 layout, drawn directly as codes (no
    quantisation here): sign and mantissa uniform, exponent field
    round(N(12.8, 1.1)) clipped to [0, 15] (the NaN code becomes 448), and a
    row scale 2^e with e uniform in {-8, -7}: values with an RMS near 0.85 and
    a 99th percentile near 3, like the unit-RMS bf16 rows; the RoPE values are
    the step's bf16 ones.  The
    append slots hold NaN codes and a NaN scale."""
    assert step.dtype == BF16, "the fp8 cache layout keeps bf16 RoPE values"
    rng = np.random.default_rng(seed)
    n, r = step.total_rows, step.r
    expo = np.clip(np.rint(rng.normal(12.8, 1.1, size=(n, r))), 0, 15).astype(np.uint8)
    codes = (rng.integers(0, 2, size=(n, r), dtype=np.uint8) << 7) | (expo << 3) | \
        rng.integers(0, 8, size=(n, r), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] -= 1
    rows = np.empty((n, r + 2 * step.d_rope), dtype=np.uint8)
    rows[:, :r] = codes
    rows[:, r:] = np.ascontiguousarray(step.kv_cache[:, r:]).view(np.uint8)
    scale = np.ldexp(1.0, rng.integers(-8, -6, size=n)).astype(np.float32)
    slots = step.row_offsets + step.lens
    rows[slots, :r] = 0x7F
    scale[slots] = np.nan
    return Fp8Cache(rows, scale)


@dataclasses.dataclass
class KvDownInputs:
    """Inputs of the latent KV production from the hidden state (bf16 bits)."""

    B: int
    d_model: int
    r: int
    d_rope: int
    eps: float
    h: np.ndarray        # [B, d_model]
    w_dkv: np.ndarray    # [r, d_model]
    w_kr: np.ndarray     # [d_rope, d_model]
    norm_w: np.ndarray   # [r]

    def f64(self, field: str) -> np.ndarray:
        return bf16_bits_to_f64(getattr(self, field))


def make_kv_down_inputs(B: int, d_model: int, r: int = 512, d_rope: int = 64, seed: int = 11,
                        eps: float = 1e-6) -> KvDownInputs:
    """Seeded bf16 inputs: h ~ N(0, 1); W_DKV, W_KR ~ N(0, 1/d_model); the
    RMSNorm gain ~ 1 + N(0, 0.1^2); eps 1e-6 (a common choice; the pages give
    none)."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, d_model))
    w_dkv = rng.standard_normal((r, d_model)) / math.sqrt(d_model)
    w_kr = rng.standard_normal((d_rope, d_model)) / math.sqrt(d_model)
    g = 1.0 + 0.1 * rng.standard_normal(r)
    return KvDownInputs(B, d_model, r, d_rope, eps, bf16_bits_from_f64(h), bf16_bits_from_f64(w_dkv),
                        bf16_bits_from_f64(w_kr), bf16_bits_from_f64(g))


@dataclasses.dataclass
class FoldInputs:
    """Weights and query latent of the folded projections (bf16 bits), for a
    step whose attention dims come from a StepInputs."""

    d_c_q: int
    d_model: int
    c_q: np.ndarray      # [B, d_c_q]        normalised query latent
    w_uq: np.ndarray     # [H * d_head, d_c_q]  Linear(d_c_q -> H*d_head) weight
    w_o: np.ndarray      # [d_model, H * d_v]   Linear(H*d_v -> d_model) weight

    def f64(self, field: str) -> np.ndarray:
        return bf16_bits_to_f64(getattr(self, field))


def make_fold_inputs(step: StepInputs, d_c_q: int = 1536, d_model: int = 5120, seed: int = 21) -> FoldInputs:
    """Seeded bf16 inputs of the folded projections at the page's DeepSeek-V2
    sizes (d_c' 1536, d_model 5120) by default: c_q rows drawn N(0, 1) and
    scaled to unit RMS (the output of the query RMSNorm, no gain), W_UQ ~
    N(0, 1/d_c_q), W_O ~ N(0, 1/(H*d_v)), in that order."""
    rng = np.random.default_rng(seed)
    H, dh, dv = step.H, step.d_head, step.d_v
    c_q = _unit_rms_rows(rng.standard_normal((step.B, d_c_q)))
    w_uq = bf16_bits_from_f64(rng.standard_normal((H * dh, d_c_q)) / math.sqrt(d_c_q))
    w_o = np.empty((d_model, H * dv), dtype=np.uint16)
    for m0 in range(0, d_model, 512):  # in row blocks (bounded fp64 temporaries)
        m1 = min(d_model, m0 + 512)
        w_o[m0:m1] = bf16_bits_from_f64(rng.standard_normal((m1 - m0, H * dv)) / math.sqrt(H * dv))
    return FoldInputs(d_c_q, d_model, bf16_bits_from_f64(c_q), w_uq, w_o)
