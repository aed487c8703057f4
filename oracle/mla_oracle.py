"""CPU oracle for one Multi-head Latent Attention (MLA) decode step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  It is never on the product path and
shares no code with the HIP library.

Everything is plain NumPy in float64, written to be checked by eye against
the pages, with no blocking, fusion or reordering beyond what the definitions
state.  Sources (page title, section):

  [P1] "DeepSeek MLA, Built From the Paper" (yiqiao-yin deepspeed-course):
       §1 the cache-size formulas, §2 decoupled RoPE, §3 matrix absorption.
  [P2] "MLA from scratch" (shivam2003.com, DeepSeek 3.2): the MLAAttention
       module (forward pass), KV cache management during decode, absorbing
       projections, shape tracing.
  [P3] "Build a DeepSeek Model (From Scratch)", chapter 3 (Manning preview):
       figure captions on RoPE pairs and on the decoupled content/position
       paths whose scores add.
  [P5] "Multi-head latent attention" (octlm blog): the latent plus shared
       RoPE key cache, and the `_project_mla` concatenated [content | rope]
       query/key layout.

Readings where the pages are silent or garbled (each also listed in the
design notes):

  * RoPE pairs adjacent dimensions (2i, 2i+1) and rotates pair i by the
    angle pos * base**(-2i/d) (the RoFormer form the pages cite; [P3] keeps
    only the captions "dimensions are paired" and "rotated by a
    position-dependent angle", its formula figure is missing).
  * The new token is appended to the cache first and then attended to, so a
    sequence with L cached tokens attends over L + 1 rows; the query sits at
    position L ([P2] concatenates the new latent before attention and its
    shape trace grows the cache by one row per step).
  * The cached RoPE keys are stored already rotated by their own positions
    ([P5]: the shared key is rotated normally and cached).
  * One RoPE key per token, shared by all heads ([P1] §2, [P5]).
  * Softmax scale 1/sqrt(d_head + d_rope) is passed in by the caller.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Cache-size formulas  [P1] §1 (values cached per token per layer)
# ---------------------------------------------------------------------------


def cache_values_mha(n_heads: int, d_head: int) -> int:
    """Keys and values for every head: 2 * n_heads * d_head."""
    return 2 * n_heads * d_head


def cache_values_gqa(n_kv_heads: int, d_head: int) -> int:
    """Keys and values for the shared kv heads only: 2 * n_kv_heads * d_head."""
    return 2 * n_kv_heads * d_head


def cache_values_mla(r_kv: int, d_rope: int) -> int:
    """One latent of rank r_kv plus one shared RoPE key: r_kv + d_rope."""
    return r_kv + d_rope


# ---------------------------------------------------------------------------
# Rotary position embedding  [P3] RoPE figure captions, [P5] shared RoPE key
# ---------------------------------------------------------------------------


def rope_frequencies(d: int, base: float) -> np.ndarray:
    """theta_i = base**(-2i/d) for pair i = 0 .. d/2-1."""
    if d % 2:
        raise ValueError("RoPE width must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return base ** (-2.0 * i / d)


def rope(x: np.ndarray, pos: float, base: float, dtype=np.float64) -> np.ndarray:
    """Rotate each adjacent pair (x[2i], x[2i+1]) of the last axis by pos*theta_i
    (evaluated in ``dtype``; float64 unless a test asks for a float32 run)."""
    x = np.asarray(x, dtype=dtype)
    ang = float(pos) * rope_frequencies(x.shape[-1], base)
    c, s = np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ---------------------------------------------------------------------------
# Softmax  [P2] MLAAttention forward (scaled scores, softmax over keys)
# ---------------------------------------------------------------------------


def softmax(s: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Softmax over the last axis: subtract the max, exponentiate, normalise."""
    s = np.asarray(s, dtype=dtype)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def logsumexp(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1)
    return m + np.log(np.sum(np.exp(s - m[..., None]), axis=-1))


# ---------------------------------------------------------------------------
# The append  [P2] KV cache management (new latent written at the current
# position, cache grows by one row), [P5] the cache holds c_t and the rotated
# shared key
# ---------------------------------------------------------------------------


def appended_row(c_new: np.ndarray, k_rope_new: np.ndarray, pos: int, base: float,
                 dtype=np.float64) -> np.ndarray:
    """The cache row the step writes: [c_kv_new | RoPE(k_rope_new, pos)]."""
    return np.concatenate([np.asarray(c_new, dtype), rope(k_rope_new, pos, base, dtype)])


def append(c_cached: np.ndarray, krot_cached: np.ndarray, c_new: np.ndarray,
           k_rope_new: np.ndarray, base: float, dtype=np.float64):
    """Cache after the step: L cached rows plus the new one at position L."""
    L = c_cached.shape[0]
    row = appended_row(c_new, k_rope_new, L, base, dtype)
    r = c_cached.shape[1]
    C = np.vstack([np.asarray(c_cached, dtype), row[None, :r]])
    KR = np.vstack([np.asarray(krot_cached, dtype), row[None, r:]])
    return C, KR


# ---------------------------------------------------------------------------
# Naive decode: rebuild K and V for every cached token and head
# [P2] MLAAttention forward (up-project all cached latents with W_UK, W_UV,
# then standard attention), [P5] `_project_mla` (query and key are
# [content | rope], the rope key broadcast to every head), [P3] the score is
# the content score plus the position score
# ---------------------------------------------------------------------------


def naive_decode_seq(q_nope, q_rope, c_cached, krot_cached, c_new, k_rope_new,
                     w_uk, w_uv, scale, base, dtype=np.float64):
    """Output [H, d_v] of one sequence's decode step, naive form.

    q_nope [H, d_head], q_rope [H, d_rope] (unrotated), c_cached [L, r],
    krot_cached [L, d_rope] (rotated), c_new [r], k_rope_new [d_rope]
    (unrotated), w_uk [H, d_head, r], w_uv [H, d_v, r].  Evaluated in
    ``dtype`` (float64 unless a test asks for a float32 run).
    """
    C, KR = append(c_cached, krot_cached, c_new, k_rope_new, base, dtype)
    pos = c_cached.shape[0]
    H = q_nope.shape[0]
    q_nope, w_uk, w_uv = (np.asarray(a, dtype) for a in (q_nope, w_uk, w_uv))
    out = np.empty((H, w_uv.shape[1]), dtype=dtype)
    for h in range(H):
        k_content = C @ w_uk[h].T                          # [L+1, d_head]
        v = C @ w_uv[h].T                                  # [L+1, d_v]
        k = np.concatenate([k_content, KR], axis=1)        # [L+1, d_head + d_rope]
        q = np.concatenate([q_nope[h], rope(q_rope[h], pos, base, dtype)])
        p = softmax(dtype(scale) * (k @ q), dtype)
        out[h] = p @ v
    return out


# ---------------------------------------------------------------------------
# Absorbed decode: attend in the latent space
# [P1] §3 (q^T (W_UK c) = (W_UK^T q)^T c, keys never rebuilt), [P2] absorbing
# projections (weights applied to the latents directly, W_UV after the
# weighted sum), [P1] §2 / [P5] (the RoPE part scores against the shared key)
# ---------------------------------------------------------------------------


def absorbed_decode_seq(q_nope, q_rope, c_cached, krot_cached, c_new, k_rope_new,
                        w_uk, w_uv, scale, base, dtype=np.float64):
    """Absorbed form of the same step; returns every intermediate.

    Returns a dict with
      q_lat   [H, r + d_rope]  [W_UK^T q_nope | RoPE(q_rope, L)]
      new_row [r + d_rope]     the appended cache row
      scores  [H, L+1]         scaled logits
      lse     [H]              natural-log sum of exp(scores)
      o_lat   [H, r]           softmax-weighted sum of latents
      out     [H, d_v]         W_UV o_lat
    """
    C, KR = append(c_cached, krot_cached, c_new, k_rope_new, base, dtype)
    pos = c_cached.shape[0]
    H, r = q_nope.shape[0], C.shape[1]
    q_nope, w_uk, w_uv = (np.asarray(a, dtype) for a in (q_nope, w_uk, w_uv))
    q_tilde = np.stack([w_uk[h].T @ q_nope[h] for h in range(H)])        # [H, r]
    q_r = np.stack([rope(q_rope[h], pos, base, dtype) for h in range(H)])  # [H, d_rope]
    scores = dtype(scale) * (q_tilde @ C.T + q_r @ KR.T)                 # [H, L+1]
    p = softmax(scores, dtype)
    o_lat = p @ C                                                        # [H, r]
    out = np.stack([w_uv[h] @ o_lat[h] for h in range(H)])               # [H, d_v]
    return dict(q_lat=np.concatenate([q_tilde, q_r], axis=1),
                new_row=np.concatenate([C[-1], KR[-1]]),
                scores=scores, lse=logsumexp(scores), o_lat=o_lat, out=out)


# ---------------------------------------------------------------------------
# Folding the up-projections into neighbouring weights ahead of time
# [P2] "Absorbing projections (inference optimisation)": W_O absorbs W_UV
# (a product of fixed weights computed once, after which the value
# up-projection is skipped and the attention-weighted latents go straight to
# the output space), and the same trick applies on the query side; [P5] "What
# we didn't build, and why": at decode time the up-projection is folded into
# the query and output matrices.  The readings (also in the design notes):
#   * Query side: [P2]'s forward pass puts the RMSNorm norm_q between W_DQ and
#     W_UQ, so a fold across it would not be an identity.  The exact fold is
#     W_UK into W_UQ per head: q~[h] = W_UK[h]^T W_UQ[h] c_q, with c_q the
#     normalised query latent and W_UQ[h] head h's d_head rows of the
#     Linear(d_c_q -> H*d_head) weight.
#   * Output side: [P2]'s shape comment multiplies (d_model, H*d_h) by
#     (H*d_h, d_c) into one (d_model, d_c) matrix, which would sum the heads'
#     latent outputs before they exist.  Each head has its own latent output,
#     so the fold is per head, W_OV[h] = W_O[:, head h's d_v columns] W_UV[h]
#     (d_model x d_c, the page's shape, once per head), and the output is the
#     sum over heads y = sum_h W_OV[h] o_lat[h] (= W_O applied to the
#     concatenated heads).
# ---------------------------------------------------------------------------


def query_projection(c_q: np.ndarray, w_uq: np.ndarray, n_heads: int) -> np.ndarray:
    """q_nope [H, d_head] = W_UQ c_q split per head ([P2] forward pass:
    q = W_UQ(c_q) reshaped to heads); w_uq is [H*d_head, d_c_q]."""
    q = np.asarray(w_uq, np.float64) @ np.asarray(c_q, np.float64)
    return q.reshape(n_heads, -1)


def output_projection(out: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """y [d_model] = W_O applied to the heads' outputs concatenated ([P2]
    forward pass: out reshaped to H*d_h, then W_O); w_o is [d_model, H*d_v]."""
    return np.asarray(w_o, np.float64) @ np.asarray(out, np.float64).reshape(-1)


def fold_query(w_uq: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """W_QK [H, r, d_c_q]: W_QK[h] = W_UK[h]^T W_UQ[h], head h's block of
    w_uq [H*d_head, d_c_q] being its rows h*d_head .. (h+1)*d_head - 1."""
    H, dh, _ = w_uk.shape
    w_uq = np.asarray(w_uq, np.float64)
    return np.stack([np.asarray(w_uk[h], np.float64).T @ w_uq[h * dh:(h + 1) * dh] for h in range(H)])


def fold_output(w_o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """W_OV [d_model, H*r]: columns h*r .. (h+1)*r - 1 hold W_O[:, h*d_v ..
    (h+1)*d_v - 1] W_UV[h]."""
    H, dv, _ = w_uv.shape
    w_o = np.asarray(w_o, np.float64)
    return np.concatenate([w_o[:, h * dv:(h + 1) * dv] @ np.asarray(w_uv[h], np.float64) for h in range(H)],
                          axis=1)


def folded_decode_seq(c_q, q_rope, c_cached, krot_cached, c_new, k_rope_new, w_qk, w_ov, scale, base):
    """One sequence's step with folded weights: q~[h] = W_QK[h] c_q, attention
    in the latent space as in the absorbed form, y = W_OV o_lat (the heads'
    latent outputs concatenated).  Returns q_tilde [H, r], lse [H],
    o_lat [H, r] and y [d_model]."""
    C, KR = append(c_cached, krot_cached, c_new, k_rope_new, base)
    pos = c_cached.shape[0]
    H = w_qk.shape[0]
    c_q = np.asarray(c_q, np.float64)
    q_tilde = np.stack([np.asarray(w_qk[h], np.float64) @ c_q for h in range(H)])   # [H, r]
    q_r = np.stack([rope(q_rope[h], pos, base) for h in range(H)])                  # [H, d_rope]
    scores = scale * (q_tilde @ C.T + q_r @ KR.T)                                   # [H, L+1]
    p = softmax(scores)
    o_lat = p @ C                                                                   # [H, r]
    y = np.asarray(w_ov, np.float64) @ o_lat.reshape(-1)                            # [d_model]
    return dict(q_tilde=q_tilde, lse=logsumexp(scores), o_lat=o_lat, y=y)


# ---------------------------------------------------------------------------
# Batched step over packed sequences
# ---------------------------------------------------------------------------


def decode_batch(seqs, q_nope, q_rope, c_new, k_rope_new, w_uk, w_uv, scale, base,
                 form: str = "absorbed", batch_ids=None):
    """Run the step for every sequence (or the listed ``batch_ids``).

    ``seqs[b]`` is ``(c_cached [L_b, r], krot_cached [L_b, d_rope])`` in fp64.
    For form="absorbed" returns a dict of stacked intermediates; for
    form="naive" returns out [nb, H, d_v].
    """
    ids = range(len(seqs)) if batch_ids is None else batch_ids
    if form == "naive":
        return np.stack([naive_decode_seq(q_nope[b], q_rope[b], seqs[b][0], seqs[b][1],
                                          c_new[b], k_rope_new[b], w_uk, w_uv, scale, base)
                         for b in ids])
    res = [absorbed_decode_seq(q_nope[b], q_rope[b], seqs[b][0], seqs[b][1],
                               c_new[b], k_rope_new[b], w_uk, w_uv, scale, base) for b in ids]
    keys = ("q_lat", "new_row", "lse", "o_lat", "out")
    return {k: np.stack([x[k] for x in res]) for k in keys}


def rope_through_projection_scores(q, w_uk, c, q_pos, k_pos, base):
    """Coupled-RoPE scores, and the single-query absorption one might attempt.

    With RoPE applied to the reconstructed content key, the score against
    token t is (R_qpos q) . (R_t W_UK c_t).  Folding W_UK into one query
    vector q~ = W_UK^T R_qpos q and scoring q~ . c_t drops R_t: the rotation
    sits between q and W_UK and differs per token ([P1] §2, [P3] summary).
    Returns (true scores [L], single-q~ scores [L]).
    """
    qr = rope(q, q_pos, base)
    true = np.array([qr @ rope(w_uk @ c[t], k_pos[t], base) for t in range(c.shape[0])])
    q_tilde = w_uk.T @ qr
    folded = c @ q_tilde
    return true, folded


# ---------------------------------------------------------------------------
# Latent KV production from the hidden state  [P2] module structure: W_DKV
# (d_model -> d_c) then norm_kv (an RMSNorm over the latent); [P1] §2 and
# [P5]: W_KR gives the one RoPE key shared by the heads (rotated later, by the
# append).  The RMSNorm's epsilon is not on the pages; the caller passes it.
# ---------------------------------------------------------------------------


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """weight * x / sqrt(mean(x**2) + eps) over the last axis."""
    return weight * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def kv_down(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray, norm_w: np.ndarray,
            eps: float) -> tuple[np.ndarray, np.ndarray]:
    """(c_kv_new, k_rope_new) for hidden states h [B, d_model]; w_dkv [d_c,
    d_model] and w_kr [d_rope, d_model] are Linear weights (out, in)."""
    c_kv = rms_norm(h @ w_dkv.T, norm_w, eps)
    k_rope = h @ w_kr.T
    return c_kv, k_rope


# ---------------------------------------------------------------------------
# FP8 latent cache  [P2] "what's not in this implementation": the latent cache
# can be quantised to FP8 for a further memory reduction.  The pages fix no
# format or scaling; the readings taken here (listed in the design notes):
#   * codes are OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits;
#     exponent field 0 is subnormal (m/8 * 2^-6), 0x7f / 0xff are NaN, no
#     infinities, 448 is the largest finite value;
#   * one power-of-two scale per cached row: 2^e with e the smallest integer in
#     [-116, 63] such that max|c_kv| <= 448 * 2^e;
#   * codes round to the nearest value, ties to the even code, and saturate at
#     448; the rotated RoPE key of the row stays bf16.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0
FP8_MIN_EXP, FP8_MAX_EXP = -116, 63


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, from the format's definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3 = np.array([e4m3_value(c) for c in range(256)])


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of each finite y: the closest of the 127 finite
    non-negative values to |y| (ties to the even code, above 448: 448), with
    the sign bit of y (also for a result of zero)."""
    y = np.asarray(y, dtype=np.float64)
    pos = _E4M3[:0x7F]                       # codes 0 .. 0x7e, increasing
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(pos, a), 1, 0x7E)   # pos[hi - 1] <= a <= pos[hi]
    lo = hi - 1
    d_lo, d_hi = a - pos[lo], pos[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a <= 0.0, 0, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def fp8_row_exponent(amax: float) -> int:
    """Smallest e in [FP8_MIN_EXP, FP8_MAX_EXP] with amax <= 448 * 2^e."""
    for e in range(FP8_MIN_EXP, FP8_MAX_EXP + 1):
        if amax <= E4M3_MAX * 2.0 ** e:
            return e
    return FP8_MAX_EXP


def fp8_quantize_row(c: np.ndarray):
    """(codes [r] uint8, scale) of one latent row."""
    c = np.asarray(c, dtype=np.float64)
    e = fp8_row_exponent(float(np.max(np.abs(c))))
    return e4m3_encode(c / 2.0 ** e), 2.0 ** e


def fp8_dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Latent values code * scale of rows [n, r] with scales [n]."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]
