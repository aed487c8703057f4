"""Test helpers: turn seeded step inputs into the oracle's fp64 arguments."""
import numpy as np

from oracle import mla_oracle as orc


def oracle_args(step):
    """(seqs, q_nope, q_rope, c_new, k_new, w_uk, w_uv) in fp64 for the oracle."""
    seqs = []
    for b in range(step.B):
        rows = step.cached_rows_f64(b)
        seqs.append((rows[:, :step.r], rows[:, step.r:]))
    return (seqs, step.f64("q_nope"), step.f64("q_rope"), step.f64("c_kv_new"),
            step.f64("k_rope_new"), step.f64("w_uk"), step.f64("w_uv"))


def oracle_step(step, form="absorbed", batch_ids=None):
    seqs, qn, qr, cn, kn, wuk, wuv = oracle_args(step)
    return orc.decode_batch(seqs, qn, qr, cn, kn, wuk, wuv, step.softmax_scale,
                            step.rope_base, form=form, batch_ids=batch_ids)


def normwise_rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


# The parity gate of the GPU tests (fp32: normwise relative error; bf16: the
# absolute max/mean bounds, plus bounds relative to the output's scale: the
# rounding of q~ and of the softmax weights to bf16 gives weight errors of a
# few 2^-9, i.e. output errors of a few 0.1% of max|out| at worst and far
# less on average).
F32_GATE = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 5e-3
BF16_TIGHT_MAX_REL, BF16_TIGHT_MEAN_REL = 1e-2, 1e-3


def gate_failures(dtype, got, ref):
    """The bounds of the parity gate that ``got`` breaks against ``ref`` (an
    empty list: it passes).  ``dtype`` is the storage dtype, "f32" or "bf16"."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    if dtype == "f32":
        return ["f32 normwise"] if normwise_rel(got, ref) > F32_GATE else []
    fails = []
    if err.max() > BF16_MAX:
        fails.append("bf16 max abs")
    if err.mean() > BF16_MEAN:
        fails.append("bf16 mean abs")
    scale = np.abs(ref).max()
    if err.max() > BF16_TIGHT_MAX_REL * scale:
        fails.append("bf16 max rel to scale")
    if err.mean() > BF16_TIGHT_MEAN_REL * scale:
        fails.append("bf16 mean rel to scale")
    return fails
