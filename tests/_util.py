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
