"""The benchmark's algorithmic bytes and flops (CPU only).

The roofline fractions the benchmark reports divide these figures by measured
times, so they are pinned here against values worked out by hand for the five
workloads.  A step reads every attended cache row once (the L_b cached rows
plus the appended one), writes the appended row, reads W_UK and W_UV once
and the step's inputs (q_nope, q_rope, c_kv_new, k_rope_new) once, and
writes out in fp32; a cached row costs 2 H (r + d_rope + r) flops (its score
over r + d_rope columns and its share of the latent weighted sum), and the two
projections 2 B H d_head r each.  The decode kernel's own figures are the
cache rows alone.  Worked by hand:

  tiny   (fp32, B 1, H 8, 32/32, r 64, d_rope 16, T 128): 129 rows of 320 B;
         step 175,552 B and 362,752 flop
  small  (fp32, B 8, H 16, 64/64, r 64, d_rope 32, T 1024): 8,200 rows of 384 B;
         step 3,761,152 B and 44,081,152 flop
  dsv2   (bf16, B 16, H 128, 128/128, r 512, d_rope 64, T 4096): 65,552 rows
         of 1,152 B = 75,515,904 B; step 110,942,208 B and 18,794,938,368 flop
  dsv2_long (B 2, T 131072): 262,146 rows = 301,992,192 B; step 335,780,608 B
         and 73,082,109,952 flop
"""
import numpy as np
import pytest

import bench
from head_latent_attention_12_amd import synthetic as syn

HAND = {
    "tiny": dict(rows=129, k3=129 * 320, step=175_552, flops=362_752),
    "small": dict(rows=8_200, k3=8_200 * 384, step=3_761_152, flops=44_081_152),
    "dsv2": dict(rows=65_552, k3=75_515_904, step=110_942_208, flops=18_794_938_368),
    "dsv2_long": dict(rows=262_146, k3=301_992_192, step=335_780_608, flops=73_082_109_952),
}


@pytest.mark.parametrize("name", list(HAND))
def test_algorithmic_figures_match_hand_values(name):
    inp = syn.make_inputs(name)
    rows, step_bytes, step_flops, k3_bytes, k3_flops = bench.algorithmic(inp)
    h = HAND[name]
    assert rows == h["rows"] and k3_bytes == h["k3"]
    assert step_bytes == h["step"] and step_flops == h["flops"]
    assert k3_flops == 2 * inp.H * (inp.W + inp.r) * rows


def test_ragged_figures_follow_its_lengths():
    """The ragged batch's figures depend on its drawn lengths: rows = sum of
    (L_b + 1), 1152 bytes each, the rest as for dsv2 (same shape, B 64)."""
    inp = syn.make_inputs("dsv2_ragged")
    rows, step_bytes, step_flops, k3_bytes, _ = bench.algorithmic(inp)
    assert rows == int(np.sum(inp.lens + 1)) == 259_540
    assert k3_bytes == rows * 1152
    fixed = 64 * 1152 + 2 * 128 * 128 * 512 * 2 + 64 * 128 * 192 * 2 + 64 * 576 * 2 + 64 * 128 * 128 * 4
    assert step_bytes == k3_bytes + fixed == 340_032_000
    assert step_flops == 2 * 128 * 1088 * rows + 2 * 2 * 64 * 128 * 128 * 512


def test_fp8_rows_count_their_stored_bytes():
    """An fp8 cache row is 512 codes, 64 bf16 RoPE values and a 4-byte scale."""
    inp = syn.make_inputs("dsv2")
    rows, _, _, k3_bytes, _ = bench.algorithmic(inp, fp8=True)
    assert k3_bytes == rows * (512 + 128 + 4) == 42_215_488
