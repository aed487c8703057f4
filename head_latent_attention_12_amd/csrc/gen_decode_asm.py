"""Generate decode_asm.inc: hand-scheduled inner blocks of the bf16 decode kernel.

    python gen_decode_asm.py > decode_asm.inc

Shape: 32-row tiles of 576-wide bf16 cache rows (1152 bytes), 32 heads per
wave, 512 latent columns.  Blocks:

  score block (18 k-steps): S^T[t][h] += cache[t][k..k+16) . q^T, A fragments
    streamed from LDS with ds_read_b128 through a 4-deep rolling window held in
    v[240:255]; B fragments (q) and the accumulator are asm operands.
  fused block (and its branch-free steady-state form): the scores of the
    next tile (36 k-steps into v[208:223]) with the current tile's softmax
    (mask of rows past the split end, exponentials, bf16 packing into
    v[196:203], running sum) interleaved between the first score MFMAs, so
    that it runs while the matrix core is busy; then the P*V product of the
    current tile, O^T[c][h] += cache^T P^T (16 column blocks x 2 k-halves;
    cache^T fragments from pairs of ds_read_b64_tr_b16 through the same kind
    of 4-deep rolling window; accumulators are AGPR operands), during which
    the next tile's scores move into the score operands that the following
    block's softmax reads.  The LDS DMA of a later tile is spread over the
    score MFMAs.

Every LDS read issued by a block is waited for inside that block, so no load
is in flight when the asm statement ends.  The dependency rules observed in
compiler output for gfx950 are followed: an MFMA may overwrite nothing its
neighbours still read, an accumulation on the same destination may follow
directly, a VALU read of a 32x32x16 result needs at least 12 wait states
(20 are given), a VALU read of a transcendental result needs one
instruction in between, and v_permlane32_swap reads a VGPR written by a VALU
op no sooner than two wait states later.
"""
import sys

ROWB = 1152          # bytes per cache row
S_DEPTH = 4          # score-phase fragments in flight
KS = 36              # k-steps of 16 over the 576-wide row
TMP = 204            # mask temporaries (v205 holds -inf)
VLIM = 206           # per-lane row limit of the mask


class _Lds:
    """In-order model of this wave's LDS reads: the wait for read r is
    lgkmcnt(reads issued after r), capped at 15 (a smaller count only waits
    longer, as LDS reads complete in order)."""

    def __init__(self):
        self.n = 0

    def issue(self):
        self.n += 1
        return self.n - 1

    def wait(self, r):
        return f"s_waitcnt lgkmcnt({min(15, self.n - r - 1)})"


def _score_lines(k0, steps, first, acc, qname, extra=None, lds=None):
    """LDS-fed score MFMAs for k-steps k0..k0+steps-1 (4 bases b0..b3).
    `extra` maps an MFMA index to lines of other LDS reads issued right after
    it (their count is taken into the waits)."""
    buf = [f"v[{240 + 4 * j}:{243 + 4 * j}]" for j in range(S_DEPTH)]
    extra = extra or {}
    lds = lds or _Lds()
    out = ["s_waitcnt lgkmcnt(0)"]
    rid = {}

    def read(j):
        kk = k0 + j
        rid[j] = lds.issue()
        out.append(f"ds_read_b128 {buf[j % S_DEPTH]}, %[b{kk & 3}] offset:{128 * (kk >> 2)}")

    for j in range(min(S_DEPTH, steps)):
        read(j)
    for j in range(steps):
        out.append(lds.wait(rid[j]))
        src_c = "0" if (first and j == 0) else acc
        out.append(f"v_mfma_f32_32x32x16_bf16 {acc}, {buf[j % S_DEPTH]}, {qname(j)}, {src_c}")
        if j + S_DEPTH < steps:
            read(j + S_DEPTH)
        for line in extra.get(j, []):
            if line.startswith("ds_read"):
                lds.issue()
            out.append(line)
    return out


def score_block(k0: int, steps: int, first: bool, last: bool) -> str:
    out = _score_lines(k0, steps, first, "%[acc]", lambda j: f"%[q{j}]")
    if last:
        out += ["s_nop 15", "s_nop 3"]
    return "\\n\\t".join(out)


PV_FRAGS = [(2 * g + dc, ks) for g in range(8) for dc, ks in ((0, 0), (1, 0), (0, 1), (1, 1))]
PV_DEPTH = 4         # P*V fragments in flight (rolling window v[240:255], as for the scores)


def _pv_reads(n, slot=None, base=None):
    """The two transpose reads of P*V fragment n (column block cb, k-half ks)
    into window slot `slot` (default n % PV_DEPTH) or into v[base:base+3]."""
    cb, ks = PV_FRAGS[n]
    r = base if base is not None else 256 - 4 * PV_DEPTH + 4 * ((n if slot is None else slot) % PV_DEPTH)
    off = 128 * (cb >> 1) + 16 * ks * ROWB
    # rows 16*ks + j (base t0/t1) and 16*ks + 8 + j (base t2/t3: rows 8 on
    # have their own swizzle), j = 4*(lane/32) + (lane%16)/4
    return [f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[t{cb & 1}] offset:{off}",
            f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[t{2 + (cb & 1)}] offset:{off}"]


SACC = 208           # the next tile's score accumulator (16 VGPRs)
MFMA_TO_VALU = 20    # instructions between the last score MFMA and a VALU read of its result
PREG = 196           # P of the tile being multiplied: v[196:199] (k-half 0), v[200:203] (k-half 1)
VALU_TAIL = 4        # score MFMAs at the end of the score phase with no softmax work after them


def _mask_lines():
    """Rows past the split end get -inf (only when %[valid] < 32, a tile that
    is the split's last): register r holds row c + 4*(lane/32) with
    c = 8*(r/4) + r%4, valid iff c < %[valid] - 4*(lane/32)."""
    s = [f"%[s{r}]" for r in range(16)]
    vl, ninf = f"v{VLIM}", f"v{TMP + 1}"
    out = ["s_cmp_ge_i32 %[valid], 32", "s_cbranch_scc1 .Lmla_full_%=",
           f"v_mbcnt_lo_u32_b32 {vl}, -1, 0", f"v_mbcnt_hi_u32_b32 {vl}, -1, {vl}",
           f"v_bfe_u32 {vl}, {vl}, 5, 1", f"v_lshlrev_b32_e32 {vl}, 2, {vl}", f"v_sub_u32_e32 {vl}, %[valid], {vl}",
           f"v_mov_b32_e32 {ninf}, 0xff800000"]  # -inf (a literal and vcc cannot share the bus)
    for r in range(16):
        c = 8 * (r // 4) + r % 4
        out.append(f"v_cmp_lt_i32_e32 vcc, {c}, {vl}")
        out.append(f"v_cndmask_b32_e32 {s[r]}, {ninf}, {s[r]}, vcc")
    out.append(".Lmla_full_%=:")
    return out


def _softmax_ops():
    """Softmax of a tile's scores in %[s0..s15] (score r holds row
    8*(r/4) + 4*(lane/32) + r%4 of the tile, head = lane%32): the
    bf16 pairs of 2^(s*scale - mref) into v[PREG:PREG+7] (the P fragments of
    the tile's P*V product) and %[l] += the sum of those rounded weights.  (No
    tile maximum: the overflow test runs once per pass on the sum, outside.)
    Ordered so that no instruction waits on a recent result: the exponent
    arguments (in place), the exponentials, the packing, then the sum."""
    s = [f"%[s{r}]" for r in range(16)]
    ops = [f"v_fma_f32 {s[r]}, {s[r]}, %[sc], -%[mref]" for r in range(16)]
    ops += [f"v_exp_f32_e32 {s[r]}, {s[r]}" for r in range(16)]
    ops += [f"v_cvt_pk_bf16_f32 v{PREG + j}, {s[2 * j]}, {s[2 * j + 1]}" for j in range(8)]
    ops += [f"v_dot2c_f32_bf16_e32 %[l], 0x3f803f80, v{PREG + j}" for j in range(8)]
    return ops


class _Valu:
    """Emits VALU ops with one instruction between a transcendental and a VALU
    read of its result (any other instruction in between counts)."""

    def __init__(self, out):
        self.out = out
        self.last_trans = None

    def other(self, line):
        self.out.append(line)
        self.last_trans = None

    def valu(self, op):
        if self.last_trans is not None and self.last_trans in op.split(",", 1)[-1]:
            self.out.append("s_nop 0")
        self.out.append(op)
        self.last_trans = op.split()[1].rstrip(",") if op.startswith("v_exp_f32") else None


DMA_PER_WAVE = 9     # 16-byte-per-lane LDS DMA instructions per wave and tile


def _dma_lines(n, steady=False):
    """LDS DMA n of a later tile (skipped when %[dma] = 0; always issued in the
    steady-state block): lane l copies 16 bytes from %[tbase] + %[d<n>] to LDS
    %[ldst] + 1024*n + 16*l."""
    copy = [f"s_add_u32 m0, %[ldst], {1024 * n}", "s_nop 0", f"global_load_lds_dwordx4 %[d{n}], %[tbase]"]
    if steady:
        return copy
    return ["s_cmp_eq_u32 %[dma], 0", f"s_cbranch_scc1 .Lmla_nodma{n}_%="] + copy + [f".Lmla_nodma{n}_%=:"]


def _score_phase(acc_out, valu_ops, steady, lds):
    """Scores of the next tile into v[acc_out:acc_out+15] (36 LDS-fed MFMAs,
    the first starting from zero), with the DMA of a later tile after MFMAs
    3, 7, ... and `valu_ops` spread over the MFMAs, the last VALU_TAIL MFMAs
    left free so that the P fragments are written well before the P*V MFMAs
    read them."""
    buf = [f"v[{256 - 4 * S_DEPTH + 4 * j}:{259 - 4 * S_DEPTH + 4 * j}]" for j in range(S_DEPTH)]
    out = ["s_waitcnt lgkmcnt(0)"]
    em = _Valu(out)
    rid = {}

    def read(j):
        rid[j] = lds.issue()
        em.other(f"ds_read_b128 {buf[j % S_DEPTH]}, %[b{j & 3}] offset:{128 * (j >> 2)}")

    for j in range(S_DEPTH):
        read(j)
    valu = list(valu_ops)
    slots = KS - VALU_TAIL
    dma_at = {3 + 4 * n: n for n in range(DMA_PER_WAVE)}
    for j in range(KS):
        em.other(lds.wait(rid[j]))
        src_c = "0" if j == 0 else f"v[{acc_out}:{acc_out + 15}]"
        em.other(f"v_mfma_f32_32x32x16_bf16 v[{acc_out}:{acc_out + 15}], {buf[j % S_DEPTH]}, %[q{j}], {src_c}")
        if j + S_DEPTH < KS:
            read(j + S_DEPTH)
        if j in dma_at:
            for line in _dma_lines(dma_at[j], steady):
                em.other(line)
        if j < slots and valu:
            take = -(-len(valu) // (slots - j))
            for _ in range(take):
                em.valu(valu.pop(0))
    assert not valu
    return out


def _pv_phase(lds, moves=()):
    """P*V MFMAs over the 32 fragments (16 column blocks x 2 k-halves) with P
    in v[PREG:PREG+7], cache^T fragments fed through a rolling window: the
    reads of fragment n + PV_DEPTH go into the slot of fragment n right after
    its MFMA has been issued.  `moves` (VALU copies of the new scores) go one
    per MFMA once MFMA_TO_VALU instructions have passed since the phase start."""
    nfr = len(PV_FRAGS)
    out, rid = [], {}
    moves = list(moves)

    def issue(n):
        for line in _pv_reads(n):
            rid[n] = lds.issue()
            out.append(line)

    for n in range(min(PV_DEPTH, nfr)):
        issue(n)
    for n in range(nfr):
        cb, ks = PV_FRAGS[n]
        r = 256 - 4 * PV_DEPTH + 4 * (n % PV_DEPTH)
        out.append(lds.wait(rid[n]))
        out.append(f"v_mfma_f32_32x32x16_bf16 %[o{cb}], v[{r}:{r + 3}], v[{PREG + 4 * ks}:{PREG + 4 * ks + 3}], %[o{cb}]")
        if n + PV_DEPTH < nfr:
            issue(n + PV_DEPTH)
        if moves and len(out) >= MFMA_TO_VALU:
            out.append(moves.pop(0))
    assert not moves
    return out


def fused_block(steady=False) -> str:
    """Iteration i of the tile loop: the scores of tile i+1 into v[SACC:SACC+15]
    with the softmax of tile i (scores in %[s0..s15], computed one iteration
    earlier) interleaved between the score MFMAs, then the P*V product of
    tile i with no other VALU work than copying the new scores into %[s*] for
    the next iteration; the LDS DMA of tile i+3 spread over the score MFMAs.
    The steady-state form (a full tile i, a next tile, a copy always issued)
    has no branches.  The general form masks the rows of tile i past the split
    end (%[valid] < 32), and at the split's last tile (%[nx] = 0) runs the
    softmax alone.  m0 (which the DMA uses) is saved and restored: the
    compiler reserves it."""
    out = ["s_mov_b32 %[m0save], m0", "s_waitcnt lgkmcnt(0)"]
    lds = _Lds()
    sm = _softmax_ops()
    if steady:
        out += _score_phase(SACC, sm, True, lds)
    else:
        out += _mask_lines()
        out += ["s_cmp_eq_u32 %[nx], 0", "s_cbranch_scc1 .Lmla_smonly_%="]
        out += _score_phase(SACC, sm, False, lds)
        out += ["s_branch .Lmla_pv_%=", ".Lmla_smonly_%=:"]
        em = _Valu(out)
        for op in sm:
            em.valu(op)
        out.append(".Lmla_pv_%=:")
        lds = _Lds()  # (one of the two paths ran)
    moves = [f"v_mov_b32_e32 %[s{r}], v{SACC + r}" for r in range(16)]
    out += _pv_phase(lds, moves)
    out.append("s_mov_b32 m0, %[m0save]")
    return "\\n\\t".join(out)


def main():
    w = sys.stdout.write
    w("// Generated by gen_decode_asm.py; do not edit by hand.\n")
    w("// Inner blocks of the bf16 decode kernel (32-row tile, 32 heads per wave).\n\n")
    w(f'#define MLA_ASM_SCORE_BLOCK0 "{score_block(0, 18, True, False)}"\n\n')
    w(f'#define MLA_ASM_SCORE_BLOCK1 "{score_block(18, 18, False, True)}"\n\n')
    w(f'#define MLA_ASM_FUSED_BLOCK "{fused_block()}"\n\n')
    w(f'#define MLA_ASM_FUSED_BLOCK_STEADY "{fused_block(True)}"\n')


if __name__ == "__main__":
    main()
