"""Generate decode_asm.inc: hand-scheduled inner blocks of the bf16 decode kernel.

    python gen_decode_asm.py > decode_asm.inc

Shape: 32-row tiles of 576-wide bf16 cache rows (1152 bytes), 32 heads per
wave, 512 latent columns.  Blocks:

  score block (18 k-steps): S^T[t][h] += cache[t][k..k+16) . q^T, A fragments
    streamed from LDS with ds_read_b128 through a 4-deep rolling window held in
    v[240:255]; B fragments (q) and the accumulator are asm operands.
  fused block (and its branch-free steady-state form): the scores of the
    next tile (36 k-steps into v[208:223]), then
    the P*V product of the current tile, O^T[c][h] += cache^T P^T (16 column
    blocks x 2 k-halves; cache^T fragments from pairs of ds_read_b64_tr_b16
    through the same kind of 4-deep rolling window; accumulators are AGPR
    operands), with the next tile's softmax (mask of rows past the split end,
    exponentials, bf16 packing, running sum) interleaved between
    the P*V MFMAs so that it runs while the matrix core is busy; the LDS DMA
    of a later tile is spread over the score MFMAs.

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
SACC = 208           # first VGPR of the next tile's score accumulator (16 regs)
TMP = 204            # mask temporaries (v205 holds -inf)
VLIM = 206           # per-lane row limit of the mask
MFMA_TO_VALU = 20    # wait states between the last score MFMA and a VALU read of it


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


PRE_BASE = 232       # first VGPR of the P*V fragments prefetched during the score phase


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


def _pv_lines(valu=None, first_valu_after=0, prelude=None, lds=None, pre=None):
    """P*V MFMAs over the 32 fragments (16 column blocks x 2 k-halves).
    Fragments in `pre` (n -> (first VGPR, id of its second read)) were read
    earlier into their own registers; the others are fed through a rolling
    window: the reads of the window's fragment k + PV_DEPTH go into the slot
    of fragment k right after its MFMA has been issued.  `valu` (list of
    instructions) is spread between the MFMAs, starting once
    `first_valu_after` wait states have passed since the block start;
    `prelude` (a list of lines) is emitted whole at that point."""
    valu = list(valu or [])
    pre = pre or {}
    lds = lds or _Lds()
    nfr = len(PV_FRAGS)
    win = [n for n in range(nfr) if n not in pre]
    pos = {n: k for k, n in enumerate(win)}
    rid = {}
    out = []
    waited = 0  # wait states since the block start

    def emit(line):
        nonlocal waited
        out.append(line)
        waited += int(line.split()[1]) + 1 if line.startswith("s_nop") else 1

    def issue(k):
        for line in _pv_reads(win[k], slot=k):
            rid[win[k]] = lds.issue()
            emit(line)

    last_trans = [None]

    def emit_valu(op):
        # one instruction between a transcendental and a VALU read of its result
        if last_trans[0] is not None and last_trans[0] in op.split(",", 1)[-1]:
            emit("s_nop 0")
        emit(op)
        last_trans[0] = op.split()[1].rstrip(",") if op.startswith("v_exp_f32") else None

    for k in range(min(PV_DEPTH, len(win))):
        issue(k)
    per_slot = None
    for n in range(nfr):
        cb, ks = PV_FRAGS[n]
        if n in pre:
            r, last_read = pre[n]
            emit(lds.wait(last_read))
        else:
            r = 256 - 4 * PV_DEPTH + 4 * (pos[n] % PV_DEPTH)
            emit(lds.wait(rid[n]))
        emit(f"v_mfma_f32_32x32x16_bf16 %[o{cb}], v[{r}:{r + 3}], %[p{ks}], %[o{cb}]")
        last_trans[0] = None
        if n not in pre and pos[n] + PV_DEPTH < len(win):
            issue(pos[n] + PV_DEPTH)
        if valu:
            if waited < first_valu_after:
                emit(f"s_nop {first_valu_after - waited - 1}")
            if prelude:
                for line in prelude:
                    emit(line)
                prelude = None
            if per_slot is None:
                per_slot = -(-len(valu) // (nfr - n))
            for _ in range(min(per_slot, len(valu))):
                emit_valu(valu.pop(0))
    while valu:  # (not reached with the shapes generated here)
        emit_valu(valu.pop(0))
    return out


def _mask_block(steady=False):
    """Rows past the split end get -inf (only when %[valid] < 32, a tile that
    is the split's last or past it): register r holds row c + 4*(lane/32) with
    c = 8*(r/4) + r%4, valid iff c < %[valid] - 4*(lane/32)."""
    if steady:  # every row of the next tile is valid
        return []
    s = [f"v{SACC + r}" for r in range(16)]
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
    """Softmax of the next tile on v[208:223] (accumulator register r holds
    row 8*(r/4) + 4*(lane/32) + r%4 of the tile, head = lane%32):
    outputs %[w0..w7] (bf16 pairs of 2^(s*scale - mref)) and %[l] += the sum
    of those rounded weights.  (No tile maximum: the overflow test runs once
    per pass on the sum, outside.)  Ordered so that no instruction waits on a
    recent result: the exponent arguments (in place), the exponentials, then
    the packing and the running sum."""
    s = [f"v{SACC + r}" for r in range(16)]
    ops = [f"v_fma_f32 {s[r]}, {s[r]}, %[sc], -%[mref]" for r in range(16)]
    ops += [f"v_exp_f32_e32 {s[r]}, {s[r]}" for r in range(16)]
    # round pairs to bf16 (the weights P*V uses), then add them to the sum
    ops += [f"v_cvt_pk_bf16_f32 %[w{j}], {s[2 * j]}, {s[2 * j + 1]}" for j in range(8)]
    ops += [f"v_dot2c_f32_bf16_e32 %[l], 0x3f803f80, %[w{j}]" for j in range(8)]
    return ops


DMA_PER_WAVE = 9     # 16-byte-per-lane LDS DMA instructions per wave and tile


def _dma_lines(n, steady=False):
    """LDS DMA n of a later tile (skipped when %[dma] = 0; always issued in the
    steady-state block): lane l copies 16 bytes from %[tbase] + %[d<n>] to LDS
    %[ldst] + 1024*n + 16*l."""
    copy = [f"s_add_u32 m0, %[ldst], {1024 * n}", "s_nop 0", f"global_load_lds_dwordx4 %[d{n}], %[tbase]"]
    if steady:
        return copy
    return ["s_cmp_eq_u32 %[dma], 0", f"s_cbranch_scc1 .Lmla_nodma{n}_%="] + copy + [f".Lmla_nodma{n}_%=:"]


PV_PRE = 2           # P*V fragments the steady-state block reads during the score phase


def fused_block(steady=False) -> str:
    # %[nx] = 0 at the last tile of a split: no next tile, the scores are
    # skipped and %[valid] = 0 masks every row, so the softmax part yields
    # weights 0, sum += 0 and max = -inf.  The DMA of a later tile is spread
    # over the score MFMAs so that its issue never queues up.  The steady-state
    # variant (a next tile that is full, a copy always issued) has no branches
    # and moves the transpose reads of the first PV_PRE P*V fragments into the
    # score phase: there the four waves' b128 reads leave LDS bandwidth spare,
    # while in the P*V phase the transpose reads alone would saturate it.
    # m0 (which the DMA uses) is saved and restored: the compiler reserves it
    out = ["s_mov_b32 %[m0save], m0", "s_waitcnt lgkmcnt(0)"]
    if not steady:
        out += ["s_cmp_eq_u32 %[nx], 0", "s_cbranch_scc1 .Lmla_pv_%="]
    lds = _Lds()
    extra, pre = {}, {}
    npre = PV_PRE if steady else 0
    for f in range(npre):
        at = 4 + f * (KS - 8) // max(1, npre)
        lines = _pv_reads(f, base=PRE_BASE + 4 * f)
        extra.setdefault(at, []).extend(lines)
        # the id of the fragment's second read: counted as the score emitter issues it
        pre[f] = PRE_BASE + 4 * f
    # the score emitter issues the extra reads through `lds`; record their ids
    issued_ids = []
    orig_issue = lds.issue

    def tracking_issue():
        r = orig_issue()
        issued_ids.append(r)
        return r

    lds.issue = tracking_issue
    score = _score_lines(0, KS, True, f"v[{SACC}:{SACC + 15}]", lambda j: f"%[q{j}]", extra, lds)
    lds.issue = orig_issue
    # ids of the extra reads, in order: the score reads are the ds_read_b128 ones
    kinds = [l for l in score if l.startswith("ds_read")]
    extra_ids = [rid for rid, l in zip(issued_ids, kinds) if l.startswith("ds_read_b64_tr")]
    pre = {f: (pre[f], extra_ids[2 * f + 1]) for f in range(npre)}
    mfma_at = [k for k, line in enumerate(score) if line.startswith("v_mfma")]
    after = {mfma_at[3 + 4 * n]: n for n in range(DMA_PER_WAVE)}
    for k, line in enumerate(score):
        out.append(line)
        if k in after:
            out += _dma_lines(after[k], steady)
    if not steady:
        out.append(".Lmla_pv_%=:")
        lds = _Lds()  # (the score phase may have been skipped)
    # P*V of the current tile; the first VALU read of the scores comes at
    # least MFMA_TO_VALU wait states after the last score MFMA
    out += _pv_lines(_softmax_ops(), MFMA_TO_VALU, _mask_block(steady), lds, pre)
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
